// Internal interface between the C-ABI layer (pld_api.cpp) and the HIP
// kernels (pld_kernels.hip). Not installed; callers use include/pld.h.
#ifndef PLD_KERNELS_H_
#define PLD_KERNELS_H_

#include <stdint.h>

#include <hip/hip_runtime_api.h>
#include <hip/hip_vector_types.h>

#include "pld.h"

namespace pld {

// Sticky device-side error bits (the context's error word).
enum : uint32_t {
    kErrLenCapacity = 1u,     // lengths[b] > max_len
    kErrLenNegative = 2u,     // lengths[b] < 0
    kErrBadRow = 4u,          // null or misaligned row pointer with L > 0
    kErrAppendCapacity = 8u,  // append would pass max_len
    kErrAppendNegative = 16u, // counts[b] < 0
    kErrBelowMinLen = 32u,    // strided batch: lengths[b] < the caller's min_len
    kErrFuseInput = 64u,      // pld_fuse: inconsistent per-request inputs
    kErrControlInput = 128u   // pld_control: an outcome or lookup input out of range
};

// Per-request reduction state of the fused gather: the packed key maximum
// and an accumulator whose low 24 bits count the workgroups that arrived
// and whose upper 40 bits sum the increases of `key` their atomicMax made
// (a key is below 2^39: length <= 64 << 32 | end < 2^31; a request has fewer
// than 2^24 tiles: max_len < 2^31 over tiles of at least 256). The
// increases telescope, so the sum is the maximum itself. One slot per 256
// bytes, so that atomics of different requests fall on different cache
// lines. Zero between calls.
struct alignas(256) ReqSlot {
    unsigned long long key;
    unsigned long long acc;
    unsigned int pad[60];
};

// Draft fusion and long-block scheduling (pld_fuse): parameters as in
// pld_fuse_params, then the per-request buffers.
struct FuseArgs {
    int32_t head, positions_long, replace_min, agree_min, agree_tokens, tail_min;
    int32_t entry_steps, sticky, near_full_slack;
    const int32_t *lookup;        // [batch * lookup_k]
    int32_t lookup_k;
    const int32_t *lookup_len;    // [batch]
    const int32_t *lookup_match;  // [batch]
    const int32_t *drafter;       // [batch * head]
    const int32_t *accepted;      // [batch]
    int32_t *state;               // [batch * 4]
    int32_t *out_block;           // [batch * positions_long]
    int32_t *out_positions;       // [batch]
    unsigned long long *out_src;  // [batch] or null
    unsigned int *err;
};

// The online cost/benefit controller (pld_control.hip, pld_control_step.h).
struct ControlArgs {
    double alpha, beta, margin, prior_accept, prior_time;
    int32_t mtp_tokens;
    int32_t edge[3];
    const int32_t *accepted;      // [batch]
    const double *round_time;     // [batch]
    const int32_t *lookup_len;    // [batch]
    const int32_t *lookup_match;  // [batch]
    double *state;                // [batch * 11]
    int32_t batch;
    int32_t *out_source;          // [batch]
    double *out_rates;            // [batch * 3] or null
    unsigned int *err;
};

struct DraftArgs {
    const int32_t *const *histories;  // row table (stride == 0)
    const int32_t *base;              // strided batch: row b at base + b * stride
    int64_t stride;                   // tokens between rows; 0 for a row table
    int32_t min_len;                  // strided batch: lower bound on every length
    const int32_t *lengths;
    int32_t batch;
    int32_t n_min, n_max, k_max;
    int32_t max_len;
    int32_t fused;
    int32_t *out_draft;
    int32_t *out_len;
    int32_t *out_match;
    int32_t *out_pos;              // may be null
    ReqSlot *slots;                // [max_batch], zero between calls
    unsigned int *err;             // sticky error word
    const int4 *zero16;            // 16 zero bytes (edge-chunk load target)
    FuseArgs fuse;                 // the fusion step, when do_fuse
    int32_t do_fuse;               // emit also fuses (pld_draft_fuse_batch)
    ControlArgs control;           // the controller step, when do_control
    int32_t do_control;            // emit also runs it (pld_draft_control_batch)
    // An append to the context's store in the same launch, when do_append
    // (strided batch over the store, lengths = the store's): row b gains
    // app_counts[b] tokens from app_tokens + b * app_stride before it is
    // drafted, as pld_append followed by the draft would leave it.
    const int32_t *app_tokens;
    int64_t app_stride;
    const int32_t *app_counts;
    int32_t *app_store;            // the store (base), written at the appended positions
    int32_t *app_lengths;          // the store's lengths, written back
    int32_t do_append;
};

struct AppendArgs {
    const int32_t *tokens;
    int64_t tokens_stride;
    const int32_t *counts;
    int32_t *store;
    int64_t pitch;
    int32_t *lengths;
    int32_t max_len;
    unsigned int *err;
};

// The context store's n-gram index (pld_index.hip): per request and per
// indexed length n in [n_lo, n_hi], `cap` 64-bit slots of
// (fingerprint << 32 | end + 1), 0 = empty.
struct IndexArgs {
    unsigned long long *table;  // [max_batch][n_hi - n_lo + 1][cap]
    int64_t cap;                // a power of two >= 2 * max_len
    int32_t n_lo, n_hi;
    int32_t *store;             // [max_batch * pitch]
    int64_t pitch;
    int32_t *lengths;           // [max_batch]
    int32_t max_len;
    uint32_t fp_mask;           // fingerprint bits kept (all 32 but in tests)
    unsigned int *err;
};

// The context store's successor-count cache (pld_ngram.hip): per request
// and context length n in [1, n_max], a gram table and a pair table of `cap`
// 32-byte slots each (count << 32 | end + 1, then the top successor or the
// 5th token, then 4 tokens) for the n-grams and the (n + 1)-grams.
struct NgramArgs {
    unsigned long long *grams;  // [max_batch][n_max][cap][4]
    unsigned long long *pairs;  // [max_batch][n_max][cap][4]
    int64_t cap;                // a power of two >= max(16, 2 * max_len)
    int32_t n_max;              // context lengths kept: 1..n_max (<= 4)
    int32_t *store;             // [max_batch * pitch]
    int64_t pitch;
    int32_t *lengths;           // [max_batch]
    int32_t max_len;
    unsigned int *err;
};

// One drafting call from the cache: thresholds per context length n at
// index n - 1.
struct NgramDraftArgs {
    int32_t n_min, n_max;
    int32_t min_count[4];
    int32_t min_percent[4];
    int32_t batch, k_max;
    int32_t *out_draft;   // [batch, k_max]
    int32_t *out_len;     // [batch]
    int32_t *out_levels;  // [batch, k_max] or null
};


// The reduction state of pld_draft_batch_noalloc: the same per-request slots,
// error word and zero block a context owns, for at most kStaticMaxBatch
// requests, in a static device array of the library (one per GPU).
constexpr int32_t kStaticMaxBatch = 4096;
struct alignas(256) StaticScratch {
    ReqSlot slots[kStaticMaxBatch];
    unsigned int err;
    unsigned int pad[3];
    int4 zero16;
};

// The calling device's StaticScratch (its address looked up once per device
// and the array cleared on `s` the first time), or an error.
hipError_t static_scratch(StaticScratch **out, hipStream_t s);

// Workgroups the scan launches for a batch (tiles per request x batch).
int64_t scan_grid(int32_t max_len, int32_t batch, int tile_tokens);

hipError_t launch_draft(const DraftArgs &a, int tile_tokens, hipStream_t s);
hipError_t launch_append(const AppendArgs &a, int32_t batch, hipStream_t s);
hipError_t launch_fill(int32_t *p, int64_t n, int32_t value, hipStream_t s);
hipError_t launch_fuse(const FuseArgs &a, int32_t batch, hipStream_t s);
hipError_t launch_index_insert(const IndexArgs &a, const int32_t *tokens, int64_t tokens_stride,
                               const int32_t *counts, int32_t batch, int32_t chunks,
                               hipStream_t s);
hipError_t launch_append_indexed(const IndexArgs &a, const int32_t *tokens,
                                 int64_t tokens_stride, const int32_t *counts, int32_t batch,
                                 hipStream_t s);
hipError_t launch_append_draft_indexed(const IndexArgs &a, const int32_t *tokens,
                                       int64_t tokens_stride, const int32_t *counts,
                                       int32_t batch, int32_t n_min, int32_t n_max,
                                       int32_t k_max, int32_t *out_draft, int32_t *out_len,
                                       int32_t *out_match, int32_t *out_pos, hipStream_t s);
hipError_t launch_index_draft(const IndexArgs &a, int32_t batch, int32_t n_min, int32_t n_max,
                              int32_t k_max, int32_t *out_draft, int32_t *out_len,
                              int32_t *out_match, int32_t *out_pos, hipStream_t s);
hipError_t launch_index_clear(const IndexArgs &a, int32_t batch, hipStream_t s);
hipError_t launch_control(const ControlArgs &a, hipStream_t s);
hipError_t launch_ngram_insert(const NgramArgs &a, const int32_t *tokens, int64_t tokens_stride,
                               const int32_t *counts, int32_t batch, int32_t chunks,
                               hipStream_t s);
hipError_t launch_append_ngram(const NgramArgs &a, const int32_t *tokens, int64_t tokens_stride,
                               const int32_t *counts, int32_t batch, hipStream_t s);
hipError_t launch_ngram_draft(const NgramArgs &a, const NgramDraftArgs &d, hipStream_t s);
hipError_t launch_append_draft_ngram(const NgramArgs &a, const int32_t *tokens,
                                     int64_t tokens_stride, const int32_t *counts,
                                     const NgramDraftArgs &d, hipStream_t s);
hipError_t launch_ngram_clear(const NgramArgs &a, int32_t batch, hipStream_t s);

}  // namespace pld

#endif  // PLD_KERNELS_H_
