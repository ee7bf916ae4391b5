// C-ABI entry points of libpld (declared in include/pld.h): argument checks,
// the context (reduction slots, error word, optional history store) and the
// launch of the HIP kernels in pld_kernels.hip. No compute happens here.

#include <stdarg.h>
#include <stdint.h>
#include <stdio.h>
#include <string.h>

#include <new>

#include <hip/hip_runtime_api.h>

#include "pld.h"
#include "pld_kernels.h"

struct pld_ctx {
    int device;
    int32_t max_batch;
    int32_t max_len;
    int32_t tile_tokens;        // scan tile size; 0: chosen per call (pick_tile)
    int32_t fused;
    pld::ReqSlot *slots;        // [max_batch] reduction state
    unsigned int *err;          // one word
    int4 *zero16;               // 16 zero bytes
    int32_t *store;             // [max_batch * pitch] or null
    int64_t pitch;              // tokens per store row
    int32_t *store_len;         // [max_batch] or null
    const int32_t **store_rows; // [max_batch] device row pointers or null
    unsigned long long *index;  // n-gram index over the store, or null
    int64_t index_cap;          // slots per (request, length) table
    int32_t index_lo, index_hi; // indexed lengths
    int32_t index_chunks;       // workgroups per request for an append's inserts
    uint32_t index_fp_mask;     // fingerprint bits kept
    unsigned long long *ngram_grams;  // successor-count cache: gram slots, or null
    unsigned long long *ngram_pairs;  // and pair slots
    int64_t ngram_cap;                // slots per (request, length) table
    int32_t ngram_n_max;              // context lengths 1..ngram_n_max
    int32_t ngram_chunks;             // workgroups per request for a large append
};

namespace {

thread_local char g_last_error[256] = "";

pld_status fail(pld_status s, const char *fmt, ...) __attribute__((format(printf, 2, 3)));

pld_status fail(pld_status s, const char *fmt, ...)
{
    va_list ap;
    va_start(ap, fmt);
    vsnprintf(g_last_error, sizeof(g_last_error), fmt, ap);
    va_end(ap);
    return s;
}

pld_status hip_fail(hipError_t e, const char *what)
{
    return fail(PLD_EHIP, "%s: %s", what, hipGetErrorString(e));
}

void release(pld_ctx *c)
{
    if (!c)
        return;
    if (c->slots) (void)hipFree(c->slots);
    if (c->err) (void)hipFree(c->err);
    if (c->zero16) (void)hipFree(c->zero16);
    if (c->store) (void)hipFree(c->store);
    if (c->store_len) (void)hipFree(c->store_len);
    if (c->store_rows) (void)hipFree(c->store_rows);
    if (c->index) (void)hipFree(c->index);
    if (c->ngram_grams) (void)hipFree(c->ngram_grams);
    if (c->ngram_pairs) (void)hipFree(c->ngram_pairs);
    delete c;
}

bool valid_tile(int32_t t)
{
    return t == 256 || t == 1024 || t == 2048 || t == 4096 || t == 8192 || t == 16384;
}
// The scan's tile size for a call: the caller's choice, or automatically
// the largest of 4,096, 2,048 and 1,024 candidate positions that still gives
// the grid at least 1,024 workgroups (4 per compute unit), so that small
// batches spread over the whole chip and large ones keep their workgroups
// few. A request that fits one 4,096-token tile is not split: its single
// workgroup emits without the cross-workgroup merge.
static int32_t auto_tile(int32_t max_len, int32_t batch)
{
    if (pld::scan_grid(max_len, 1, 4096) <= 1)
        return 4096;
    for (int32_t t = 4096; t > 1024; t /= 2)
        if (pld::scan_grid(max_len, batch, t) >= 1024)
            return t;
    return 1024;
}

static int32_t pick_tile(const pld_ctx *ctx, int32_t batch)
{
    return ctx->tile_tokens != 0 ? ctx->tile_tokens : auto_tile(ctx->max_len, batch);
}


pld_status check_draft_args(pld_ctx *ctx, const int32_t *const *histories,
                            const int32_t *lengths, int32_t batch, int32_t n_min,
                            int32_t n_max, int32_t k_max, int32_t *out_draft,
                            int32_t *out_len, int32_t *out_match)
{
    if (!ctx)
        return fail(PLD_EINVAL, "ctx is null");
    if (n_min < 1 || n_max < n_min || n_max > PLD_N_MAX_LIMIT)
        return fail(PLD_EINVAL, "need 1 <= n_min <= n_max <= %d (got n_min=%d n_max=%d)",
                    PLD_N_MAX_LIMIT, n_min, n_max);
    if (k_max < 1)
        return fail(PLD_EINVAL, "k_max must be >= 1 (got %d)", k_max);
    if (batch < 0 || batch > ctx->max_batch)
        return fail(PLD_EINVAL, "batch %d outside [0, max_batch=%d]", batch, ctx->max_batch);
    if (batch > 0 && (!histories || !lengths || !out_draft || !out_len || !out_match))
        return fail(PLD_EINVAL, "null buffer pointer");
    if (batch > 0 && (((uintptr_t)lengths | (uintptr_t)out_draft | (uintptr_t)out_len |
                       (uintptr_t)out_match) & 3u))
        return fail(PLD_EINVAL, "lengths and outputs must be 4-byte aligned");
    if ((int64_t)batch * k_max > INT64_MAX / 4)
        return fail(PLD_EINVAL, "batch * k_max too large");
    if (pld::scan_grid(ctx->max_len, batch, pick_tile(ctx, batch)) > 0x7fffffffLL)
        return fail(PLD_EINVAL, "grid too large: batch %d x tiles for max_len %d", batch,
                    ctx->max_len);
    return PLD_OK;
}

// An append to the context's store made inside the draft's own launch.
struct AppendIn {
    const int32_t *tokens;
    int64_t tokens_stride;
    const int32_t *counts;
};

pld_status draft(pld_ctx *ctx, const int32_t *const *histories, const int32_t *base,
                 int64_t stride, int32_t min_len, const int32_t *lengths,
                 int32_t batch, int32_t n_min, int32_t n_max, int32_t k_max,
                 int32_t *out_draft, int32_t *out_len, int32_t *out_match,
                 int32_t *out_pos, hipStream_t stream, const pld::FuseArgs *fuse = nullptr,
                 const pld::ControlArgs *control = nullptr, const AppendIn *append = nullptr)
{
    // a strided batch stands in for the row table in the common checks
    const int32_t *const *rows_or_base =
        stride ? (const int32_t *const *)(const void *)base : histories;
    pld_status s = check_draft_args(ctx, rows_or_base, lengths, batch, n_min, n_max, k_max,
                                    out_draft, out_len, out_match);
    if (s != PLD_OK)
        return s;
    if (stride) {
        if ((uintptr_t)base & 15u)
            return fail(PLD_EINVAL, "strided batch: base must be 16-byte aligned");
        if (stride < 4 || (stride & 3))
            return fail(PLD_EINVAL, "strided batch: stride must be a positive multiple of 4 "
                        "tokens (got %lld)", (long long)stride);
        if (min_len < 0 || min_len > ctx->max_len || min_len > stride)
            return fail(PLD_EINVAL, "strided batch: min_len %d outside [0, min(max_len, stride)]",
                        min_len);
    }
    if (batch == 0)
        return PLD_OK;
    pld::DraftArgs a;
    a.histories = histories;
    a.base = base;
    a.stride = stride;
    a.min_len = min_len;
    a.lengths = lengths;
    a.batch = batch;
    a.n_min = n_min;
    a.n_max = n_max;
    a.k_max = k_max;
    a.max_len = ctx->max_len;
    a.fused = ctx->fused;
    a.out_draft = out_draft;
    a.out_len = out_len;
    a.out_match = out_match;
    a.out_pos = out_pos;
    a.slots = ctx->slots;
    a.err = ctx->err;
    a.zero16 = ctx->zero16;
    a.do_fuse = fuse != nullptr;
    if (fuse)
        a.fuse = *fuse;
    else
        memset(&a.fuse, 0, sizeof(a.fuse));
    a.do_control = control != nullptr;
    if (control)
        a.control = *control;
    else
        memset(&a.control, 0, sizeof(a.control));
    a.do_append = append != nullptr;
    a.app_tokens = append ? append->tokens : nullptr;
    a.app_stride = append ? append->tokens_stride : 0;
    a.app_counts = append ? append->counts : nullptr;
    a.app_store = append ? ctx->store : nullptr;
    a.app_lengths = append ? ctx->store_len : nullptr;
    hipError_t e = pld::launch_draft(a, pick_tile(ctx, a.batch), stream);
    if (e != hipSuccess)
        return hip_fail(e, "draft kernel launch");
    return PLD_OK;
}

// An indexed append whose rows are at most this many tokens apart takes the
// one-kernel path (the stride bounds the counts of non-overlapping rows).
constexpr int64_t kSmallAppend = 1024;

pld::IndexArgs index_args(pld_ctx *ctx)
{
    pld::IndexArgs a;
    a.table = ctx->index;
    a.cap = ctx->index_cap;
    a.n_lo = ctx->index_lo;
    a.n_hi = ctx->index_hi;
    a.store = ctx->store;
    a.pitch = ctx->pitch;
    a.lengths = ctx->store_len;
    a.max_len = ctx->max_len;
    a.fp_mask = ctx->index_fp_mask;
    a.err = ctx->err;
    return a;
}

pld::NgramArgs ngram_args(pld_ctx *ctx)
{
    pld::NgramArgs a;
    a.grams = ctx->ngram_grams;
    a.pairs = ctx->ngram_pairs;
    a.cap = ctx->ngram_cap;
    a.n_max = ctx->ngram_n_max;
    a.store = ctx->store;
    a.pitch = ctx->pitch;
    a.lengths = ctx->store_len;
    a.max_len = ctx->max_len;
    a.err = ctx->err;
    return a;
}

// Checks a fusion step's arguments and fills `a`; PLD_OK or the failure.
pld_status fuse_args(pld_ctx *ctx, const pld_fuse_params *params, const int32_t *lookup,
                     int32_t lookup_k, const int32_t *lookup_len, const int32_t *lookup_match,
                     const int32_t *drafter, const int32_t *accepted, int32_t *state,
                     int32_t batch, int32_t *out_block, int32_t *out_positions,
                     uint64_t *out_src, pld::FuseArgs &a)
{
    if (!ctx)
        return fail(PLD_EINVAL, "ctx is null");
    if (!params)
        return fail(PLD_EINVAL, "params is null");
    const pld_fuse_params &p = *params;
    if (p.head < 1 || p.positions_long < p.head || p.positions_long > PLD_FUSE_MAX_POSITIONS)
        return fail(PLD_EINVAL, "need 1 <= head <= positions_long <= %d (got %d, %d)",
                    PLD_FUSE_MAX_POSITIONS, p.head, p.positions_long);
    if (p.agree_tokens < 1 || p.agree_tokens > p.head)
        return fail(PLD_EINVAL, "need 1 <= agree_tokens <= head (got %d)", p.agree_tokens);
    if (p.replace_min < 1 || p.agree_min < 1 || p.tail_min < 1)
        return fail(PLD_EINVAL, "match thresholds must be >= 1");
    if (p.entry_steps < 0 || p.sticky < 0 || p.near_full_slack < 0)
        return fail(PLD_EINVAL, "entry_steps, sticky and near_full_slack must be >= 0");
    if (lookup_k < 1)
        return fail(PLD_EINVAL, "lookup_k must be >= 1 (got %d)", lookup_k);
    if (batch < 0 || batch > ctx->max_batch)
        return fail(PLD_EINVAL, "batch %d outside [0, max_batch=%d]", batch, ctx->max_batch);
    if (batch > 0 && (!lookup || !lookup_len || !lookup_match || !drafter || !accepted ||
                      !state || !out_block || !out_positions))
        return fail(PLD_EINVAL, "null buffer pointer");
    if (((uintptr_t)lookup | (uintptr_t)lookup_len | (uintptr_t)lookup_match |
         (uintptr_t)drafter | (uintptr_t)accepted | (uintptr_t)state | (uintptr_t)out_block |
         (uintptr_t)out_positions) & 3u)
        return fail(PLD_EINVAL, "int32 buffers must be 4-byte aligned");
    if ((uintptr_t)out_src & 7u)
        return fail(PLD_EINVAL, "out_src must be 8-byte aligned");
    a.head = p.head;
    a.positions_long = p.positions_long;
    a.replace_min = p.replace_min;
    a.agree_min = p.agree_min;
    a.agree_tokens = p.agree_tokens;
    a.tail_min = p.tail_min;
    a.entry_steps = p.entry_steps;
    a.sticky = p.sticky;
    a.near_full_slack = p.near_full_slack;
    a.lookup = lookup;
    a.lookup_k = lookup_k;
    a.lookup_len = lookup_len;
    a.lookup_match = lookup_match;
    a.drafter = drafter;
    a.accepted = accepted;
    a.state = state;
    a.out_block = out_block;
    a.out_positions = out_positions;
    a.out_src = (unsigned long long *)out_src;
    a.err = ctx->err;
    return PLD_OK;
}

// Creates a context; index_lo > 0 adds an n-gram index over the store.
pld_status create(pld_ctx **out, int32_t max_batch, int64_t max_len64, int32_t own_store,
                  int32_t index_lo, int32_t index_hi, hipStream_t stream,
                  int32_t ngram_n_max = 0)
{
    if (!out)
        return fail(PLD_EINVAL, "out is null");
    if (max_batch < 1)
        return fail(PLD_EINVAL, "max_batch must be >= 1 (got %d)", max_batch);
    // positions are the low 32 bits of the scan's packed key
    if (max_len64 < 1 || max_len64 > 0x7fffffffLL)
        return fail(PLD_EINVAL, "max_len must be in [1, 2^31-1] (got %lld)",
                    (long long)max_len64);
    const int32_t max_len = (int32_t)max_len64;
    pld_ctx *c = new (std::nothrow) pld_ctx();
    if (!c)
        return fail(PLD_ENOMEM, "host allocation failed");
    memset(c, 0, sizeof(*c));
    c->max_batch = max_batch;
    c->max_len = max_len;
    c->tile_tokens = 0;  // automatic (pick_tile)
    c->fused = 1;
    hipError_t e = hipGetDevice(&c->device);
    if (e != hipSuccess) {
        release(c);
        return hip_fail(e, "hipGetDevice");
    }
    const size_t nb = (size_t)max_batch;
    if (hipMalloc((void **)&c->slots, nb * sizeof(pld::ReqSlot)) != hipSuccess ||
        hipMalloc((void **)&c->err, sizeof(unsigned int)) != hipSuccess ||
        hipMalloc((void **)&c->zero16, sizeof(int4)) != hipSuccess) {
        (void)hipGetLastError();
        release(c);
        return fail(PLD_ENOMEM, "device allocation of reduction slots failed");
    }
    if (own_store) {
        c->pitch = ((int64_t)max_len + 63) / 64 * 64;
        const double bytes = (double)nb * (double)c->pitch * 4.0;
        if (bytes > 9.0e18 ||
            hipMalloc((void **)&c->store, nb * (size_t)c->pitch * sizeof(int32_t)) != hipSuccess ||
            hipMalloc((void **)&c->store_len, nb * sizeof(int32_t)) != hipSuccess ||
            hipMalloc((void **)&c->store_rows, nb * sizeof(int32_t *)) != hipSuccess) {
            (void)hipGetLastError();
            release(c);
            return fail(PLD_ENOMEM, "device allocation of the %d x %d token store failed",
                        max_batch, max_len);
        }
    }
    if (index_lo > 0) {
        int64_t cap = 1;
        while (cap < 2 * (int64_t)max_len)
            cap <<= 1;
        const int64_t lens = (int64_t)index_hi - index_lo + 1;
        const double bytes = (double)nb * (double)lens * (double)cap * 8.0;
        if (bytes > 9.0e18 ||
            hipMalloc((void **)&c->index, (size_t)nb * (size_t)lens * (size_t)cap * 8) !=
                hipSuccess) {
            (void)hipGetLastError();
            release(c);
            return fail(PLD_ENOMEM, "device allocation of the n-gram index (%.0f MB) failed",
                        bytes / 1e6);
        }
        c->index_cap = cap;
        c->index_fp_mask = 0xffffffffu;
        c->index_lo = index_lo;
        c->index_hi = index_hi;
        // an append's inserts spread over up to 16 workgroups per request
        const int64_t chunks = max_len / 8192;
        c->index_chunks = (int32_t)(chunks < 1 ? 1 : (chunks > 16 ? 16 : chunks));
    }
    if (ngram_n_max > 0) {
        int64_t cap = 16;
        while (cap < 2 * (int64_t)max_len)
            cap <<= 1;
        const double slots = (double)nb * (double)ngram_n_max * (double)cap;
        const size_t n = (size_t)nb * (size_t)ngram_n_max * (size_t)cap;
        if (slots * 64.0 > 9.0e18 ||
            hipMalloc((void **)&c->ngram_grams, n * 32) != hipSuccess ||
            hipMalloc((void **)&c->ngram_pairs, n * 32) != hipSuccess) {
            (void)hipGetLastError();
            release(c);
            return fail(PLD_ENOMEM, "device allocation of the successor-count cache (%.0f MB) "
                        "failed", slots * 64.0 / 1e6);
        }
        c->ngram_cap = cap;
        c->ngram_n_max = ngram_n_max;
        const int64_t chunks = max_len / 8192;
        c->ngram_chunks = (int32_t)(chunks < 1 ? 1 : (chunks > 16 ? 16 : chunks));
    }
    // every clear is enqueued on the caller's stream, then waited for
    const int32_t **rows = nullptr;
    e = hipMemsetAsync(c->slots, 0, nb * sizeof(pld::ReqSlot), stream);
    if (e == hipSuccess && c->index)
        e = pld::launch_index_clear(index_args(c), max_batch, stream);
    if (e == hipSuccess && c->ngram_grams)
        e = pld::launch_ngram_clear(ngram_args(c), max_batch, stream);
    if (e == hipSuccess) e = hipMemsetAsync(c->err, 0, sizeof(unsigned int), stream);
    if (e == hipSuccess) e = hipMemsetAsync(c->zero16, 0, sizeof(int4), stream);
    if (e == hipSuccess && own_store) {
        e = hipMemsetAsync(c->store_len, 0, nb * sizeof(int32_t), stream);
        rows = new (std::nothrow) const int32_t *[nb];
        if (!rows) {
            (void)hipStreamSynchronize(stream);
            release(c);
            return fail(PLD_ENOMEM, "host allocation failed");
        }
        for (size_t b = 0; b < nb; ++b)
            rows[b] = c->store + (int64_t)b * c->pitch;
        if (e == hipSuccess)
            e = hipMemcpyAsync(c->store_rows, rows, nb * sizeof(int32_t *),
                               hipMemcpyHostToDevice, stream);
    }
    // the host row table must outlive the copy: wait before freeing it
    const hipError_t w = hipStreamSynchronize(stream);
    if (e == hipSuccess)
        e = w;
    delete[] rows;
    if (e != hipSuccess) {
        release(c);
        return hip_fail(e, "context initialisation");
    }
    *out = c;
    return PLD_OK;
}

// Checks a controller step's arguments and fills `a`; PLD_OK or the
// failure. With `own_lookup` the lookup draft comes from the same call (no
// lookup_len / lookup_match buffers).
pld_status control_args(pld_ctx *ctx, const pld_control_params *params, const int32_t *accepted,
                        const double *round_time, const int32_t *lookup_len,
                        const int32_t *lookup_match, double *state, int32_t batch,
                        int32_t *out_source, double *out_rates, bool own_lookup,
                        pld::ControlArgs &a)
{
    if (!ctx)
        return fail(PLD_EINVAL, "ctx is null");
    if (!params)
        return fail(PLD_EINVAL, "params is null");
    const pld_control_params &p = *params;
    if (!(p.alpha >= 0.0 && p.alpha <= 1.0 && p.beta >= 0.0 && p.beta <= 1.0))
        return fail(PLD_EINVAL, "alpha and beta must be in [0, 1]");
    if (!(p.margin > 0.0) || !(p.prior_accept >= 0.0 && p.prior_accept <= 1.0) ||
        !(p.prior_time > 0.0))
        return fail(PLD_EINVAL, "need margin > 0, prior_accept in [0, 1], prior_time > 0");
    if (p.mtp_tokens < 0 || p.bucket_edge[0] > p.bucket_edge[1] ||
        p.bucket_edge[1] > p.bucket_edge[2])
        return fail(PLD_EINVAL, "need mtp_tokens >= 0 and nondecreasing bucket edges");
    if (batch < 0 || batch > ctx->max_batch)
        return fail(PLD_EINVAL, "batch %d outside [0, max_batch=%d]", batch, ctx->max_batch);
    if (batch > 0 && (!accepted || !round_time || !state || !out_source ||
                      (!own_lookup && (!lookup_len || !lookup_match))))
        return fail(PLD_EINVAL, "null buffer pointer");
    if ((((uintptr_t)accepted | (uintptr_t)lookup_len | (uintptr_t)lookup_match |
          (uintptr_t)out_source) & 3u) ||
        (((uintptr_t)round_time | (uintptr_t)state | (uintptr_t)out_rates) & 7u))
        return fail(PLD_EINVAL, "misaligned buffer (int32: 4 bytes, double: 8 bytes)");
    a.alpha = p.alpha;
    a.beta = p.beta;
    a.margin = p.margin;
    a.prior_accept = p.prior_accept;
    a.prior_time = p.prior_time;
    a.mtp_tokens = p.mtp_tokens;
    for (int i = 0; i < 3; ++i)
        a.edge[i] = p.bucket_edge[i];
    a.accepted = accepted;
    a.round_time = round_time;
    a.lookup_len = lookup_len;
    a.lookup_match = lookup_match;
    a.state = state;
    a.batch = batch;
    a.out_source = out_source;
    a.out_rates = out_rates;
    a.err = ctx->err;
    return PLD_OK;
}


}  // namespace

extern "C" {

pld_status pld_create(pld_ctx **out, int32_t max_batch, int64_t max_len, int32_t own_store,
                      hipStream_t stream)
{
    return create(out, max_batch, max_len, own_store, 0, 0, stream);
}

pld_status pld_create_indexed(pld_ctx **out, int32_t max_batch, int64_t max_len, int32_t n_min,
                              int32_t n_max, hipStream_t stream)
{
    if (n_min < 1 || n_max < n_min || n_max > PLD_N_MAX_LIMIT)
        return fail(PLD_EINVAL, "need 1 <= n_min <= n_max <= %d (got n_min=%d n_max=%d)",
                    PLD_N_MAX_LIMIT, n_min, n_max);
    return create(out, max_batch, max_len, 1, n_min, n_max, stream);
}

pld_status pld_create_ngram(pld_ctx **out, int32_t max_batch, int64_t max_len, int32_t n_max,
                            hipStream_t stream)
{
    if (n_max < 1 || n_max > PLD_NGRAM_MAX_N)
        return fail(PLD_EINVAL, "need 1 <= n_max <= %d (got %d)", PLD_NGRAM_MAX_N, n_max);
    return create(out, max_batch, max_len, 1, 0, 0, stream, n_max);
}

pld_status pld_destroy(pld_ctx *ctx)
{
    if (!ctx)
        return PLD_OK;
    hipError_t e = hipDeviceSynchronize();
    release(ctx);
    if (e != hipSuccess)
        return hip_fail(e, "hipDeviceSynchronize before destroy");
    return PLD_OK;
}

pld_status pld_configure(pld_ctx *ctx, int32_t tile_tokens, int32_t fused_gather)
{
    if (!ctx)
        return fail(PLD_EINVAL, "ctx is null");
    if (tile_tokens != 0 && tile_tokens != -1 && !valid_tile(tile_tokens))
        return fail(PLD_EINVAL,
                    "tile_tokens %d not one of 256, 1024, 2048, 4096, 8192, 16384, 0 or -1",
                    tile_tokens);
    if (fused_gather < -1 || fused_gather > 1)
        return fail(PLD_EINVAL, "fused_gather must be -1, 0 or 1 (got %d)", fused_gather);
    if (tile_tokens != 0)
        ctx->tile_tokens = tile_tokens == -1 ? 0 : tile_tokens;
    if (fused_gather >= 0)
        ctx->fused = fused_gather;
    return PLD_OK;
}

pld_status pld_append(pld_ctx *ctx, const int32_t *tokens, int64_t tokens_stride,
                      const int32_t *counts, int32_t batch, hipStream_t stream)
{
    if (!ctx)
        return fail(PLD_EINVAL, "ctx is null");
    if (!ctx->store)
        return fail(PLD_EINVAL, "context was created without a store");
    if (batch < 0 || batch > ctx->max_batch)
        return fail(PLD_EINVAL, "batch %d outside [0, max_batch=%d]", batch, ctx->max_batch);
    if (tokens_stride < 0)
        return fail(PLD_EINVAL, "tokens_stride must be >= 0");
    if (batch == 0)
        return PLD_OK;
    if (!tokens || !counts)
        return fail(PLD_EINVAL, "null buffer pointer");
    pld::AppendArgs a;
    a.tokens = tokens;
    a.tokens_stride = tokens_stride;
    a.counts = counts;
    a.store = ctx->store;
    a.pitch = ctx->pitch;
    a.lengths = ctx->store_len;
    a.max_len = ctx->max_len;
    a.err = ctx->err;
    hipError_t e = hipSuccess;
    if (ctx->ngram_grams) {
        if (tokens_stride > 0 && tokens_stride <= kSmallAppend) {
            // counts and copy in one workgroup per request
            e = pld::launch_append_ngram(ngram_args(ctx), tokens, tokens_stride, counts, batch,
                                         stream);
        } else {
            // before the copy: it reads the old length and the store
            e = pld::launch_ngram_insert(ngram_args(ctx), tokens, tokens_stride, counts, batch,
                                         ctx->ngram_chunks, stream);
            if (e == hipSuccess)
                e = pld::launch_append(a, batch, stream);
        }
    } else if (ctx->index && tokens_stride > 0 && tokens_stride <= kSmallAppend) {
        // rows of at most kSmallAppend tokens (a decode loop's appends):
        // inserts and copy in one workgroup per request
        e = pld::launch_append_indexed(index_args(ctx), tokens, tokens_stride, counts, batch,
                                       stream);
    } else {
        if (ctx->index)  // before the copy: it reads the old length and the store
            e = pld::launch_index_insert(index_args(ctx), tokens, tokens_stride, counts, batch,
                                         ctx->index_chunks, stream);
        if (e == hipSuccess)
            e = pld::launch_append(a, batch, stream);
    }
    if (e != hipSuccess)
        return hip_fail(e, "append kernel launch");
    return PLD_OK;
}

pld_status pld_scan_tile(pld_ctx *ctx, int32_t batch, int32_t *tile_tokens)
{
    if (!ctx || !tile_tokens)
        return fail(PLD_EINVAL, "ctx or tile_tokens is null");
    if (batch < 1 || batch > ctx->max_batch)
        return fail(PLD_EINVAL, "batch %d outside [1, max_batch=%d]", batch, ctx->max_batch);
    *tile_tokens = pick_tile(ctx, batch);
    return PLD_OK;
}

pld_status pld_histories(pld_ctx *ctx, const int32_t *const **histories,
                           const int32_t **lengths)
{
    if (!ctx || !histories || !lengths)
        return fail(PLD_EINVAL, "null argument");
    if (!ctx->store)
        return fail(PLD_EINVAL, "context was created without a store");
    *histories = ctx->store_rows;
    *lengths = ctx->store_len;
    return PLD_OK;
}

pld_status pld_store_reset(pld_ctx *ctx, hipStream_t stream)
{
    if (!ctx)
        return fail(PLD_EINVAL, "ctx is null");
    if (!ctx->store)
        return fail(PLD_EINVAL, "context was created without a store");
    hipError_t e = pld::launch_fill(ctx->store_len, ctx->max_batch, 0, stream);
    if (e == hipSuccess && ctx->index)
        e = pld::launch_index_clear(index_args(ctx), ctx->max_batch, stream);
    if (e == hipSuccess && ctx->ngram_grams)
        e = pld::launch_ngram_clear(ngram_args(ctx), ctx->max_batch, stream);
    if (e != hipSuccess)
        return hip_fail(e, "store reset launch");
    return PLD_OK;
}

pld_status pld_append_draft_store(pld_ctx *ctx, const int32_t *tokens, int64_t tokens_stride,
                                  const int32_t *counts, int32_t batch, int32_t n_min,
                                  int32_t n_max, int32_t k_max, int32_t *out_draft,
                                  int32_t *out_len, int32_t *out_match, int32_t *out_pos,
                                  hipStream_t stream)
{
    if (!ctx)
        return fail(PLD_EINVAL, "ctx is null");
    if (!ctx->store)
        return fail(PLD_EINVAL, "context was created without a store");
    // every draft argument is checked before the append is enqueued
    const int32_t lo = ctx->index ? ctx->index_lo : 1;
    const int32_t hi = ctx->index ? ctx->index_hi : PLD_N_MAX_LIMIT;
    if (n_min < lo || n_max < n_min || n_max > hi)
        return fail(PLD_EINVAL, "need %d <= n_min <= n_max <= %d (got n_min=%d n_max=%d)", lo,
                    hi, n_min, n_max);
    if (k_max < 1)
        return fail(PLD_EINVAL, "k_max must be >= 1 (got %d)", k_max);
    if (batch < 0 || batch > ctx->max_batch)
        return fail(PLD_EINVAL, "batch %d outside [0, max_batch=%d]", batch, ctx->max_batch);
    if (batch > 0 && (!out_draft || !out_len || !out_match))
        return fail(PLD_EINVAL, "null buffer pointer");
    const bool small = tokens_stride > 0 && tokens_stride <= kSmallAppend;
    // a store with neither an index nor a successor-count cache is drafted
    // by scanning it; with the fused gather the append runs inside that scan
    const bool fused_scan = !ctx->index && !ctx->ngram_grams && ctx->fused && small;
    const bool fused = (ctx->index && small) || fused_scan;
    if (!fused) {
        // the same two steps, one after the other on the stream
        pld_status st = pld_append(ctx, tokens, tokens_stride, counts, batch, stream);
        if (st != PLD_OK)
            return st;
        if (ctx->index)
            return pld_draft_store(ctx, batch, n_min, n_max, k_max, out_draft, out_len,
                                   out_match, out_pos, stream);
        return draft(ctx, ctx->store_rows, nullptr, 0, 0, ctx->store_len, batch, n_min, n_max,
                     k_max, out_draft, out_len, out_match, out_pos, stream);
    }
    if (batch == 0)
        return PLD_OK;
    if (!tokens || !counts)
        return fail(PLD_EINVAL, "null buffer pointer");
    if (((uintptr_t)tokens | (uintptr_t)counts | (uintptr_t)out_draft | (uintptr_t)out_len |
         (uintptr_t)out_match | (uintptr_t)out_pos) & 3u)
        return fail(PLD_EINVAL, "buffers must be 4-byte aligned");
    if (fused_scan) {
        const AppendIn app{tokens, tokens_stride, counts};
        return draft(ctx, nullptr, ctx->store, ctx->pitch, 0, ctx->store_len, batch, n_min,
                     n_max, k_max, out_draft, out_len, out_match, out_pos, stream, nullptr,
                     nullptr, &app);
    }
    hipError_t e = pld::launch_append_draft_indexed(index_args(ctx), tokens, tokens_stride, counts,
                                                    batch, n_min, n_max, k_max, out_draft,
                                                    out_len, out_match, out_pos, stream);
    if (e != hipSuccess)
        return hip_fail(e, "append-draft launch");
    return PLD_OK;
}

pld_status pld_ngram_params_default(pld_ngram_params *params)
{
    if (!params)
        return fail(PLD_EINVAL, "params is null");
    params->n_min = 1;
    params->n_max = PLD_NGRAM_MAX_N;
    for (int i = 0; i < PLD_NGRAM_MAX_N; ++i) {
        params->min_count[i] = 1;
        params->min_percent[i] = 50;
    }
    return PLD_OK;
}

// Checks a successor-count draft's arguments and fills `d`; PLD_OK or the
// failure.
pld_status ngram_draft_args(pld_ctx *ctx, const pld_ngram_params *params, int32_t batch,
                            int32_t k_max, int32_t *out_draft, int32_t *out_len,
                            int32_t *out_levels, pld::NgramDraftArgs &d)
{
    if (!ctx)
        return fail(PLD_EINVAL, "ctx is null");
    if (!ctx->ngram_grams)
        return fail(PLD_EINVAL, "context has no successor-count cache (see pld_create_ngram)");
    if (!params)
        return fail(PLD_EINVAL, "params is null");
    const pld_ngram_params &p = *params;
    if (p.n_min < 1 || p.n_max < p.n_min || p.n_max > ctx->ngram_n_max)
        return fail(PLD_EINVAL, "need 1 <= n_min <= n_max <= %d, the cached lengths "
                    "(got n_min=%d n_max=%d)", ctx->ngram_n_max, p.n_min, p.n_max);
    for (int i = 0; i < PLD_NGRAM_MAX_N; ++i) {
        if (p.min_count[i] < 0 || p.min_percent[i] < 0 || p.min_percent[i] > 100)
            return fail(PLD_EINVAL, "need min_count >= 0 and 0 <= min_percent <= 100 "
                        "(length %d: %d, %d)", i + 1, p.min_count[i], p.min_percent[i]);
    }
    if (k_max < 1)
        return fail(PLD_EINVAL, "k_max must be >= 1 (got %d)", k_max);
    if (batch < 0 || batch > ctx->max_batch)
        return fail(PLD_EINVAL, "batch %d outside [0, max_batch=%d]", batch, ctx->max_batch);
    if (batch > 0 && (!out_draft || !out_len))
        return fail(PLD_EINVAL, "null buffer pointer");
    if (((uintptr_t)out_draft | (uintptr_t)out_len | (uintptr_t)out_levels) & 3u)
        return fail(PLD_EINVAL, "outputs must be 4-byte aligned");
    if ((int64_t)batch * k_max > INT64_MAX / 4)
        return fail(PLD_EINVAL, "batch * k_max too large");
    d.n_min = p.n_min;
    d.n_max = p.n_max;
    for (int i = 0; i < PLD_NGRAM_MAX_N; ++i) {
        d.min_count[i] = p.min_count[i];
        d.min_percent[i] = p.min_percent[i];
    }
    d.batch = batch;
    d.k_max = k_max;
    d.out_draft = out_draft;
    d.out_len = out_len;
    d.out_levels = out_levels;
    return PLD_OK;
}

pld_status pld_draft_ngram(pld_ctx *ctx, const pld_ngram_params *params, int32_t batch,
                           int32_t k_max, int32_t *out_draft, int32_t *out_len,
                           int32_t *out_levels, hipStream_t stream)
{
    pld::NgramDraftArgs d;
    pld_status st = ngram_draft_args(ctx, params, batch, k_max, out_draft, out_len, out_levels, d);
    if (st != PLD_OK || batch == 0)
        return st;
    hipError_t e = pld::launch_ngram_draft(ngram_args(ctx), d, stream);
    if (e != hipSuccess)
        return hip_fail(e, "n-gram draft launch");
    return PLD_OK;
}

pld_status pld_append_draft_ngram(pld_ctx *ctx, const int32_t *tokens, int64_t tokens_stride,
                                  const int32_t *counts, int32_t batch,
                                  const pld_ngram_params *params, int32_t k_max,
                                  int32_t *out_draft, int32_t *out_len, int32_t *out_levels,
                                  hipStream_t stream)
{
    // every argument of both steps is checked before anything is enqueued
    pld::NgramDraftArgs d;
    pld_status st = ngram_draft_args(ctx, params, batch, k_max, out_draft, out_len, out_levels, d);
    if (st != PLD_OK)
        return st;
    if (tokens_stride < 0)
        return fail(PLD_EINVAL, "tokens_stride must be >= 0");
    if (batch == 0)
        return PLD_OK;
    if (!tokens || !counts)
        return fail(PLD_EINVAL, "null buffer pointer");
    if (tokens_stride == 0 || tokens_stride > kSmallAppend) {
        st = pld_append(ctx, tokens, tokens_stride, counts, batch, stream);
        if (st != PLD_OK)
            return st;
        return pld_draft_ngram(ctx, params, batch, k_max, out_draft, out_len, out_levels, stream);
    }
    hipError_t e = pld::launch_append_draft_ngram(ngram_args(ctx), tokens, tokens_stride, counts,
                                                  d, stream);
    if (e != hipSuccess)
        return hip_fail(e, "n-gram append-draft launch");
    return PLD_OK;
}

pld_status pld_index_fingerprint_bits(pld_ctx *ctx, int32_t bits)
{
    if (!ctx)
        return fail(PLD_EINVAL, "ctx is null");
    if (!ctx->index)
        return fail(PLD_EINVAL, "context has no n-gram index (see pld_create_indexed)");
    if (bits < 0 || bits > 32)
        return fail(PLD_EINVAL, "bits must be in [0, 32] (got %d)", bits);
    ctx->index_fp_mask = bits == 32 ? 0xffffffffu : ((1u << bits) - 1u);
    return PLD_OK;
}

pld_status pld_draft_store(pld_ctx *ctx, int32_t batch, int32_t n_min, int32_t n_max,
                           int32_t k_max, int32_t *out_draft, int32_t *out_len,
                           int32_t *out_match, int32_t *out_pos, hipStream_t stream)
{
    if (!ctx)
        return fail(PLD_EINVAL, "ctx is null");
    if (!ctx->index)
        return fail(PLD_EINVAL, "context has no n-gram index (see pld_create_indexed)");
    if (n_min < ctx->index_lo || n_max < n_min || n_max > ctx->index_hi)
        return fail(PLD_EINVAL, "need %d <= n_min <= n_max <= %d, the indexed lengths "
                    "(got n_min=%d n_max=%d)", ctx->index_lo, ctx->index_hi, n_min, n_max);
    if (k_max < 1)
        return fail(PLD_EINVAL, "k_max must be >= 1 (got %d)", k_max);
    if (batch < 0 || batch > ctx->max_batch)
        return fail(PLD_EINVAL, "batch %d outside [0, max_batch=%d]", batch, ctx->max_batch);
    if (batch == 0)
        return PLD_OK;
    if (!out_draft || !out_len || !out_match)
        return fail(PLD_EINVAL, "null buffer pointer");
    if (((uintptr_t)out_draft | (uintptr_t)out_len | (uintptr_t)out_match |
         (uintptr_t)out_pos) & 3u)
        return fail(PLD_EINVAL, "outputs must be 4-byte aligned");
    hipError_t e = pld::launch_index_draft(index_args(ctx), batch, n_min, n_max, k_max,
                                           out_draft, out_len, out_match, out_pos, stream);
    if (e != hipSuccess)
        return hip_fail(e, "index draft launch");
    return PLD_OK;
}

pld_status pld_draft_batch(pld_ctx *ctx, const int32_t *const *histories,
                           const int32_t *lengths, int32_t batch, int32_t n_min,
                           int32_t n_max, int32_t k_max, int32_t *out_draft,
                           int32_t *out_len, int32_t *out_match, hipStream_t stream)
{
    return draft(ctx, histories, nullptr, 0, 0, lengths, batch, n_min, n_max, k_max, out_draft,
                 out_len, out_match, nullptr, stream);
}

pld_status pld_draft_batch_pos(pld_ctx *ctx, const int32_t *const *histories,
                               const int32_t *lengths, int32_t batch, int32_t n_min,
                               int32_t n_max, int32_t k_max, int32_t *out_draft,
                               int32_t *out_len, int32_t *out_match, int32_t *out_pos,
                               hipStream_t stream)
{
    if (batch > 0 && !out_pos)
        return fail(PLD_EINVAL, "out_pos is null");
    return draft(ctx, histories, nullptr, 0, 0, lengths, batch, n_min, n_max, k_max, out_draft,
                 out_len, out_match, out_pos, stream);
}

pld_status pld_draft_batch_noalloc(const int32_t *const *histories, const int32_t *lengths,
                                   int32_t batch, int64_t max_len, int32_t n_min, int32_t n_max,
                                   int32_t k_max, int32_t *out_draft, int32_t *out_len,
                                   int32_t *out_match, int32_t *out_pos, uint32_t *out_err,
                                   hipStream_t stream)
{
    if (n_min < 1 || n_max < n_min || n_max > PLD_N_MAX_LIMIT)
        return fail(PLD_EINVAL, "need 1 <= n_min <= n_max <= %d (got n_min=%d n_max=%d)",
                    PLD_N_MAX_LIMIT, n_min, n_max);
    if (k_max < 1)
        return fail(PLD_EINVAL, "k_max must be >= 1 (got %d)", k_max);
    if (batch < 0 || batch > pld::kStaticMaxBatch)
        return fail(PLD_EINVAL, "batch %d outside [0, %d] (the static reduction state's size)",
                    batch, pld::kStaticMaxBatch);
    if (max_len < 1 || max_len > 0x7fffffffLL)
        return fail(PLD_EINVAL, "max_len must be in [1, 2^31-1] (got %lld)", (long long)max_len);
    if (batch > 0 && (!histories || !lengths || !out_draft || !out_len || !out_match || !out_pos))
        return fail(PLD_EINVAL, "null buffer pointer");
    if (batch > 0 && (((uintptr_t)lengths | (uintptr_t)out_draft | (uintptr_t)out_len |
                       (uintptr_t)out_match | (uintptr_t)out_pos | (uintptr_t)out_err) & 3u))
        return fail(PLD_EINVAL, "lengths, outputs and out_err must be 4-byte aligned");
    if ((int64_t)batch * k_max > INT64_MAX / 4)
        return fail(PLD_EINVAL, "batch * k_max too large");
    const int32_t ml = (int32_t)max_len;
    const int32_t tile = auto_tile(ml, batch);
    if (pld::scan_grid(ml, batch, tile) > 0x7fffffffLL)
        return fail(PLD_EINVAL, "grid too large: batch %d x tiles for max_len %d", batch, ml);
    if (batch == 0)
        return PLD_OK;
    pld::StaticScratch *sc = nullptr;
    hipError_t e = pld::static_scratch(&sc, stream);
    if (e != hipSuccess)
        return hip_fail(e, "static reduction state");
    pld::DraftArgs a;
    memset(&a, 0, sizeof(a));
    a.histories = histories;
    a.lengths = lengths;
    a.batch = batch;
    a.n_min = n_min;
    a.n_max = n_max;
    a.k_max = k_max;
    a.max_len = ml;
    a.fused = 1;
    a.out_draft = out_draft;
    a.out_len = out_len;
    a.out_match = out_match;
    a.out_pos = out_pos;
    a.slots = sc->slots;
    a.err = out_err ? (unsigned int *)out_err : &sc->err;
    a.zero16 = &sc->zero16;
    e = pld::launch_draft(a, tile, stream);
    if (e != hipSuccess)
        return hip_fail(e, "draft kernel launch");
    return PLD_OK;
}

pld_status pld_draft_batch_strided(pld_ctx *ctx, const int32_t *base, int64_t stride,
                                   const int32_t *lengths, int32_t min_len, int32_t batch,
                                   int32_t n_min, int32_t n_max, int32_t k_max,
                                   int32_t *out_draft, int32_t *out_len, int32_t *out_match,
                                   int32_t *out_pos, hipStream_t stream)
{
    if (stride <= 0)
        return fail(PLD_EINVAL, "strided batch: stride must be positive (got %lld)",
                    (long long)stride);
    return draft(ctx, nullptr, base, stride, min_len, lengths, batch, n_min, n_max, k_max,
                 out_draft, out_len, out_match, out_pos, stream);
}

pld_status pld_fuse_params_default(pld_fuse_params *params)
{
    if (!params)
        return fail(PLD_EINVAL, "params is null");
    // HyperQwen lookup-drafting page, steps 2 and 3: a 7-token drafter head,
    // 15 draft positions in a long block, replace at a match of 8 (6 with 2
    // agreeing tokens), fill the tail at 4, enter after 2 near-full steps,
    // hold 3; near-full = at most 1 position short (a reading)
    *params = pld_fuse_params{7, 15, 8, 6, 2, 4, 2, 3, 1};
    return PLD_OK;
}

pld_status pld_fuse(pld_ctx *ctx, const pld_fuse_params *params, const int32_t *lookup,
                    int32_t lookup_k, const int32_t *lookup_len, const int32_t *lookup_match,
                    const int32_t *drafter, const int32_t *accepted, int32_t *state,
                    int32_t batch, int32_t *out_block, int32_t *out_positions,
                    uint64_t *out_src, hipStream_t stream)
{
    pld::FuseArgs a;
    pld_status st = fuse_args(ctx, params, lookup, lookup_k, lookup_len, lookup_match, drafter,
                              accepted, state, batch, out_block, out_positions, out_src, a);
    if (st != PLD_OK || batch == 0)
        return st;
    hipError_t e = pld::launch_fuse(a, batch, stream);
    if (e != hipSuccess)
        return hip_fail(e, "fuse kernel launch");
    return PLD_OK;
}

pld_status pld_draft_fuse_batch(pld_ctx *ctx, const int32_t *const *histories,
                                const int32_t *lengths, int32_t batch, int32_t n_min,
                                int32_t n_max, int32_t k_max, int32_t *out_draft,
                                int32_t *out_len, int32_t *out_match,
                                const pld_fuse_params *params, const int32_t *drafter,
                                const int32_t *accepted, int32_t *state, int32_t *out_block,
                                int32_t *out_positions, uint64_t *out_src, hipStream_t stream)
{
    if (ctx && k_max < 1)
        return fail(PLD_EINVAL, "k_max must be >= 1 (got %d)", k_max);
    // the lookup draft the fusion reads is this call's own output row
    pld::FuseArgs f;
    pld_status st = fuse_args(ctx, params, out_draft, k_max, out_len, out_match, drafter,
                              accepted, state, batch, out_block, out_positions, out_src, f);
    if (st != PLD_OK)
        return st;
    return draft(ctx, histories, nullptr, 0, 0, lengths, batch, n_min, n_max, k_max, out_draft,
                 out_len, out_match, nullptr, stream, &f);
}

pld_status pld_control_params_default(pld_control_params *params)
{
    if (!params)
        return fail(PLD_EINVAL, "params is null");
    // Strata prompt-lookup page, section 5: the lookup must beat the MTP
    // draft by 5%; section 1: the MTP layer drafts 3 tokens. The weights,
    // priors and bucket edges are readings.
    *params = pld_control_params{0.1, 0.1, 1.05, 0.5, 1.0, 3, {6, 8, 12}};
    return PLD_OK;
}


pld_status pld_control(pld_ctx *ctx, const pld_control_params *params, const int32_t *accepted,
                       const double *round_time, const int32_t *lookup_len,
                       const int32_t *lookup_match, double *state, int32_t batch,
                       int32_t *out_source, double *out_rates, hipStream_t stream)
{
    pld::ControlArgs a;
    pld_status st = control_args(ctx, params, accepted, round_time, lookup_len, lookup_match,
                                 state, batch, out_source, out_rates, false, a);
    if (st != PLD_OK || batch == 0)
        return st;
    hipError_t e = pld::launch_control(a, stream);
    if (e != hipSuccess)
        return hip_fail(e, "control kernel launch");
    return PLD_OK;
}

pld_status pld_draft_control_batch(pld_ctx *ctx, const int32_t *const *histories,
                                   const int32_t *lengths, int32_t batch, int32_t n_min,
                                   int32_t n_max, int32_t k_max, int32_t *out_draft,
                                   int32_t *out_len, int32_t *out_match,
                                   const pld_control_params *params, const int32_t *accepted,
                                   const double *round_time, double *state, int32_t *out_source,
                                   double *out_rates, hipStream_t stream)
{
    // the lookup draft the controller reads is this call's own output
    pld::ControlArgs c;
    pld_status st = control_args(ctx, params, accepted, round_time, out_len, out_match, state,
                                 batch, out_source, out_rates, true, c);
    if (st != PLD_OK)
        return st;
    return draft(ctx, histories, nullptr, 0, 0, lengths, batch, n_min, n_max, k_max, out_draft,
                 out_len, out_match, nullptr, stream, nullptr, &c);
}

pld_status pld_sync(pld_ctx *ctx, hipStream_t stream)
{
    if (!ctx)
        return fail(PLD_EINVAL, "ctx is null");
    unsigned int bits = 0;
    // every stream first: a kernel of this context still running elsewhere
    // could otherwise set a bit between the read and the clear below
    hipError_t e = hipStreamSynchronize(stream);
    if (e == hipSuccess)
        e = hipDeviceSynchronize();
    if (e == hipSuccess)
        e = hipMemcpy(&bits, ctx->err, sizeof(bits), hipMemcpyDeviceToHost);
    if (e == hipSuccess && bits)
        e = hipMemset(ctx->err, 0, sizeof(unsigned int));
    if (e == hipSuccess && bits)
        e = hipDeviceSynchronize();
    if (e != hipSuccess)
        return hip_fail(e, "pld_sync");
    if (!bits)
        return PLD_OK;
    // every problem read in this call is named; capacity wins the status
    const pld_status st =
        (bits & (pld::kErrLenCapacity | pld::kErrAppendCapacity)) ? PLD_ECAPACITY : PLD_EINVAL;
    return fail(st, "device reported:%s%s%s%s%s%s%s%s",
                (bits & pld::kErrLenCapacity) ? " a history longer than max_len;" : "",
                (bits & pld::kErrAppendCapacity) ? " an append past max_len;" : "",
                (bits & pld::kErrLenNegative) ? " a negative length;" : "",
                (bits & pld::kErrBadRow) ? " a null or misaligned row pointer;" : "",
                (bits & pld::kErrAppendNegative) ? " a negative append count;" : "",
                (bits & pld::kErrBelowMinLen) ? " a length below the promised min_len;" : "",
                (bits & pld::kErrFuseInput) ? " inconsistent fusion inputs;" : "",
                (bits & pld::kErrControlInput) ? " a controller outcome out of range;" : "");
}

const char *pld_strerror(pld_status status)
{
    switch (status) {
    case PLD_OK: return "success";
    case PLD_EINVAL: return "invalid argument";
    case PLD_ENOMEM: return "out of device memory";
    case PLD_EHIP: return "HIP runtime error";
    case PLD_ECAPACITY: return "history capacity exceeded";
    }
    return "unknown status";
}

const char *pld_last_error(void)
{
    return g_last_error;
}

}  // extern "C"
