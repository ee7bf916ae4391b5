// Successor-count n-gram cache over the context's history store, and
// drafting from it, for gfx950 (MI355X).
//
// The llama.cpp page (the section on what prompt lookup decoding is)
// describes a context cache: statistics of the n-grams of sizes 1 to 4 in
// the current token stream and of the tokens that followed them. A draft is
// built one token at a time, each token one lookup of the tokens just before
// it, and fixed thresholds decide whether a lookup may propose its most
// frequent successor. The rule computed here: for each draft token, the
// contexts of n_max down to n_min tokens (the history followed by the tokens
// drafted so far) are looked up; the first length whose context was followed
// at least max(1, min_count[n]) times, with its most frequent successor
// holding at least min_percent[n] percent of them, proposes that successor
// (the smaller token on a tie). The draft ends at the first token no length
// can propose, or at k_max. Drafted tokens are never counted.
//
// Layout, per request and context length n, two open-addressed tables of
// `cap` slots (a power of two at least twice max_len, so at most half full
// and every probe sequence reaches an empty slot):
//  - the pair table holds one 64-bit word per (n + 1)-gram of the history,
//    (count << 32 | end + 1) with `end` the end position of one occurrence;
//    count is how often the n-gram's first n tokens were followed by its
//    last one;
//  - the gram table holds 32 bytes per n-gram that was followed at least
//    once: (count << 32 | end + 1), the occurrences followed by a token;
//    `top`, the packed maximum of (successor count << 32 | ~order(token))
//    over its successors; and the n tokens themselves, for the query.
// The maximum over packed words is the most frequent successor, the
// smaller token on a tie (order() maps signed order onto unsigned). Counts
// only grow, and each increment of a pair's count offers (new count,
// token) to the gram's maximum, so after an append the maximum is exactly
// the one over final counts whatever order the atomics ran in. Nothing is
// approximate: slots are identified by their full tokens (compared in the
// history while inserting, against the stored tokens while drafting), so
// the drafts equal those of a brute-force recount.
//
// Inserts: appending token p (p >= 1) adds, for each n <= min(n_max, p), one
// occurrence of the n-gram h[p - n .. p) followed by h[p]. A slot is claimed
// with a compare-and-swap of its first word; a claimed slot whose stored
// occurrence has the same tokens is incremented with an atomic add.
// Old tokens come from the store and new ones from the append's source row.
//
// Drafting: one wavefront per request; 16 lanes per context length each
// read one slot of a 16-slot window of its probe sequence, so one round
// trip answers all four lengths of one draft token.

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "pld_device.h"
#include "pld_kernels.h"

namespace pld {

namespace {

typedef unsigned long long u64;
constexpr int kWave = 64;
constexpr int kWindow = 16;      // slots one length reads per round trip
constexpr int kGramWords = 4;    // 64-bit words per gram slot
constexpr u64 kOne = 1ull << 32; // count 1 in a slot's first word

__device__ __forceinline__ u64 *gram_table(const NgramArgs &a, int b, int n)
{
    return a.grams + ((int64_t)b * a.n_max + (n - 1)) * a.cap * kGramWords;
}

__device__ __forceinline__ u64 *pair_table(const NgramArgs &a, int b, int n)
{
    return a.pairs + ((int64_t)b * a.n_max + (n - 1)) * a.cap;
}

// (count, token) packed so that the u64 maximum is the larger count, then
// the smaller token.
__device__ __forceinline__ u64 pack_top(uint32_t count, int32_t tok)
{
    return ((u64)count << 32) | (uint32_t)~((uint32_t)tok ^ 0x80000000u);
}

__device__ __forceinline__ int32_t top_token(u64 top)
{
    return (int32_t)(~(uint32_t)top ^ 0x80000000u);
}

// Counts one more occurrence of the (n + 1)-gram tk[0..n] ending at p;
// returns its count after the increment.
__device__ uint32_t insert_pair(u64 *tab, int64_t cap, u64 f, int64_t p, int n,
                                const int32_t *tk, const AppendView &v)
{
    int64_t slot = (int64_t)(f & (u64)(cap - 1));
    for (int64_t probe = 0; probe < cap; ++probe) {
        u64 cur = 0;
        if (__hip_atomic_compare_exchange_strong(tab + slot, &cur, kOne | (uint32_t)(p + 1),
                                                 __ATOMIC_RELAXED, __ATOMIC_RELAXED,
                                                 __HIP_MEMORY_SCOPE_AGENT))
            return 1;
        // the slot counts the (n + 1)-gram ending at r: the same tokens?
        const int64_t r = (int64_t)(uint32_t)cur - 1;
        bool same = true;
        for (int j = 0; j <= n; ++j)
            same = same && v.at(r - n + j) == tk[j];
        if (same)
            return (uint32_t)(__hip_atomic_fetch_add(tab + slot, kOne, __ATOMIC_RELAXED,
                                                     __HIP_MEMORY_SCOPE_AGENT) >> 32) + 1;
        slot = (slot + 1) & (cap - 1);
    }
    return 0;  // not reached: a table is at most half full
}

// Counts one more followed occurrence of the n-gram tk[0..n) ending at
// p - 1 and offers its successor tk[n], now seen `count` times after it.
__device__ void insert_gram(u64 *tab, int64_t cap, u64 f, int64_t p, int n, const int32_t *tk,
                            uint32_t count, const AppendView &v)
{
    const u64 top = pack_top(count, tk[n]);
    int64_t slot = (int64_t)(f & (u64)(cap - 1));
    for (int64_t probe = 0; probe < cap; ++probe) {
        u64 *s = tab + slot * kGramWords;
        u64 cur = 0;
        if (__hip_atomic_compare_exchange_strong(s, &cur, kOne | (uint32_t)p, __ATOMIC_RELAXED,
                                                 __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT)) {
            // this slot is ours: store the tokens for the query (the words
            // past n stay 0 from the clear)
            s[2] = (uint32_t)tk[0] | (n > 1 ? (u64)(uint32_t)tk[1] << 32 : 0);
            if (n > 2)
                s[3] = (uint32_t)tk[2] | (n > 3 ? (u64)(uint32_t)tk[3] << 32 : 0);
            __hip_atomic_fetch_max(s + 1, top, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
            return;
        }
        const int64_t r = (int64_t)(uint32_t)cur - 1;  // end of the n-gram held
        bool same = true;
        for (int j = 0; j < n; ++j)
            same = same && v.at(r - n + 1 + j) == tk[j];
        if (same) {
            __hip_atomic_fetch_add(s, kOne, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
            __hip_atomic_fetch_max(s + 1, top, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
            return;
        }
        slot = (slot + 1) & (cap - 1);
    }
}

// The checks pld_append_kernel makes, in the same words.
__device__ __forceinline__ bool append_ok(const NgramArgs &a, int32_t old_len, int32_t c)
{
    return c >= 0 && old_len >= 0 && (int64_t)old_len + c <= a.max_len;
}

// Inserts items i0, i0 + step, ... of one append: item i is position
// old_len + i / n_max and context length 1 + i % n_max.
__device__ void insert_items(const NgramArgs &a, int b, const AppendView &v, int32_t c,
                             int64_t i0, int64_t step)
{
    const int64_t items = (int64_t)c * a.n_max;
    for (int64_t i = i0; i < items; i += step) {
        const int64_t p = v.old_len + i / a.n_max;
        const int n = 1 + (int)(i % a.n_max);
        if (p - n < 0)
            continue;
        int32_t tk[5];
        u64 h = kHashSeed;
        for (int j = 0; j < n; ++j) {
            tk[j] = v.at(p - n + j);
            h = hstep(h, tk[j]);
        }
        tk[n] = v.at(p);
        const u64 fg = hfinal(h);
        const u64 fp = hfinal(hstep(h, tk[n]));
        const uint32_t count = insert_pair(pair_table(a, b, n), a.cap, fp, p, n, tk, v);
        insert_gram(gram_table(a, b, n), a.cap, fg, p, n, tk, count, v);
    }
}

// Inserts of an append spread over several workgroups per request (large
// appends); pld_append_kernel copies the tokens afterwards.
__global__ __launch_bounds__(256) void pld_ngram_insert(NgramArgs a, const int32_t *tokens,
                                                        int64_t tokens_stride,
                                                        const int32_t *counts)
{
    const int b = blockIdx.x;
    const int32_t old_len = a.lengths[b];
    const int32_t c = counts[b];
    if (c <= 0 || !append_ok(a, old_len, c))
        return;  // nothing to insert, or the copy kernel rejects the append
    AppendView v{a.store + (int64_t)b * a.pitch, tokens + (int64_t)b * tokens_stride, old_len};
    insert_items(a, b, v, c, (int64_t)blockIdx.y * blockDim.x + threadIdx.x,
                 (int64_t)gridDim.y * blockDim.x);
}

// A whole append of one request in one workgroup (small appends, as in a
// decode loop): inserts, copy, then the new length. The inserts read new
// tokens from the source row, so they do not depend on the copy.
__global__ __launch_bounds__(256) void pld_append_ngram(NgramArgs a, const int32_t *tokens,
                                                        int64_t tokens_stride,
                                                        const int32_t *counts)
{
    __shared__ int s_ok;
    const int b = blockIdx.x;
    const int32_t old_len = a.lengths[b];
    const int32_t c = counts[b];
    if (threadIdx.x == 0) {
        const bool ok = append_ok(a, old_len, c);
        if (!ok)
            atomicOr(a.err, c < 0 ? kErrAppendNegative : kErrAppendCapacity);
        s_ok = ok;
    }
    __syncthreads();
    if (!s_ok || c == 0)
        return;
    int32_t *row = a.store + (int64_t)b * a.pitch;
    const int32_t *src = tokens + (int64_t)b * tokens_stride;
    AppendView v{row, src, old_len};
    insert_items(a, b, v, c, threadIdx.x, blockDim.x);
    for (int32_t t = threadIdx.x; t < c; t += blockDim.x)
        row[old_len + t] = src[t];
    __syncthreads();
    if (threadIdx.x == 0)
        a.lengths[b] = old_len + c;
}

__device__ __forceinline__ int32_t by_length(int n, int32_t v1, int32_t v2, int32_t v3, int32_t v4)
{
    return n == 1 ? v1 : n == 2 ? v2 : n == 3 ? v3 : v4;
}

__device__ __forceinline__ u64 readlane64(u64 x, int lane)
{
    const uint32_t lo = __builtin_amdgcn_readlane((uint32_t)x, lane);
    const uint32_t hi = __builtin_amdgcn_readlane((uint32_t)(x >> 32), lane);
    return ((u64)hi << 32) | lo;
}

// One wavefront per request. Lanes 16(n - 1) .. 16n - 1 look up context
// length n: lane w of the group reads slot w of the current 16-slot window
// of the probe sequence. The first slot in probe order that is empty or
// holds the context's tokens ends the group's search; the longest length
// that passes its thresholds proposes the token.
__global__ __launch_bounds__(kWave) void pld_ngram_draft(NgramArgs a, NgramDraftArgs d)
{
    const int b = blockIdx.x;
    const int lane = threadIdx.x;
    int32_t L = a.lengths[b];
    if (L < 0 || L > a.max_len) {
        if (lane == 0)
            atomicOr(a.err, L < 0 ? kErrLenNegative : kErrLenCapacity);
        L = 0;
    }
    const int32_t *row = a.store + (int64_t)b * a.pitch;
    // the last 4 tokens of the stream, oldest first (t3 the newest)
    const int32_t tl = lane < 4 && L - 4 + lane >= 0 ? row[L - 4 + lane] : 0;
    int32_t t0 = __builtin_amdgcn_readlane(tl, 0), t1 = __builtin_amdgcn_readlane(tl, 1);
    int32_t t2 = __builtin_amdgcn_readlane(tl, 2), t3 = __builtin_amdgcn_readlane(tl, 3);
    const int g = lane >> 4, w = lane & (kWindow - 1), n = g + 1;
    const int64_t need = by_length(n, d.min_count[0], d.min_count[1], d.min_count[2],
                                   d.min_count[3]) > 1
                             ? by_length(n, d.min_count[0], d.min_count[1], d.min_count[2],
                                         d.min_count[3])
                             : 1;
    const int64_t pct = by_length(n, d.min_percent[0], d.min_percent[1], d.min_percent[2],
                                  d.min_percent[3]);
    const u64 *tab = n <= a.n_max ? gram_table(a, b, n) : a.grams;
    int32_t *draft_row = d.out_draft + (int64_t)b * d.k_max;
    int32_t *level_row = d.out_levels ? d.out_levels + (int64_t)b * d.k_max : nullptr;
    int64_t len = L;
    int32_t s = 0;
    for (; s < d.k_max; ++s) {
        const bool on = n >= d.n_min && n <= d.n_max && len >= n;
        // this group's context, oldest token first: the last n of t0..t3
        const int32_t c0 = n == 4 ? t0 : n == 3 ? t1 : n == 2 ? t2 : t3;
        const int32_t c1 = n == 4 ? t1 : n == 3 ? t2 : t3;
        const int32_t c2 = n == 4 ? t2 : t3;
        u64 h = hstep(kHashSeed, c0);
        if (n > 1)
            h = hstep(h, c1);
        if (n > 2)
            h = hstep(h, c2);
        if (n > 3)
            h = hstep(h, t3);
        const int64_t home = (int64_t)(hfinal(h) & (u64)(a.cap - 1));
        bool pending = on, found = false;
        u64 word = 0, top = 0;
        for (int64_t it = 0; it < a.cap; it += kWindow) {
            if (__ballot(pending) == 0)
                break;
            bool stop = false, hit = false;
            u64 w0 = 0, w1 = 0;
            if (pending) {
                const u64 *sp = tab + ((home + it + w) & (a.cap - 1)) * kGramWords;
                const ulonglong2 head = *(const ulonglong2 *)sp;
                const ulonglong2 key = *(const ulonglong2 *)(sp + 2);
                w0 = head.x;
                w1 = head.y;
                const bool empty = (uint32_t)w0 == 0;
                const bool same = (int32_t)(uint32_t)key.x == c0 &&
                                  (n < 2 || (int32_t)(key.x >> 32) == c1) &&
                                  (n < 3 || (int32_t)(uint32_t)key.y == c2) &&
                                  (n < 4 || (int32_t)(key.y >> 32) == t3);
                hit = !empty && same;
                stop = empty || hit;
            }
            const u64 stops = __ballot(stop);
            const uint32_t mine = (uint32_t)(stops >> (g * kWindow)) & 0xffffu;
            // the group's first stopping slot in probe order
            const int src = g * kWindow + (mine ? __builtin_ctz(mine) : 0);
            const int src_hit = __shfl((int)hit, src);
            const u64 src_w0 = __shfl(w0, src);
            const u64 src_w1 = __shfl(w1, src);
            if (pending && mine) {
                found = src_hit != 0;
                word = src_w0;
                top = src_w1;
                pending = false;
            }
        }
        const int64_t count = (int64_t)(word >> 32);
        const int64_t topc = (int64_t)(top >> 32);
        const bool pass = on && found && count >= need && 100 * topc >= pct * count;
        const u64 leaders = __ballot(pass && w == 0);
        if (leaders == 0)
            break;
        const int best = 63 - __builtin_clzll(leaders);  // the longest passing length
        const int32_t tok = top_token(readlane64(top, best));
        if (lane == 0) {
            draft_row[s] = tok;
            if (level_row)
                level_row[s] = best / kWindow + 1;
        }
        t0 = t1;
        t1 = t2;
        t2 = t3;
        t3 = tok;
        ++len;
    }
    for (int32_t i = s + lane; i < d.k_max; i += kWave) {
        draft_row[i] = -1;
        if (level_row)
            level_row[i] = 0;
    }
    if (lane == 0)
        d.out_len[b] = s;
}

__global__ __launch_bounds__(256) void pld_fill_zero(u64 *p, int64_t n)
{
    const int64_t stride = (int64_t)gridDim.x * blockDim.x;
    for (int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; i < n; i += stride)
        p[i] = 0;
}

hipError_t fill_zero(u64 *p, int64_t n, hipStream_t s)
{
    if (n <= 0)
        return hipSuccess;
    int64_t blocks = (n + 255) / 256;
    if (blocks > 65536)
        blocks = 65536;
    hipLaunchKernelGGL(pld_fill_zero, dim3((unsigned)blocks), dim3(256), 0, s, p, n);
    return hipGetLastError();
}

}  // namespace

hipError_t launch_ngram_insert(const NgramArgs &a, const int32_t *tokens, int64_t tokens_stride,
                               const int32_t *counts, int32_t batch, int32_t chunks,
                               hipStream_t s)
{
    if (batch <= 0)
        return hipSuccess;
    hipLaunchKernelGGL(pld_ngram_insert, dim3((unsigned)batch, (unsigned)chunks), dim3(256), 0, s,
                       a, tokens, tokens_stride, counts);
    return hipGetLastError();
}

hipError_t launch_append_ngram(const NgramArgs &a, const int32_t *tokens, int64_t tokens_stride,
                               const int32_t *counts, int32_t batch, hipStream_t s)
{
    if (batch <= 0)
        return hipSuccess;
    hipLaunchKernelGGL(pld_append_ngram, dim3((unsigned)batch), dim3(256), 0, s, a, tokens,
                       tokens_stride, counts);
    return hipGetLastError();
}

hipError_t launch_ngram_draft(const NgramArgs &a, const NgramDraftArgs &d, hipStream_t s)
{
    if (d.batch <= 0)
        return hipSuccess;
    hipLaunchKernelGGL(pld_ngram_draft, dim3((unsigned)d.batch), dim3(kWave), 0, s, a, d);
    return hipGetLastError();
}

hipError_t launch_ngram_clear(const NgramArgs &a, int32_t batch, hipStream_t s)
{
    const int64_t slots = (int64_t)batch * a.n_max * a.cap;
    hipError_t e = fill_zero(a.grams, slots * kGramWords, s);
    if (e == hipSuccess)
        e = fill_zero(a.pairs, slots, s);
    return e;
}

}  // namespace pld
