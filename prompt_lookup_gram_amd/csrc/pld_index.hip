// Incremental n-gram index over the context's history store, and drafting
// from it, for gfx950 (MI355X).
//
// The Strata prompt-lookup page (section 4) keeps an index from n-grams to
// history positions that grows by O(1) work per appended token, so that a
// lookup does not rescan the history. Here the index answers exactly the
// same question as the scan (HyperQwen lookup-drafting page, step 1): the
// longest suffix of n_min..n_max tokens with an earlier occurrence, and its
// most recent occurrence. For each length n the index holds one
// open-addressed table mapping every n-gram of the history to the end
// position of its most recent occurrence that can be drafted from (an end
// e <= L - 2: the suffix itself and its own end are left out). A query
// probes the tables of all lengths at once, one lane per length; the
// longest length whose suffix n-gram is found, with the position stored for
// it, is the scan's answer:
//  - the longest length with any occurrence is the longest n whose table
//    holds the suffix n-gram;
//  - at that length the table keeps the largest end position, which is the
//    most recent start j = e - n + 1.
//
// Table entries are 64-bit words (fingerprint << 32 | end + 1); 0 is empty.
// A matching fingerprint is confirmed by comparing the n tokens in the
// history, so a fingerprint collision only costs another probe. Tables have
// at least twice as many slots as max_len, so a free slot always exists and
// a probe sequence always ends. Entries are never removed (positions only
// grow) except when the whole store is reset.
//
// pld_index_insert runs before the append's copy: for every end position
// that the append makes draftable (old L - 1 .. new L - 2) it inserts the
// n-grams ending there, reading old tokens from the store and new ones from
// the append's source buffer. Concurrent inserts of one n-gram claim a slot
// with a compare-and-swap and keep the largest position with a 64-bit
// atomicMax (the fingerprint half of the word is the same).

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "pld_kernels.h"

namespace pld {

namespace {

typedef unsigned long long u64;
constexpr int kWave = 64;

// Hash of an n-gram read backwards from its end: one step per token, then a
// final mix (a 64-bit multiply-xorshift finaliser).
__device__ __forceinline__ u64 hstep(u64 h, int32_t t)
{
    h ^= (uint32_t)t;
    h *= 0x9e3779b97f4a7c15ull;
    return h ^ (h >> 29);
}

__device__ __forceinline__ u64 hfinal(u64 h)
{
    h ^= h >> 33;
    h *= 0xff51afd7ed558ccdull;
    h ^= h >> 33;
    h *= 0xc4ceb9fe1a85ec53ull;
    return h ^ (h >> 33);
}

constexpr u64 kHashSeed = 0x243f6a8885a308d3ull;

__device__ __forceinline__ u64 *table_of(const IndexArgs &a, int b, int n)
{
    return a.table + ((int64_t)b * (a.n_hi - a.n_lo + 1) + (n - a.n_lo)) * a.cap;
}

// Token q of request b during an append: from the store below the old
// length, from the append's source row above it.
struct AppendView {
    const int32_t *store_row;
    const int32_t *src;
    int32_t old_len;
    __device__ __forceinline__ int32_t at(int64_t q) const
    {
        return q < old_len ? store_row[q] : src[q - old_len];
    }
};

__device__ __forceinline__ bool same_gram(const AppendView &v, int64_t p, int64_t q, int n)
{
    for (int i = 0; i < n; ++i)
        if (v.at(p - i) != v.at(q - i))
            return false;
    return true;
}

// Inserts the n-gram ending at e (hash f) into its table, keeping the
// largest end position per n-gram.
__device__ void insert_gram(u64 *tab, int64_t cap, const AppendView &v, int64_t e, int n, u64 f)
{
    const uint32_t fp = (uint32_t)(f >> 32);
    const u64 word = ((u64)fp << 32) | (uint32_t)(e + 1);
    int64_t slot = (int64_t)(f & (u64)(cap - 1));
    for (int64_t probe = 0; probe < cap; ++probe) {
        u64 cur = __hip_atomic_load(tab + slot, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        if (cur == 0) {
            u64 expected = 0;
            if (__hip_atomic_compare_exchange_strong(tab + slot, &expected, word, __ATOMIC_RELAXED,
                                                     __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT))
                return;
            cur = expected;  // another insert claimed the slot first
        }
        if ((uint32_t)(cur >> 32) == fp) {
            const int64_t q = (int64_t)(uint32_t)cur - 1;
            if (same_gram(v, e, q, n)) {
                __hip_atomic_fetch_max(tab + slot, word, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
                return;
            }
        }
        slot = (slot + 1) & (cap - 1);
    }
}

__global__ __launch_bounds__(256) void pld_index_insert(IndexArgs a, const int32_t *tokens,
                                                        int64_t tokens_stride,
                                                        const int32_t *counts)
{
    const int b = blockIdx.x;
    const int32_t old_len = a.lengths[b];
    const int32_t c = counts[b];
    // an append the copy kernel will reject inserts nothing
    if (c <= 0 || old_len < 0 || (int64_t)old_len + c > a.max_len)
        return;
    const int64_t new_len = (int64_t)old_len + c;
    AppendView v{a.store + (int64_t)b * a.pitch, tokens + (int64_t)b * tokens_stride, old_len};
    const int64_t e_first = old_len > 0 ? old_len - 1 : 0;
    const int64_t step = (int64_t)gridDim.y * blockDim.x;
    for (int64_t e = e_first + (int64_t)blockIdx.y * blockDim.x + threadIdx.x; e <= new_len - 2;
         e += step) {
        u64 h = kHashSeed;
        for (int n = 1; n <= a.n_hi && e - n + 1 >= 0; ++n) {
            h = hstep(h, v.at(e - n + 1));
            if (n >= a.n_lo)
                insert_gram(table_of(a, b, n), a.cap, v, e, n, hfinal(h));
        }
    }
}

// One wavefront per request: lane i holds suffix token L - 1 - i, lane
// n - 1 probes the table of length n.
__global__ __launch_bounds__(kWave) void pld_index_draft(IndexArgs a, int32_t n_min, int32_t n_max,
                                                         int32_t k_max, int32_t *out_draft,
                                                         int32_t *out_len, int32_t *out_match,
                                                         int32_t *out_pos)
{
    const int b = blockIdx.x;
    const int lane = threadIdx.x;
    const int32_t len = a.lengths[b];
    const int32_t L = len >= 0 && len <= a.max_len ? len : 0;
    if (lane == 0 && L != len)
        atomicOr(a.err, len < 0 ? kErrLenNegative : kErrLenCapacity);
    const int32_t *row = a.store + (int64_t)b * a.pitch;
    const int32_t mhat = L - 1 < n_max ? L - 1 : n_max;

    const int32_t tok = lane < mhat ? row[L - 1 - lane] : 0;
    // hash of the suffix n-gram for n = lane + 1, built token by token
    u64 h = kHashSeed, mine = 0;
    for (int i = 0; i < mhat; ++i) {
        h = hstep(h, __builtin_amdgcn_readlane(tok, i));
        if (lane == i)
            mine = h;
    }
    const int n = lane + 1;
    u64 key = 0;
    if (n >= n_min && n <= mhat) {
        const u64 f = hfinal(mine);
        const uint32_t fp = (uint32_t)(f >> 32);
        const u64 *tab = table_of(a, b, n);
        int64_t slot = (int64_t)(f & (u64)(a.cap - 1));
        for (int64_t probe = 0; probe < a.cap; ++probe) {
            const u64 cur = tab[slot];
            if (cur == 0)
                break;
            if ((uint32_t)(cur >> 32) == fp) {
                const int64_t q = (int64_t)(uint32_t)cur - 1;
                bool same = q <= L - 2 && q - n + 1 >= 0;
                for (int i = 0; same && i < n; ++i)
                    same = row[q - i] == row[L - 1 - i];
                if (same) {
                    key = ((u64)(uint32_t)n << 32) | (uint32_t)q;
                    break;
                }
            }
            slot = (slot + 1) & (a.cap - 1);
        }
    }
    // longest length, then (the one position kept for it) the key's end
    for (int off = 32; off >= 1; off >>= 1) {
        const u64 o = __shfl_xor(key, off);
        key = o > key ? o : key;
    }
    int32_t m = 0, d = 0, e = -1;
    if (key != 0) {
        m = (int32_t)(key >> 32);
        e = (int32_t)(key & 0xffffffffu);
        const int32_t follow = L - 1 - e;
        d = follow < k_max ? follow : k_max;
    }
    int32_t *orow = out_draft + (int64_t)b * k_max;
    for (int t = lane; t < k_max; t += kWave)
        orow[t] = t < d ? row[(int64_t)e + 1 + t] : -1;
    if (lane == 0) {
        out_len[b] = d;
        out_match[b] = m;
        if (out_pos)
            out_pos[b] = key != 0 ? e - m + 1 : -1;
    }
}

__global__ __launch_bounds__(256) void pld_fill_u64(u64 *p, int64_t n)
{
    const int64_t stride = (int64_t)gridDim.x * blockDim.x;
    for (int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; i < n; i += stride)
        p[i] = 0;
}

}  // namespace

hipError_t launch_index_insert(const IndexArgs &a, const int32_t *tokens, int64_t tokens_stride,
                               const int32_t *counts, int32_t batch, int32_t chunks,
                               hipStream_t s)
{
    if (batch <= 0)
        return hipSuccess;
    hipLaunchKernelGGL(pld_index_insert, dim3((unsigned)batch, (unsigned)chunks), dim3(256), 0, s,
                       a, tokens, tokens_stride, counts);
    return hipGetLastError();
}

hipError_t launch_index_draft(const IndexArgs &a, int32_t batch, int32_t n_min, int32_t n_max,
                              int32_t k_max, int32_t *out_draft, int32_t *out_len,
                              int32_t *out_match, int32_t *out_pos, hipStream_t s)
{
    if (batch <= 0)
        return hipSuccess;
    hipLaunchKernelGGL(pld_index_draft, dim3((unsigned)batch), dim3(kWave), 0, s, a, n_min, n_max,
                       k_max, out_draft, out_len, out_match, out_pos);
    return hipGetLastError();
}

hipError_t launch_index_clear(const IndexArgs &a, int32_t batch, hipStream_t s)
{
    const int64_t n = (int64_t)batch * (a.n_hi - a.n_lo + 1) * a.cap;
    if (n <= 0)
        return hipSuccess;
    int64_t blocks = (n + 255) / 256;
    if (blocks > 65536)
        blocks = 65536;
    hipLaunchKernelGGL(pld_fill_u64, dim3((unsigned)blocks), dim3(256), 0, s, a.table, n);
    return hipGetLastError();
}

}  // namespace pld
