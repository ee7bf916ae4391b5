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
// An insert walks the probe sequence of its hash to the first slot that is
// empty (claimed with a compare-and-swap) or holds its fingerprint, and
// keeps the larger end there with a 64-bit atomicMax (the fingerprint half
// is the same). Slots are never emptied and never change fingerprint, so
// for each fingerprint that first slot is fixed, every n-gram with that
// fingerprint merges into it, and the slot holds the largest end over all of
// them. A query walks the same sequence: an empty slot first means the
// n-gram was never inserted; otherwise the stored end is confirmed against
// the history's tokens, and a confirmed end is the n-gram's most recent
// occurrence (it is the largest end of all n-grams merged there). An end
// that does not confirm means two n-grams share a fingerprint; the request
// is then answered by an exact scan of its history. Tables have at least
// twice as many slots as max_len, so a free slot always exists and every
// probe sequence ends.
//
// Inserts run before the append's copy: for every end position that the
// append makes draftable (old L - 1 .. new L - 2) the n-grams ending there
// are inserted, old tokens read from the store and new ones from the
// append's source rows.

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "pld_device.h"
#include "pld_kernels.h"

namespace pld {

namespace {

typedef unsigned long long u64;
constexpr int kWave = 64;

// LDS tokens for the n-grams of a one-workgroup append (appends up to 1,024
// tokens plus the 63 before them; longer ones hash from memory).
constexpr int kAppendWindow = 1024 + 64;

__device__ __forceinline__ u64 *table_of(const IndexArgs &a, int b, int n)
{
    return a.table + ((int64_t)b * (a.n_hi - a.n_lo + 1) + (n - a.n_lo)) * a.cap;
}

// Inserts the end e of an n-gram with hash f into its table: into the
// first slot of the probe sequence that is empty or holds the fingerprint.
__device__ void insert_gram(u64 *tab, int64_t cap, uint32_t fp_mask, int64_t e, u64 f)
{
    const uint32_t fp = (uint32_t)(f >> 32) & fp_mask;
    const u64 word = ((u64)fp << 32) | (uint32_t)(e + 1);
    int64_t slot = (int64_t)(f & (u64)(cap - 1));
    for (int64_t probe = 0; probe < cap; ++probe) {
        // claim an empty slot; a failed claim returns what the slot holds
        u64 cur = 0;
        if (__hip_atomic_compare_exchange_strong(tab + slot, &cur, word, __ATOMIC_RELAXED,
                                                 __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT))
            return;
        if ((uint32_t)(cur >> 32) == fp) {
            __hip_atomic_fetch_max(tab + slot, word, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
            return;
        }
        slot = (slot + 1) & (cap - 1);
    }
}

// Inserts the (end, length) pairs p0, p0 + step, ... of one append:
// pairs are numbered end-major over ends e_first..new_len-2 and lengths
// n_lo..n_hi, so the threads of a workgroup take neighbouring lengths of the
// same ends and every pair costs one hash of n tokens and one probe sequence.
// The tokens are read through `tok(q)` (LDS or memory).
template <typename Tok>
__device__ __forceinline__ void insert_pairs(const IndexArgs &a, int b, const AppendView &v,
                                             int64_t new_len, int64_t p0, int64_t step,
                                             const Tok &tok)
{
    const int64_t e_first = v.old_len > 0 ? v.old_len - 1 : 0;
    if (new_len - 2 < e_first)
        return;
    const int nl = a.n_hi - a.n_lo + 1;
    const int64_t pairs = (new_len - 2 - e_first + 1) * nl;
    for (int64_t p = p0; p < pairs; p += step) {
        const int64_t e = e_first + p / nl;
        const int n = a.n_lo + (int)(p % nl);
        if (e - n + 1 < 0)
            continue;
        u64 h = kHashSeed;
        for (int i = 0; i < n; ++i)
            h = hstep(h, tok(e - i));
        insert_gram(table_of(a, b, n), a.cap, a.fp_mask, e, hfinal(h));
    }
}

struct MemTok {
    const AppendView *v;
    __device__ __forceinline__ int32_t operator()(int64_t q) const { return v->at(q); }
};

// Tokens q0 .. q0 + n - 1 of the request staged in LDS.
struct LdsTok {
    const int32_t *w;
    int64_t q0;
    __device__ __forceinline__ int32_t operator()(int64_t q) const { return w[q - q0]; }
};

// The checks pld_append_kernel makes, in the same words.
__device__ __forceinline__ bool append_ok(const IndexArgs &a, int32_t old_len, int32_t c)
{
    return c >= 0 && old_len >= 0 && (int64_t)old_len + c <= a.max_len;
}

// Inserts of an append spread over several workgroups per request (large
// appends); pld_append_kernel copies the tokens afterwards.
__global__ __launch_bounds__(256) void pld_index_insert(IndexArgs a, const int32_t *tokens,
                                                        int64_t tokens_stride,
                                                        const int32_t *counts)
{
    const int b = blockIdx.x;
    const int32_t old_len = a.lengths[b];
    const int32_t c = counts[b];
    if (c <= 0 || !append_ok(a, old_len, c))
        return;  // nothing to insert, or the copy kernel rejects the append
    AppendView v{a.store + (int64_t)b * a.pitch, tokens + (int64_t)b * tokens_stride, old_len};
    insert_pairs(a, b, v, (int64_t)old_len + c,
                 (int64_t)blockIdx.y * blockDim.x + threadIdx.x, (int64_t)gridDim.y * blockDim.x,
                 MemTok{&v});
}

// A whole append of one request in one workgroup (small appends, as in a
// decode loop): inserts, copy, then the new length. The inserts read new
// tokens from the source row, so they do not depend on the copy.
__global__ __launch_bounds__(256) void pld_append_indexed(IndexArgs a, const int32_t *tokens,
                                                          int64_t tokens_stride,
                                                          const int32_t *counts)
{
    __shared__ int s_ok;
    __shared__ int32_t win[kAppendWindow];
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
    const int64_t new_len = (int64_t)old_len + c;
    // the tokens the new n-grams span: from n_hi - 1 before the first new
    // end to the last new end
    const int64_t e_first = old_len > 0 ? old_len - 1 : 0;
    const int64_t q0 = e_first - (a.n_hi - 1) > 0 ? e_first - (a.n_hi - 1) : 0;
    const int64_t nw = new_len - 1 - q0;
    if (nw <= kAppendWindow) {
        for (int64_t i = threadIdx.x; i < nw; i += blockDim.x)
            win[i] = v.at(q0 + i);
        __syncthreads();
        insert_pairs(a, b, v, new_len, threadIdx.x, blockDim.x, LdsTok{win, q0});
    } else {
        insert_pairs(a, b, v, new_len, threadIdx.x, blockDim.x, MemTok{&v});
    }
    for (int32_t t = threadIdx.x; t < c; t += blockDim.x)
        row[old_len + t] = src[t];
    __syncthreads();
    if (threadIdx.x == 0)
        a.lengths[b] = old_len + c;
}

// Walks the probe sequence of hash f in the table of one length: the end
// stored in the first slot that holds the fingerprint, or -1 when an empty
// slot comes first (the n-gram was never inserted). COHERENT reads the
// slots with agent-scope atomic loads (after this kernel's own inserts).
template <bool COHERENT>
__device__ __forceinline__ int64_t probe_fp(const u64 *tab, int64_t cap, uint32_t fp_mask, u64 f)
{
    const uint32_t fp = (uint32_t)(f >> 32) & fp_mask;
    int64_t slot = (int64_t)(f & (u64)(cap - 1));
    for (int64_t probe = 0; probe < cap; ++probe) {
        const u64 cur = COHERENT ? __hip_atomic_load(tab + slot, __ATOMIC_RELAXED,
                                                     __HIP_MEMORY_SCOPE_AGENT)
                                 : tab[slot];
        if (cur == 0)
            break;
        if ((uint32_t)(cur >> 32) == fp)
            return (int64_t)(uint32_t)cur - 1;
        slot = (slot + 1) & (cap - 1);
    }
    return -1;
}

__device__ __forceinline__ u64 wave_max(u64 key)
{
    for (int off = 32; off >= 1; off >>= 1) {
        const u64 o = __shfl_xor(key, off);
        key = o > key ? o : key;
    }
    return key;
}

struct RowTok {
    const int32_t *row;
    __device__ __forceinline__ int32_t operator()(int64_t q) const { return row[q]; }
};

// The exact answer by a scan of the history (only after a fingerprint
// collision): the maximum over end positions e <= L - 2 of
// (l(e) << 32 | e), l(e) the backward agreement with the suffix capped at
// mhat, counted when l(e) >= n_min.
template <typename Tok>
__device__ u64 scan_row(const Tok &tok_at, int32_t L, int32_t mhat, int32_t n_min,
                        const int32_t *suf, int lane)
{
    u64 best = 0;
    for (int64_t e = lane; e <= (int64_t)L - 2; e += kWave) {
        int32_t l = 0;
        while (l < mhat && e - l >= 0 && tok_at(e - l) == suf[l])
            ++l;
        if (l >= n_min) {
            const u64 k = ((u64)(uint32_t)l << 32) | (uint32_t)e;
            best = k > best ? k : best;
        }
    }
    return wave_max(best);
}

// The draft of request b (history of length L read through tok_at) from the
// index, written to the outputs by one wavefront: lane i holds suffix token
// L - 1 - i, lane n - 1 probes the table of length n. The longest length
// whose suffix n-gram is in the index is confirmed against the history in
// the same round trip that loads its draft tokens. `suf` is 64 ints of LDS.
template <bool COHERENT, typename Tok>
__device__ void index_query(const IndexArgs &a, int b, int lane, int32_t L, const Tok &tok_at,
                            int32_t n_min, int32_t n_max, int32_t k_max, int32_t *out_draft,
                            int32_t *out_len, int32_t *out_match, int32_t *out_pos, int32_t *suf)
{
    const int32_t mhat = L - 1 < n_max ? L - 1 : n_max;
    const int32_t tok = lane < mhat ? tok_at(L - 1 - lane) : 0;
    // hash of the suffix n-gram for n = lane + 1, built token by token
    u64 h = kHashSeed, mine = 0;
    for (int i = 0; i < mhat; ++i) {
        h = hstep(h, __builtin_amdgcn_readlane(tok, i));
        if (lane == i)
            mine = h;
    }
    const int n = lane + 1;
    int64_t q = -1;
    if (n >= n_min && n <= mhat)
        q = probe_fp<COHERENT>(table_of(a, b, n), a.cap, a.fp_mask, hfinal(mine));
    u64 key = wave_max(q >= 0 ? ((u64)(uint32_t)n << 32) | (uint32_t)q : 0);

    int32_t m = 0, d = 0, e = -1;
    if (key != 0) {
        m = (int32_t)(key >> 32);
        e = (int32_t)(key & 0xffffffffu);
        const int32_t follow = L - 1 - e;
        d = follow < k_max ? follow : k_max;
    }
    // confirm the end (lane i < m: token e - i) and load the draft tokens
    // (lane t < d) in one round trip
    const bool in_range = key != 0 && e <= L - 2 && e - m + 1 >= 0;
    const bool agree = !(in_range && lane < m) || tok_at(e - lane) == tok;
    int32_t cont = in_range && lane < d ? tok_at((int64_t)e + 1 + lane) : -1;
    if (key != 0 && !(in_range && __all(agree))) {
        // two n-grams share a fingerprint: answer by scanning the history
        suf[lane] = tok;
        __builtin_amdgcn_wave_barrier();
        key = scan_row(tok_at, L, mhat, n_min, suf, lane);
        m = 0, d = 0, e = -1;
        if (key != 0) {
            m = (int32_t)(key >> 32);
            e = (int32_t)(key & 0xffffffffu);
            const int32_t follow = L - 1 - e;
            d = follow < k_max ? follow : k_max;
        }
        cont = lane < d ? tok_at((int64_t)e + 1 + lane) : -1;
    }
    int32_t *orow = out_draft + (int64_t)b * k_max;
    if (lane < k_max)
        orow[lane] = cont;
    for (int t = lane + kWave; t < k_max; t += kWave)
        orow[t] = t < d ? tok_at((int64_t)e + 1 + t) : -1;
    if (lane == 0) {
        out_len[b] = d;
        out_match[b] = m;
        if (out_pos)
            out_pos[b] = key != 0 ? e - m + 1 : -1;
    }
}

// pld_draft_store: one wavefront per request, history from the store.
__global__ __launch_bounds__(kWave) void pld_index_draft(IndexArgs a, int32_t n_min, int32_t n_max,
                                                         int32_t k_max, int32_t *out_draft,
                                                         int32_t *out_len, int32_t *out_match,
                                                         int32_t *out_pos)
{
    __shared__ int32_t suf[kWave];
    const int b = blockIdx.x;
    const int lane = threadIdx.x;
    const int32_t len = a.lengths[b];
    const int32_t L = len >= 0 && len <= a.max_len ? len : 0;
    if (lane == 0 && L != len)
        atomicOr(a.err, len < 0 ? kErrLenNegative : kErrLenCapacity);
    index_query<false>(a, b, lane, L, RowTok{a.store + (int64_t)b * a.pitch}, n_min, n_max, k_max,
                       out_draft, out_len, out_match, out_pos, suf);
}

// pld_append_draft_store on an indexed context, one workgroup per request.
// The draft of the new history needs, per length n, the most recent end of
// the suffix n-gram among the ends the append adds (old L - 1 .. new L - 2)
// and among the older ones. The first wavefront finds the newer ones
// exactly by comparing the suffix with the append's LDS window, and probes
// the tables for the older ones as soon as the suffix is known, while the
// other three wavefronts insert the append's n-grams (a probe that meets a
// slot claimed meanwhile sees a valid table state: slots only fill). Per
// length the newer end wins when there is one; of the longest length found,
// an end that came from a table is confirmed against the history (with the
// draft tokens in the same round trip), and one that does not confirm
// sends the request to an exact scan. Then the copy and the new length.
constexpr int kAppendThreads = 256;

__global__ __launch_bounds__(kAppendThreads) void pld_append_draft_indexed(
    IndexArgs a, const int32_t *tokens, int64_t tokens_stride, const int32_t *counts,
    int32_t n_min, int32_t n_max, int32_t k_max, int32_t *out_draft, int32_t *out_len,
    int32_t *out_match, int32_t *out_pos)
{
    __shared__ int32_t win[kAppendWindow];
    __shared__ int32_t suf[kWave];
    const int b = blockIdx.x;
    const int tid = threadIdx.x;
    const int32_t old_len = a.lengths[b];
    const int32_t c = counts[b];
    const bool ok = append_ok(a, old_len, c);
    if (tid == 0 && !ok)
        atomicOr(a.err, c < 0 ? kErrAppendNegative : kErrAppendCapacity);
    // a rejected append leaves the history as it was; it is still drafted
    const int32_t base_len = old_len >= 0 && old_len <= a.max_len ? old_len : 0;
    const int32_t add = ok ? c : 0;
    int32_t *row = a.store + (int64_t)b * a.pitch;
    const int32_t *src = tokens + (int64_t)b * tokens_stride;
    const AppendView v{row, src, base_len};
    const int64_t new_len = (int64_t)base_len + add;
    const int32_t L = (int32_t)new_len;
    const int64_t e_first = base_len > 0 ? base_len - 1 : 0;  // first new end
    const int64_t q0 = e_first - (a.n_hi - 1) > 0 ? e_first - (a.n_hi - 1) : 0;
    const int64_t nw = new_len - 1 - q0;                       // window tokens
    const bool in_lds = add > 0 && nw <= kAppendWindow;

    // first wavefront: suffix, hashes and table probes
    const int lane = tid & (kWave - 1);
    const int32_t mhat = L - 1 < n_max ? L - 1 : n_max;
    const int n = lane + 1;
    const bool active = n >= n_min && n <= mhat;
    int32_t tok = 0;
    u64 f = 0;
    int64_t q_tab = -1;
    if (tid < kWave) {
        tok = lane < mhat ? v.at(L - 1 - lane) : 0;
        u64 h = kHashSeed, mine = 0;
        for (int i = 0; i < mhat; ++i) {
            h = hstep(h, __builtin_amdgcn_readlane(tok, i));
            if (lane == i)
                mine = h;
        }
        f = hfinal(mine);
        if (active)
            q_tab = probe_fp<true>(table_of(a, b, n), a.cap, a.fp_mask, f);
        suf[lane] = tok;
    }
    // every thread stages the window
    if (in_lds)
        for (int64_t i = tid; i < nw; i += kAppendThreads)
            win[i] = v.at(q0 + i);
    __syncthreads();
    if (tid >= kWave) {
        // the other wavefronts insert the append's n-grams
        if (add > 0) {
            if (in_lds)
                insert_pairs(a, b, v, new_len, tid - kWave, kAppendThreads - kWave,
                             LdsTok{win, q0});
            else
                insert_pairs(a, b, v, new_len, tid - kWave, kAppendThreads - kWave, MemTok{&v});
        }
        for (int32_t t = tid - kWave; t < add; t += kAppendThreads - kWave)
            row[base_len + t] = src[t];
        return;
    }

    // the newest end among the append's ends whose n tokens are the suffix
    // n-gram (exact, from the window or the view)
    int64_t q_new = -1;
    if (active && add > 0) {
        for (int64_t e = new_len - 2; e >= e_first && q_new < 0; --e) {
            if (e - n + 1 < 0)
                break;
            bool same = true;
            for (int i = 0; same && i < n; ++i)
                same = (in_lds ? win[e - i - q0] : v.at(e - i)) == suf[i];
            if (same)
                q_new = e;
        }
    }
    const bool from_table = q_new < 0;
    const int64_t q = from_table ? q_tab : q_new;
    u64 key = wave_max(active && q >= 0 ? ((u64)(uint32_t)n << 32) | (uint32_t)q : 0);
    int32_t m = 0, d = 0, e = -1;
    if (key != 0) {
        m = (int32_t)(key >> 32);
        e = (int32_t)(key & 0xffffffffu);
        const int32_t follow = L - 1 - e;
        d = follow < k_max ? follow : k_max;
    }
    // an end from a table is confirmed with the draft tokens' round trip
    const bool check = key != 0 && __builtin_amdgcn_readlane((int)from_table, m - 1) != 0;
    const bool in_range = key != 0 && e <= L - 2 && e - m + 1 >= 0;
    const bool agree = !(check && in_range && lane < m) || v.at(e - lane) == tok;
    int32_t cont = in_range && lane < d ? v.at((int64_t)e + 1 + lane) : -1;
    if (check && !(in_range && __all(agree))) {
        // two n-grams share a fingerprint: answer by scanning the history
        key = scan_row(MemTok{&v}, L, mhat, n_min, suf, lane);
        m = 0, d = 0, e = -1;
        if (key != 0) {
            m = (int32_t)(key >> 32);
            e = (int32_t)(key & 0xffffffffu);
            const int32_t follow = L - 1 - e;
            d = follow < k_max ? follow : k_max;
        }
        cont = lane < d ? v.at((int64_t)e + 1 + lane) : -1;
    }
    int32_t *orow = out_draft + (int64_t)b * k_max;
    if (lane < k_max)
        orow[lane] = cont;
    for (int t = lane + kWave; t < k_max; t += kWave)
        orow[t] = t < d ? v.at((int64_t)e + 1 + t) : -1;
    if (lane == 0) {
        out_len[b] = d;
        out_match[b] = m;
        if (out_pos)
            out_pos[b] = key != 0 ? e - m + 1 : -1;
        // every thread read the old length before the barrier
        if (add > 0)
            a.lengths[b] = L;
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

hipError_t launch_append_indexed(const IndexArgs &a, const int32_t *tokens,
                                 int64_t tokens_stride, const int32_t *counts, int32_t batch,
                                 hipStream_t s)
{
    if (batch <= 0)
        return hipSuccess;
    hipLaunchKernelGGL(pld_append_indexed, dim3((unsigned)batch), dim3(256), 0, s, a, tokens,
                       tokens_stride, counts);
    return hipGetLastError();
}

hipError_t launch_append_draft_indexed(const IndexArgs &a, const int32_t *tokens,
                                       int64_t tokens_stride, const int32_t *counts,
                                       int32_t batch, int32_t n_min, int32_t n_max,
                                       int32_t k_max, int32_t *out_draft, int32_t *out_len,
                                       int32_t *out_match, int32_t *out_pos, hipStream_t s)
{
    if (batch <= 0)
        return hipSuccess;
    hipLaunchKernelGGL(pld_append_draft_indexed, dim3((unsigned)batch), dim3(256), 0, s, a, tokens,
                       tokens_stride, counts, n_min, n_max, k_max, out_draft, out_len, out_match,
                       out_pos);
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
