// HIP kernels for batched prompt-lookup drafting on gfx950 (MI355X).
//
// The operation (HyperQwen lookup-drafting page, step 1 of the three-step
// principle): per request, the most recent earlier occurrence of the longest
// n_min..n_max-token suffix of its own history, overlap allowed; the tokens
// after it are the draft.
//
// How the search is laid out here. For an end position e in [0, L-2] let
// l(e) be the number of tokens, capped at m = min(n_max, L-1), for which the
// history read backwards from e agrees with the history read backwards from
// L-1. Any occurrence of the length-l suffix ending at e is one of length l-1
// ending at e too (dropping its first token keeps it admissible), so the
// longest suffix with an occurrence is max_e l(e), and among end positions
// with that l the largest e is the most recent start j = e - l + 1. Packing
// key(e) = l(e) << 32 | e (0 when l(e) < n_min) makes the answer the plain
// unsigned maximum of key(e) over all e. A maximum can be taken in any order,
// so the positions are split into tiles, one workgroup each, and the partial
// maxima are merged with a 64-bit atomicMax; the result does not depend on
// the tiling or on the order workgroups run in.
//
// pld_scan (one workgroup per tile of TILE candidate end positions):
//   1. Coalesced 16-byte loads bring the tile, plus HALO tokens to its left,
//      into registers; rows that are not 16-byte aligned are handled by
//      addressing aligned 16-byte chunks and shifting by the misalignment.
//   2. First-token rejection in registers: only positions holding the
//      history's last token survive (about 2-3% on Zipf text).
//   3. The registers are staged into LDS; survivors extend backwards from
//      LDS against the suffix (also in LDS) up to m tokens.
//   4. Per-thread max -> wavefront max (cross-lane shuffles on 2x32-bit) ->
//      workgroup max (LDS) -> 64-bit atomicMax into the request's slot when
//      the request spans more than one tile.
//   5. Fused gather: the last workgroup of a request to arrive (an agent-scope
//      acquire-release counter) decodes the key, writes the draft row, and
//      clears the request's slot and counter for the next call.
// pld_gather is the same step 5 as its own kernel, for the unfused mode.

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "pld_kernels.h"

namespace pld {

namespace {

constexpr int kHalo = 64;                 // >= PLD_N_MAX_LIMIT - 1, multiple of 4
constexpr int kHaloChunks = kHalo / 4;    // 16-byte chunks of halo
constexpr int kWave = 64;

typedef unsigned long long u64;

__device__ __forceinline__ u64 wave_max_u64(u64 v)
{
#pragma unroll
    for (int off = kWave / 2; off > 0; off >>= 1) {
        const u64 o = __shfl_xor(v, off, kWave);
        v = o > v ? o : v;
    }
    return v;
}

// Loads through the global address space (global_load_* rather than
// flat_load_*): every pointer the kernels read through is device memory.
template <typename T>
__device__ __forceinline__ T gld(const T *p)
{
    typedef __attribute__((address_space(1))) const T gT;
    return *(gT *)p;
}

typedef int32_t v4i32 __attribute__((ext_vector_type(4)));

__device__ __forceinline__ int4 gld(const int4 *p)
{
    typedef __attribute__((address_space(1))) const v4i32 gV;
    const v4i32 x = *(gV *)p;
    return make_int4(x[0], x[1], x[2], x[3]);
}

__device__ __forceinline__ int32_t comp(const int4 &v, int i)
{
    return i == 0 ? v.x : i == 1 ? v.y : i == 2 ? v.z : v.w;
}

// Per-request facts every kernel derives the same way from lengths/rows.
struct Req {
    const int32_t *h;
    int32_t L;      // usable length (0 when the request is invalid)
    int32_t ncand;  // candidate end positions: L - 1 (or 0)
    int32_t ntiles; // tiles that hold candidates (at least 1)
    uint32_t err;   // error bits for this request
};

__device__ __forceinline__ Req load_req(const DraftArgs &a, int b, int tile_tokens)
{
    Req r;
    const int32_t len = a.lengths[b];
    const int32_t *h = a.histories[b];
    r.err = 0;
    if (len < 0)
        r.err |= kErrLenNegative;
    else if (len > a.max_len)
        r.err |= kErrLenCapacity;
    else if (len > 0 && (h == nullptr || ((uintptr_t)h & 3u)))
        r.err |= kErrBadRow;
    r.h = h;
    r.L = r.err ? 0 : len;
    r.ncand = r.L > 0 ? r.L - 1 : 0;
    r.ntiles = r.ncand > 0 ? (int32_t)((r.ncand + (int64_t)tile_tokens - 1) / tile_tokens) : 1;
    return r;
}

// Writes row b of the outputs from a packed key (0 = no match). Called by
// all threads of a workgroup (threads stride over the k_max slots).
__device__ __forceinline__ void emit(const DraftArgs &a, int b, const Req &r,
                                     u64 key, int tid, int nthreads)
{
    int32_t m = 0, d = 0, e = -1;
    if (key != 0) {
        m = (int32_t)(key >> 32);
        e = (int32_t)(key & 0xffffffffu);
        const int32_t follow = r.L - 1 - e;
        d = follow < a.k_max ? follow : a.k_max;
    }
    int32_t *row = a.out_draft + (int64_t)b * a.k_max;
    const int32_t *src = r.h + (int64_t)e + 1;
    for (int t = tid; t < a.k_max; t += nthreads)
        row[t] = t < d ? gld(src + t) : -1;
    if (tid == 0) {
        a.out_len[b] = d;
        a.out_match[b] = m;
        if (a.out_pos)
            a.out_pos[b] = key != 0 ? e - m + 1 : -1;
    }
}

// A 16-byte chunk covering positions p0 .. p0+3 is loaded whole when all
// four positions lie in [0, L). Chunks at the row's edges (p0 < 0 or past
// the end) are first loaded from a 16-byte zero block owned by the context,
// so every thread issues its loads back to back with no branch in between,
// and then patched token by token from the row (only in-range tokens are
// read; the others are never compared).
__device__ __forceinline__ bool chunk_inside(int64_t p0, int32_t L)
{
    return p0 >= 0 && p0 + 3 < (int64_t)L;
}

__device__ __forceinline__ int4 patch_chunk(int4 v, int64_t p0, const int32_t *h, int32_t L)
{
    if (p0 + 0 >= 0 && p0 + 0 < L) v.x = gld(h + p0 + 0);
    if (p0 + 1 >= 0 && p0 + 1 < L) v.y = gld(h + p0 + 1);
    if (p0 + 2 >= 0 && p0 + 2 < L) v.z = gld(h + p0 + 2);
    if (p0 + 3 >= 0 && p0 + 3 < L) v.w = gld(h + p0 + 3);
    return v;
}

template <int TILE, int THREADS>
__global__ __launch_bounds__(THREADS) void pld_scan(DraftArgs a)
{
    static_assert(TILE % (4 * THREADS) == 0, "tile must be whole chunks per thread");
    static_assert(THREADS >= kHaloChunks + 1, "halo needs 17 loader threads");
    constexpr int kBody = TILE / 4;            // chunks in the tile body
    constexpr int kPer = kBody / THREADS;      // body chunks per thread
    constexpr int kWin = kHaloChunks + kBody + 1;
    constexpr int kWaves = THREADS / kWave;
    static_assert(4 * (kPer + 1) <= 64, "candidate mask is 64 bits");

    __shared__ int4 win[kWin];
    __shared__ int32_t pat[PLD_N_MAX_LIMIT];
    __shared__ u64 wave_best[kWaves];
    __shared__ int s_last;

    const int tid = threadIdx.x;
    const int tile = blockIdx.x / a.batch;
    const int b = blockIdx.x - tile * a.batch;

    const Req r = load_req(a, b, TILE);
    if (tile >= r.ntiles)
        return;  // this request has no candidates in this tile
    if (r.err && tid == 0)
        atomicOr(a.err, r.err);

    const int32_t mhat = r.L - 1 < a.n_max ? r.L - 1 : a.n_max;
    u64 best = 0;

    if (mhat >= a.n_min) {
        const int64_t t0 = (int64_t)tile * TILE;
        const int32_t nrel = (int32_t)(((int64_t)r.ncand - t0) < TILE ? (r.ncand - t0) : TILE);
        const int32_t last = gld(r.h + r.L - 1);
        const int delta = (int)(((uintptr_t)r.h >> 2) & 3u);
        const int4 *arow = (const int4 *)(r.h - delta);
        const int64_t gc0 = (t0 - kHalo) / 4;  // exact: t0 and kHalo are multiples of 4
        const int64_t p_base = t0 - kHalo - delta;  // position of window token 0

        // 1. loads: kPer body chunks, plus one halo/spill chunk for 17 threads
        // window chunk of body slot k is kHaloChunks + k * THREADS + tid; the
        // extra slot kPer is a halo chunk (tid < 16), the spill chunk past
        // the body (tid == 16, used when the row is not 16-byte aligned) or
        // nothing (wx < 0).
        const int wx = tid < kHaloChunks ? tid : (tid == kHaloChunks ? kHaloChunks + kBody : -1);
        int4 v[kPer + 1];
        bool inside[kPer + 1];
#pragma unroll
        for (int k = 0; k <= kPer; ++k) {
            const int wk = k < kPer ? kHaloChunks + k * THREADS + tid : wx;
            inside[k] = wk >= 0 && chunk_inside(p_base + 4 * wk, r.L);
            const int4 *src = inside[k] ? arow + (gc0 + wk) : a.zero16;
            v[k] = gld(src);
        }
        if (tid < mhat)
            pat[tid] = gld(r.h + r.L - mhat + tid);
#pragma unroll
        for (int k = 0; k <= kPer; ++k) {
            const int wk = k < kPer ? kHaloChunks + k * THREADS + tid : wx;
            if (wk >= 0 && !inside[k])
                v[k] = patch_chunk(v[k], p_base + 4 * wk, r.h, r.L);
        }

        // 2. first-token rejection on registers. rel = position - t0.
        u64 cand = 0;
#pragma unroll
        for (int k = 0; k <= kPer; ++k) {
            const int wk = k < kPer ? kHaloChunks + k * THREADS + tid : wx;
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                const int32_t rel = 4 * wk + i - kHalo - delta;
                const bool hit = wk >= 0 && rel >= 0 && rel < nrel && comp(v[k], i) == last;
                cand |= (u64)hit << (4 * k + i);
            }
        }

        // 3. stage in LDS, then extend the survivors backwards.
#pragma unroll
        for (int k = 0; k < kPer; ++k)
            win[kHaloChunks + k * THREADS + tid] = v[k];
        if (wx >= 0)
            win[wx] = v[kPer];
        __syncthreads();

        const int32_t *wt = (const int32_t *)win;
        const int32_t floor_rel = t0 < kHalo ? -(int32_t)t0 : -kHalo;  // rel of position 0 (or the halo start)
        while (cand) {
            const int bit = __builtin_ctzll(cand);
            cand &= cand - 1;
            const int k = bit >> 2, i = bit & 3;
            const int wk = k < kPer ? kHaloChunks + k * THREADS + tid : wx;
            const int32_t slot = 4 * wk + i;
            const int32_t rel = slot - kHalo - delta;
            int32_t ell = 1;
            while (ell < mhat && rel - ell >= floor_rel && wt[slot - ell] == pat[mhat - 1 - ell])
                ++ell;
            if (ell >= a.n_min) {
                const u64 key = ((u64)(uint32_t)ell << 32) | (uint32_t)(t0 + rel);
                best = key > best ? key : best;
            }
        }
    }

    // 4. thread -> wavefront -> workgroup maximum.
    if (__any(best != 0))
        best = wave_max_u64(best);
    if ((tid & (kWave - 1)) == 0)
        wave_best[tid / kWave] = best;
    __syncthreads();

    if (tid == 0) {
        u64 m = 0;
#pragma unroll
        for (int i = 0; i < kWaves; ++i)
            m = wave_best[i] > m ? wave_best[i] : m;
        int last_one = 1;
        if (r.ntiles > 1) {
            if (m)
                __hip_atomic_fetch_max(&a.keys[b], m, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
            if (a.fused) {
                const unsigned prev = __hip_atomic_fetch_add(&a.arrivals[b], 1u, __ATOMIC_ACQ_REL,
                                                             __HIP_MEMORY_SCOPE_AGENT);
                last_one = prev == (unsigned)(r.ntiles - 1);
                if (last_one) {
                    m = __hip_atomic_load(&a.keys[b], __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
                    __hip_atomic_store(&a.keys[b], 0ull, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
                    __hip_atomic_store(&a.arrivals[b], 0u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
                }
            }
        } else if (!a.fused && m) {
            // single-tile request in unfused mode: hand the key to pld_gather
            __hip_atomic_store(&a.keys[b], m, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        }
        wave_best[0] = m;
        s_last = a.fused && last_one;
    }
    __syncthreads();

    // 5. fused gather by the last workgroup of the request.
    if (s_last)
        emit(a, b, r, wave_best[0], tid, THREADS);
}

__global__ __launch_bounds__(kWave) void pld_gather(DraftArgs a)
{
    const int b = blockIdx.x;
    const Req r = load_req(a, b, 1);
    const u64 key = a.keys[b];
    emit(a, b, r, r.err ? 0ull : key, threadIdx.x, kWave);
    __syncthreads();
    if (threadIdx.x == 0 && key != 0)
        a.keys[b] = 0;
}

// One workgroup per request: append counts[b] tokens to store row b.
__global__ __launch_bounds__(256) void pld_append_kernel(AppendArgs a)
{
    __shared__ int32_t s_len;
    __shared__ int s_ok;
    const int b = blockIdx.x;
    if (threadIdx.x == 0) {
        const int32_t len = a.lengths[b];
        const int32_t c = a.counts[b];
        int ok = 1;
        if (c < 0) {
            atomicOr(a.err, kErrAppendNegative);
            ok = 0;
        } else if ((int64_t)len + c > a.max_len) {
            atomicOr(a.err, kErrAppendCapacity);
            ok = 0;
        }
        s_len = len;
        s_ok = ok;
    }
    __syncthreads();
    if (!s_ok)
        return;
    const int32_t len = s_len;
    const int32_t c = a.counts[b];
    const int32_t *src = a.tokens + (int64_t)b * a.tokens_stride;
    int32_t *dst = a.store + (int64_t)b * a.pitch + len;
    for (int32_t t = threadIdx.x; t < c; t += blockDim.x)
        dst[t] = src[t];
    __syncthreads();
    if (threadIdx.x == 0)
        a.lengths[b] = len + c;
}

__global__ __launch_bounds__(256) void pld_fill_i32(int32_t *p, int64_t n, int32_t value)
{
    const int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
    if (i < n)
        p[i] = value;
}

template <int TILE, int THREADS>
hipError_t launch_scan(const DraftArgs &a, int64_t tiles_per_req, hipStream_t s)
{
    const int64_t grid = tiles_per_req * a.batch;
    hipLaunchKernelGGL((pld_scan<TILE, THREADS>), dim3((unsigned)grid), dim3(THREADS), 0, s, a);
    return hipGetLastError();
}

}  // namespace

hipError_t launch_draft(const DraftArgs &a, int tile_tokens, hipStream_t s)
{
    const int64_t tiles = a.max_len > 1 ? ((int64_t)a.max_len - 1 + tile_tokens - 1) / tile_tokens : 1;
    hipError_t e;
    switch (tile_tokens) {
    case 256: e = launch_scan<256, 64>(a, tiles, s); break;
    case 1024: e = launch_scan<1024, 256>(a, tiles, s); break;
    case 2048: e = launch_scan<2048, 256>(a, tiles, s); break;
    case 4096: e = launch_scan<4096, 256>(a, tiles, s); break;
    case 8192: e = launch_scan<8192, 256>(a, tiles, s); break;
    default: return hipErrorInvalidValue;
    }
    if (e != hipSuccess || a.fused)
        return e;
    hipLaunchKernelGGL(pld_gather, dim3((unsigned)a.batch), dim3(kWave), 0, s, a);
    return hipGetLastError();
}

int64_t scan_grid(int32_t max_len, int32_t batch, int tile_tokens)
{
    const int64_t tiles = max_len > 1 ? ((int64_t)max_len - 1 + tile_tokens - 1) / tile_tokens : 1;
    return tiles * batch;
}

hipError_t launch_append(const AppendArgs &a, int32_t batch, hipStream_t s)
{
    hipLaunchKernelGGL(pld_append_kernel, dim3((unsigned)batch), dim3(256), 0, s, a);
    return hipGetLastError();
}

hipError_t launch_fill(int32_t *p, int64_t n, int32_t value, hipStream_t s)
{
    if (n <= 0)
        return hipSuccess;
    const int64_t blocks = (n + 255) / 256;
    hipLaunchKernelGGL(pld_fill_i32, dim3((unsigned)blocks), dim3(256), 0, s, p, n, value);
    return hipGetLastError();
}

}  // namespace pld
