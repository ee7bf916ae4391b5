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
// pld_scan (one workgroup per tile of TILE candidate end positions; each
// wavefront takes a contiguous share of the tile and works on its own):
//   1. Coalesced, non-temporal 16-byte loads bring the wavefront's span plus
//      the 64 tokens to its left into registers; rows that are not 16-byte
//      aligned are read as aligned chunks shifted by the misalignment. A
//      request's last tile (unless it is also its first) loads through a
//      buffer resource whose record count ends at the row's last 16-byte
//      block, so the blocks past the row read as zeros with no branch, and
//      it runs the interior tiles' tests; its first tile range-checks every
//      chunk and position.
//   2. The registers are staged in the wavefront's own LDS region.
//   3. Rejection in registers: a position survives only if it holds the
//      history's last token (about 2-4% on Zipf text) and, when n_min >= 3,
//      its two predecessors hold the two tokens before that (the tokens
//      before a chunk come from the neighbouring lane by a DPP wavefront
//      shift; two of the three tokens are compared as one 64-bit pair);
//      survivors extend backwards from LDS up to m tokens: when a wavefront
//      has only a few, the whole wavefront extends each in one LDS round
//      trip (one token per lane, the first mismatch from a ballot);
//      otherwise each lane extends its own: 4 tokens in the first round
//      trip, 8 in each later one.
//   4. Per-thread max -> wavefront max (DPP row shifts and broadcasts on
//      2x32-bit halves) where the lanes hold different values (a value all
//      lanes share, as the wavefront-level extension leaves, needs none),
//      then either a 64-bit atomicMax into the request's slot per wavefront
//      (separate gather kernel), or the fused gather.
//   5. Fused gather: in a multi-tile request each wavefront with a match
//      merges its max with a 64-bit atomicMax as soon as its tests end; the
//      workgroup (one LDS word per wavefront, a single barrier) counts
//      itself in with an atomic add that also carries the increases its
//      wavefronts' atomicMax calls made; the increases sum to the maximum,
//      so the last workgroup to arrive has it from its own add. It writes
//      the draft row and clears the slot for the next call. Single-tile
//      requests take the workgroup max and emit directly.
// pld_gather is the same step 5 as its own kernel, for the unfused mode.

#include <hip/hip_runtime.h>
#include <stdint.h>

#include <mutex>

#include "pld_control_step.h"
#include "pld_kernels.h"

namespace pld {

namespace {

constexpr int kHalo = 64;                 // >= PLD_N_MAX_LIMIT - 1, multiple of 4
constexpr int kHaloChunks = kHalo / 4;    // 16-byte chunks of halo
constexpr int kWave = 64;
constexpr int kExtBlock = 4;             // tokens a lane compares in its first LDS round trip when extending (twice as many later)
constexpr int kWaveExt = 4;              // most survivors a wavefront extends together
constexpr unsigned kGridY = 65535;       // largest y extent of a grid

typedef unsigned long long u64;

// One step of a wavefront maximum over 64-bit keys: each lane takes the max
// of its value and the value DPP control `ctrl` routes to it (the two 32-bit
// halves move separately). Lanes left out by the row/bank masks, or whose
// source is outside the wavefront, see 0, which leaves a maximum unchanged.
template <int CTRL, int ROW_MASK, int BANK_MASK>
__device__ __forceinline__ u64 dpp_max_step(u64 v)
{
    const uint32_t lo = __builtin_amdgcn_update_dpp(0u, (uint32_t)v, CTRL, ROW_MASK, BANK_MASK, false);
    const uint32_t hi = __builtin_amdgcn_update_dpp(0u, (uint32_t)(v >> 32), CTRL, ROW_MASK, BANK_MASK, false);
    const u64 o = ((u64)hi << 32) | lo;
    return o > v ? o : v;
}

// Maximum over the wavefront, delivered in lane 63: shifts by 1, 2 and 3
// within each row of 16 lanes, then by 4 and 8 in the upper banks, then the
// row-15 and row-31 broadcasts carry the partial maxima across rows.
__device__ __forceinline__ u64 wave_max_u64(u64 v)
{
    v = dpp_max_step<0x111, 0xf, 0xf>(v);  // row_shr:1
    v = dpp_max_step<0x112, 0xf, 0xf>(v);  // row_shr:2
    v = dpp_max_step<0x113, 0xf, 0xf>(v);  // row_shr:3
    v = dpp_max_step<0x114, 0xf, 0xe>(v);  // row_shr:4, banks 1-3
    v = dpp_max_step<0x118, 0xf, 0xc>(v);  // row_shr:8, banks 2-3
    v = dpp_max_step<0x142, 0xa, 0xf>(v);  // row_bcast:15, rows 1 and 3
    v = dpp_max_step<0x143, 0xc, 0xf>(v);  // row_bcast:31, rows 2 and 3
    const uint32_t lo = __builtin_amdgcn_readlane((uint32_t)v, kWave - 1);
    const uint32_t hi = __builtin_amdgcn_readlane((uint32_t)(v >> 32), kWave - 1);
    return ((u64)hi << 32) | lo;
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


// Streaming load of history data, read once per call: marked non-temporal
// so it does not push the kernel's own code and the small shared arrays out
// of the L2.
__device__ __forceinline__ int4 gld_stream(const int4 *p)
{
    typedef __attribute__((address_space(1))) const v4i32 gV;
    const v4i32 x = __builtin_nontemporal_load((gV *)p);
    return make_int4(x[0], x[1], x[2], x[3]);
}

__device__ __forceinline__ int32_t comp(const int4 &v, int i)
{
    return i == 0 ? v.x : i == 1 ? v.y : i == 2 ? v.z : v.w;
}

// Per-request facts every kernel derives the same way from lengths/rows.
struct Req {
    const int32_t *h;
    const int32_t *src; // appended tokens: position p >= split is src[p - split]
    int32_t L;      // usable length (0 when the request is invalid)
    int32_t split;  // positions below it are read from h (L without an append)
    int32_t add;    // tokens appended in this launch (0 without an append)
    uint32_t app_err; // error bits of a rejected append (0 without an append)
    int32_t ncand;  // candidate end positions: L - 1 (or 0)
    int32_t ntiles; // tiles that hold candidates (at least 1)
    uint32_t err;   // error bits for this request
};

// The error bits of appending c tokens to a row of length len (0 when the
// append is accepted); pld_append_kernel and the appending scan agree.
__device__ __forceinline__ uint32_t append_error(int32_t len, int32_t c, int32_t max_len)
{
    if (c < 0)
        return kErrAppendNegative;
    if (len < 0 || (int64_t)len + c > max_len)
        return kErrAppendCapacity;
    return 0;
}

// The error bits of a strided row whose stored length is len: negative,
// beyond max_len or the stride, or below the caller's min_len.
__device__ __forceinline__ uint32_t strided_len_error(const DraftArgs &a, int32_t len)
{
    if (len < 0)
        return kErrLenNegative;
    if (len > a.max_len || len > a.stride)
        return kErrLenCapacity;
    if (len < a.min_len)
        return kErrBelowMinLen;
    return 0;
}

// Row b is histories[b], or base + b * stride for a strided batch (a.stride
// > 0, rows 16-byte aligned as checked on the host). With APPEND the row
// first gains the counts[b] new tokens when that append is accepted, and
// the batch is known to be strided.
template <bool APPEND = false>
__device__ __forceinline__ Req load_req(const DraftArgs &a, int b, int tile_tokens)
{
    Req r;
    const int32_t old_len = a.lengths[b];
    const bool strided = APPEND || a.stride != 0;
    const int32_t *h = strided ? a.base + (int64_t)b * a.stride : a.histories[b];
    r.add = 0;
    r.app_err = 0;
    if constexpr (APPEND) {
        const int32_t c = a.app_counts[b];
        r.app_err = append_error(old_len, c, a.max_len);
        r.add = r.app_err == 0 ? c : 0;
        r.src = a.app_tokens + (int64_t)b * a.app_stride;
    }
    const int32_t len = old_len + r.add;
    r.err = 0;
    if (strided)
        r.err = strided_len_error(a, len);
    else if (len < 0)
        r.err |= kErrLenNegative;
    else if (len > a.max_len)
        r.err |= kErrLenCapacity;
    else if (len > 0 && (h == nullptr || ((uintptr_t)h & 3u)))
        r.err |= kErrBadRow;
    r.h = h;
    r.L = r.err ? 0 : len;
    if constexpr (APPEND) {
        // an accepted append leaves a valid length, so r.err is 0 whenever r.add > 0
        r.split = r.err ? 0 : old_len;
    } else {
        r.split = r.L;
        r.src = h;
    }
    r.ncand = r.L > 0 ? r.L - 1 : 0;
    r.ntiles = r.ncand > 0 ? (int32_t)((r.ncand + (int64_t)tile_tokens - 1) / tile_tokens) : 1;
    return r;
}

// Token p of request r's history: from its row, or with APPEND from the
// source of this launch's append when p is at or past the old length (one
// load either way).
template <bool APPEND>
__device__ __forceinline__ int32_t tok_at(const Req &r, int64_t p)
{
    if constexpr (APPEND) {
        // one of two uniform byte bases, then the position's offset
        const uint64_t hb = (uint64_t)(uintptr_t)r.h;
        const uint64_t sb = (uint64_t)(uintptr_t)r.src - 4 * (uint64_t)(uint32_t)r.split;
        return gld((const int32_t *)(uintptr_t)((p < r.split ? hb : sb) + 4 * (uint64_t)p));
    } else {
        return gld(r.h + p);
    }
}

// Writes row b of the outputs from a packed key (0 = no match). Called by
// all threads of a workgroup (threads stride over the k_max slots).
template <bool APPEND = false>
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
    // the per-request outputs first: they do not wait for the continuation
    if (tid == 0) {
        a.out_len[b] = d;
        a.out_match[b] = m;
        if (a.out_pos)
            a.out_pos[b] = key != 0 ? e - m + 1 : -1;
    }
    int32_t *row = a.out_draft + (int64_t)b * a.k_max;
    const int32_t *src = r.h + (int64_t)e + 1;
    for (int t = tid; t < a.k_max; t += nthreads) {
        if constexpr (APPEND)
            row[t] = t < d ? tok_at<true>(r, (int64_t)e + 1 + t) : -1;
        else
            row[t] = t < d ? gld(src + t) : -1;
    }
}

// Draft fusion and long-block scheduling of request b by one wavefront
// (HyperQwen lookup-drafting page, steps 2 and 3); lane t owns block
// position t and holds the lookup draft's token t in `lk` (t < d). In the
// page's order: the run of near-full steps is brought up to date with the
// previous step's accepted count, the block size is chosen (entry
// condition, or the sticky hold), then the head is fused and the tail
// filled from the lookup draft.
// The inputs of a request's fusion step that do not depend on its lookup
// draft: its state row, its accepted count and lane t's drafter token. The
// scan kernel reads them before it scans, so they are at hand when the
// draft is.
struct FusePre {
    int32_t was_long, hold, streak, prev_n, acc, dr;
};

__device__ __forceinline__ FusePre fuse_preload(const FuseArgs &a, int b, int t)
{
    const int32_t *st = a.state + (int64_t)b * 4;
    FusePre p;
    p.was_long = st[0];
    p.hold = st[1];
    p.streak = st[2];
    p.prev_n = st[3];
    p.acc = a.accepted[b];
    // every lane loads (lanes past the head re-read the last head token), so
    // no load sits inside a branch
    const int32_t dr = a.drafter[(int64_t)b * a.head + (t < a.head ? t : a.head - 1)];
    p.dr = t < a.head ? dr : -1;
    return p;
}

__device__ __forceinline__ void fuse_request(const FuseArgs &a, int b, int t, int32_t d,
                                             int32_t m, int32_t lk, const FusePre &pre)
{
    int32_t *st = a.state + (int64_t)b * 4;
    const int32_t was_long = pre.was_long;
    int32_t hold = pre.hold;
    int32_t streak = pre.streak;
    const int32_t prev_n = pre.prev_n;
    const int32_t acc = pre.acc;
    const bool ok = d >= 0 && d <= a.lookup_k && m >= 0 && hold >= 0 && streak >= 0 &&
                    prev_n >= 0 && prev_n <= PLD_FUSE_MAX_POSITIONS &&
                    (prev_n == 0 || (acc >= 0 && acc <= prev_n));
    const int32_t dr = pre.dr;

    int32_t n = a.head;
    int32_t is_long = 0;
    bool from_lookup = false;
    if (ok) {
        // step 3: near-full run, entry condition, sticky hold
        if (prev_n > 0) {
            // only "at least entry_steps" matters, so the run is capped there
            const bool near_full = acc >= prev_n - a.near_full_slack;
            const int32_t run = streak < a.entry_steps ? streak + 1 : a.entry_steps;
            streak = near_full ? run : 0;
        }
        const bool fills_tail = m >= a.tail_min && d >= a.positions_long;
        if (fills_tail && streak >= a.entry_steps) {
            is_long = 1;
            hold = a.sticky;
        } else if (was_long != 0 && hold > 0) {
            is_long = 1;
            hold -= 1;
        } else {
            hold = 0;
        }
        // step 2: the head, replaced outright or on agreement of the first
        // agree_tokens tokens (each of which the lookup draft must have)
        const u64 agree_mask = a.agree_tokens >= kWave ? ~0ull : (1ull << a.agree_tokens) - 1;
        const u64 eq = __ballot(t < a.agree_tokens && t < d && dr == lk);
        const bool agree = (eq & agree_mask) == agree_mask;
        const bool replace = m >= a.replace_min || (m >= a.agree_min && agree);
        if (is_long && m >= a.tail_min) {
            const int32_t cover = d < a.positions_long ? d : a.positions_long;
            n = cover > a.head ? cover : a.head;
        }
        from_lookup = t < a.head ? (replace && t < d) : t < n;
    } else {
        streak = 0;
        hold = 0;
    }
    const u64 src = __ballot(from_lookup);
    if (t < a.positions_long)
        a.out_block[(int64_t)b * a.positions_long + t] = t >= n ? -1 : (from_lookup ? lk : dr);
    if (t == 0) {
        a.out_positions[b] = n;
        if (a.out_src)
            a.out_src[b] = src;
        st[0] = is_long;
        st[1] = hold;
        st[2] = streak;
        st[3] = ok ? n : 0;
        if (!ok)
            atomicOr(a.err, kErrFuseInput);
    }
}

// Writes row b of the lookup outputs (as emit does) and fuses them with the
// drafter's proposal (fuse_request) in one wavefront: lane t holds the
// lookup draft's token t. Used instead of emit when the call also fuses.
__device__ __forceinline__ void emit_and_fuse(const DraftArgs &a, int b, const Req &r, u64 key,
                                              int lane, const FusePre &pre)
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
    const int32_t lk = lane < d ? gld(src + lane) : -1;
    if (lane < a.k_max)
        row[lane] = lk;
    for (int t = lane + kWave; t < a.k_max; t += kWave)
        row[t] = t < d ? gld(src + t) : -1;
    if (lane == 0) {
        a.out_len[b] = d;
        a.out_match[b] = m;
        if (a.out_pos)
            a.out_pos[b] = key != 0 ? e - m + 1 : -1;
    }
    fuse_request(a.fuse, b, lane, d, m, lk, pre);
}

// The inputs of a request's controller step that do not depend on its
// lookup draft, one value per lane of a wavefront: lane i < 11 holds state
// word i, every lane the round time and accepted count of the previous
// round. Every lane loads (indices clamped), so no load sits in a branch.
struct CtlPre {
    double sv, rt;
    int32_t acc;
};

__device__ __forceinline__ CtlPre control_preload(const ControlArgs &a, int b, int lane)
{
    CtlPre p;
    p.sv = a.state[(int64_t)b * kCtlWords + (lane < kCtlWords ? lane : kCtlWords - 1)];
    p.rt = a.round_time[b];
    p.acc = a.accepted[b];
    return p;
}

// The controller step of request b from its lookup draft (d tokens, match
// m), by one wavefront holding its preloaded inputs; lane 0 writes.
__device__ __forceinline__ void emit_control(const ControlArgs &a, int b, int32_t d, int32_t m,
                                             int lane, const CtlPre &pre)
{
    auto word = [&](int i) {
        const u64 w = (u64)__double_as_longlong(pre.sv);
        const u64 lo = (uint32_t)__builtin_amdgcn_readlane((int)(uint32_t)w, i);
        const u64 hi = (uint32_t)__builtin_amdgcn_readlane((int)(w >> 32), i);
        return __longlong_as_double((long long)(hi << 32 | lo));
    };
    CtlState st;
    st.acc = ctl_double4{word(kCtlAcc0), word(kCtlAcc0 + 1), word(kCtlAcc0 + 2),
                         word(kCtlAcc0 + 3)};
    st.acc_mtp = word(kCtlAccMtp);
    st.t_plain = word(kCtlTPlain);
    st.t_mtp = word(kCtlTMtp);
    st.t_lookup = word(kCtlTLookup);
    st.last_src = word(kCtlLastSrc);
    st.last_bucket = word(kCtlLastBucket);
    st.last_drafted = word(kCtlLastDrafted);
    const ControlResult res = control_step(a, st, pre.acc, pre.rt, d, m);
    if (lane == 0) {
        ctl_store(a.state + (int64_t)b * kCtlWords, st);
        control_write(a, b, res);
    }
}

// The emit step of a request by the workgroup that holds its final key:
// lookup outputs only, or lookup outputs and fusion (wavefront 0), or
// lookup outputs and the controller step (wavefront 0).
template <bool FUSE, bool CONTROL>
__device__ __forceinline__ void emit_request(const DraftArgs &a, int b, const Req &r, u64 key,
                                             int tid, int nthreads, const FusePre &pre,
                                             const CtlPre &cpre)
{
    if constexpr (FUSE) {
        if (tid < kWave)
            emit_and_fuse(a, b, r, key, tid, pre);
    } else {
        emit(a, b, r, key, tid, nthreads);
        if constexpr (CONTROL) {
            if (tid < kWave) {
                int32_t m = 0, d = 0;
                if (key != 0) {
                    m = (int32_t)(key >> 32);
                    const int32_t follow = r.L - 1 - (int32_t)(key & 0xffffffffu);
                    d = follow < a.k_max ? follow : a.k_max;
                }
                emit_control(a.control, b, d, m, tid, cpre);
            }
        }
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

// The same with APPEND: a chunk is loaded whole only below the old length
// (the row holds nothing newer yet); its other positions below the new
// length come from the row or from the append's source, one load each.
__device__ __forceinline__ int4 patch_chunk_append(int4 v, int64_t p0, const Req &r)
{
    const int32_t L = r.L;
    if (p0 + 0 >= 0 && p0 + 0 < L) v.x = tok_at<true>(r, p0 + 0);
    if (p0 + 1 >= 0 && p0 + 1 < L) v.y = tok_at<true>(r, p0 + 1);
    if (p0 + 2 >= 0 && p0 + 2 < L) v.z = tok_at<true>(r, p0 + 2);
    if (p0 + 3 >= 0 && p0 + 3 < L) v.w = tok_at<true>(r, p0 + 3);
    return v;
}

// Scans this wavefront's share of one tile and returns the lane's best key.
//
// A workgroup's tile of TILE candidate end positions [t0, t0 + TILE) is cut
// into one contiguous span per wavefront (kSpan 16-byte chunks). Each
// wavefront works alone, with no workgroup barrier: it loads its span plus
// the kHalo tokens before it (and, for the last wavefront, the chunk after
// it, which holds the tile's last positions when the row is not 16-byte
// aligned) and stages them in its own LDS region. Lane l holds chunks
// l, 64 + l, 128 + l, ... of the span, so each load instruction reads 1 KiB
// of consecutive bytes.
//
// FILTER3 (n_min >= 3): a position survives the register test only if its
// token and the two before it equal the suffix's last three tokens; the
// tokens before a chunk come from the lane to the left (DPP wavefront shift)
// or, for lane 0, from the previous slot's lane 63 or the halo. A rejected
// position matches fewer than 3 <= n_min tokens, so it can never produce a
// key. Otherwise only the first token is tested. Survivors extend backwards
// from LDS up to m tokens.
// CHECKED (the first and last tile of a request): loads stay inside the row
// and every position is range-checked; interior tiles skip both.
template <int TILE, int THREADS>
struct WaveGeom {
    static constexpr int kWaves = THREADS / kWave;
    static constexpr int kSpan = TILE / 4 / kWaves;  // chunks per wavefront
    static constexpr int kPer = kSpan / kWave;       // chunks per lane
};

// Issues this lane's loads of an interior tile (no range checks): its kPer
// span chunks and the extra chunk (halo for lanes 0..15, the chunk after the
// span for lane 16; other lanes re-read their first chunk). With `real`
// false every lane reads the context's 16 zero bytes instead (a load with
// no branch around it that moves no data worth counting).
template <int TILE, int THREADS>
__device__ __forceinline__ void load_interior(const int4 *arow, int64_t t0, bool real,
                                              const int4 *zero16,
                                              int4 (&v)[WaveGeom<TILE, THREADS>::kPer + 1])
{
    constexpr int kSpan = WaveGeom<TILE, THREADS>::kSpan;
    constexpr int kPer = WaveGeom<TILE, THREADS>::kPer;
    const int wave = threadIdx.x / kWave;
    const int lane = threadIdx.x & (kWave - 1);
    const int64_t gq0 = (t0 - kHalo) / 4 + (int64_t)wave * kSpan;  // exact
    const int qx = lane < kHaloChunks ? lane : (lane == kHaloChunks ? kHaloChunks + kSpan : -1);
    // the extra chunk first: slot 0's tests need the halo
    v[kPer] = gld_stream(real ? arow + (gq0 + (qx >= 0 ? qx : kHaloChunks + lane)) : zero16);
#pragma unroll
    for (int k = 0; k < kPer; ++k)
        v[k] = gld_stream(real ? arow + (gq0 + kHaloChunks + k * kWave + lane) : zero16);
}

// Buffer resource over one wavefront's window of a tile (load_window).
// Word 3 of the resource: 32-bit data format, no swizzle, no thread-id
// offset (the CDNA raw-buffer layout).
constexpr int32_t kBufWord3 = 0x00020000;

__device__ __forceinline__ int4 bld_stream(__amdgpu_buffer_rsrc_t rs, int32_t off)
{
    const v4i32 x = __builtin_amdgcn_raw_buffer_load_b128(rs, off, 0, 2 /* nt */);
    return make_int4(x[0], x[1], x[2], x[3]);
}

// Issues this lane's loads of a request's last tile, one that starts at
// least kHalo + 4 tokens into its row, through a buffer resource over this
// wavefront's window. The window's 16-byte blocks begin at local token 0 (a
// 16-byte boundary of the row); (avail + 3) / 4 of them hold a token of the
// row, avail being the row's length less local token 0's position. The
// resource's record count ends there, so the hardware returns zeros for
// every later block without touching memory: the chunks past the row cost
// no branch and no address select. The block that holds the row's last
// token is read whole (an aligned 16-byte block lies on one page); its
// positions past the end are never candidates. Chunk offsets are multiples
// of 16 and so is the record count, so every block is either wholly in
// range or wholly out.
template <int TILE, int THREADS>
__device__ __forceinline__ void load_window(const int4 *wbase, int32_t avail,
                                            int4 (&v)[WaveGeom<TILE, THREADS>::kPer + 1])
{
    constexpr int kSpan = WaveGeom<TILE, THREADS>::kSpan;
    constexpr int kPer = WaveGeom<TILE, THREADS>::kPer;
    constexpr int kWinW = kHaloChunks + kSpan + 1;
    const int lane = threadIdx.x & (kWave - 1);
    // the window's base and size are the same in every lane: taken into
    // scalar registers, so the resource needs no per-lane loop
    const int32_t av = __builtin_amdgcn_readfirstlane(avail < 4 * kWinW ? avail : 4 * kWinW);
    const int32_t nb = av <= 0 ? 0 : (av + 3) >> 2;
    const uint64_t wb = (uint64_t)(uintptr_t)wbase;
    const uint64_t wbu = (uint64_t)(uint32_t)__builtin_amdgcn_readfirstlane((int32_t)(uint32_t)wb) |
                         (uint64_t)(uint32_t)__builtin_amdgcn_readfirstlane((int32_t)(uint32_t)(wb >> 32)) << 32;
    const __amdgpu_buffer_rsrc_t rs =
        __builtin_amdgcn_make_buffer_rsrc((void *)(uintptr_t)wbu, (short)0, nb * 16, kBufWord3);
    // the extra chunk first: slot 0's tests need the halo
    const int qx = lane < kHaloChunks ? lane : (lane == kHaloChunks ? kHaloChunks + kSpan : kHaloChunks + lane);
    v[kPer] = bld_stream(rs, 16 * qx);
#pragma unroll
    for (int k = 0; k < kPer; ++k)
        v[k] = bld_stream(rs, 16 * (kHaloChunks + lane) + 16 * kWave * k);
}

template <int TILE, int THREADS, bool CHECKED, bool FILTER3, bool PRELOADED, bool APPEND,
          bool TAIL = false>
__device__ __forceinline__ u64 scan_wave(const DraftArgs &a, const Req &r, int64_t t0,
                                         int32_t mhat, int4 *lds_win, int32_t *lds_pat,
                                         int4 (&v)[WaveGeom<TILE, THREADS>::kPer + 1])
{
    constexpr int kWaves = THREADS / kWave;
    constexpr int kSpan = TILE / 4 / kWaves;         // chunks per wavefront
    constexpr int kPer = kSpan / kWave;              // chunks per lane
    static_assert(!(PRELOADED && APPEND), "an appending scan loads after the length");
    constexpr int kWinW = kHaloChunks + kSpan + 1;   // per-wavefront window
    static_assert(kSpan % kWave == 0, "whole chunks per lane");

    const int tid = threadIdx.x;
    const int wave = tid / kWave;
    const int lane = tid & (kWave - 1);
    const bool last_wave = wave == kWaves - 1;
    int4 *win = lds_win + wave * kWinW;
    int32_t *pat = lds_pat + wave * kWave;

    const int32_t nrel = (int32_t)(((int64_t)r.ncand - t0) < TILE ? (r.ncand - t0) : TILE);
    const int delta = (int)(((uintptr_t)r.h >> 2) & 3u);
    const int4 *arow = (const int4 *)(r.h - delta);
    // local chunk q of this wavefront is tile-window chunk wave * kSpan + q;
    // tile-window chunk 0 starts kHalo + delta tokens before t0.
    const int64_t gq0 = (t0 - kHalo) / 4 + (int64_t)wave * kSpan;  // exact
    const int64_t pq0 = t0 - kHalo - delta + 4 * (int64_t)wave * kSpan;  // position of local token 0
    const int32_t rq0 = (int32_t)(pq0 - t0);  // rel (position - t0) of local token 0
    // the extra chunk: halo (lanes 0..15), the chunk after the span (lane 16)
    const int qx = lane < kHaloChunks ? lane : (lane == kHaloChunks ? kHaloChunks + kSpan : -1);

    // 1. loads, all issued back to back with no branch in between (a load
    // inside a branch makes the compiler wait for it at the join). Lanes
    // without an extra chunk re-read their first chunk; lanes past the
    // suffix length re-read its first token.
    int32_t p1, p2, p3, pv;  // L >= 2 whenever a tile is scanned
    if constexpr (APPEND) {
        p1 = tok_at<true>(r, r.L - 1);
        p2 = tok_at<true>(r, r.L - 2);
        p3 = tok_at<true>(r, r.L - (mhat >= 3 ? 3 : 1));
        pv = tok_at<true>(r, r.L - mhat + (lane < mhat ? lane : 0));
    } else {
        p1 = gld(r.h + r.L - 1);
        p2 = gld(r.h + r.L - 2);
        p3 = gld(r.h + r.L - (mhat >= 3 ? 3 : 1));
        pv = gld(r.h + r.L - mhat + (lane < mhat ? lane : 0));
    }
    static_assert(!(PRELOADED && CHECKED), "tiles loaded ahead are interior tiles");
    if constexpr (PRELOADED) {
        // the caller issued this tile's loads before the length was known
    } else if constexpr (TAIL) {
        // the row's length less the position of local token 0: the true
        // difference lies in (-TILE - kHalo, 2^31), so it is exact modulo 2^32
        const int32_t avail = (int32_t)((uint32_t)r.L - (uint32_t)pq0);
        load_window<TILE, THREADS>(arow + gq0, avail, v);
    } else if constexpr (!CHECKED) {
        load_interior<TILE, THREADS>(arow, t0, true, a.zero16, v);
    } else {
        bool inside[kPer + 1];
#pragma unroll
        for (int k = 0; k <= kPer; ++k) {
            const int q = k < kPer ? kHaloChunks + k * kWave + lane : qx;
            inside[k] = q >= 0 && chunk_inside(pq0 + 4 * q, APPEND ? r.split : r.L);
            v[k] = gld_stream(inside[k] ? arow + (gq0 + q) : a.zero16);
        }
#pragma unroll
        for (int k = 0; k <= kPer; ++k) {
            const int q = k < kPer ? kHaloChunks + k * kWave + lane : qx;
            if (q >= 0 && !inside[k]) {
                if constexpr (APPEND)
                    v[k] = patch_chunk_append(v[k], pq0 + 4 * q, r);
                else
                    v[k] = patch_chunk(v[k], pq0 + 4 * q, r.h, r.L);
            }
        }
    }

    // 2. stage the window and the suffix in this wavefront's LDS region
    // (DS operations of one wavefront complete in order, so no barrier).
#pragma unroll
    for (int k = 0; k < kPer; ++k)
        win[kHaloChunks + k * kWave + lane] = v[k];
    if (qx >= 0)
        win[qx] = v[kPer];
    pat[lane] = pv;  // slots >= mhat are unused
    __builtin_amdgcn_wave_barrier();

    // 3. rejection tests. Bit 4k + i of `bits` says token i of slot k (slot
    // kPer: the extra chunk) goes on to extend.
    static_assert(4 * (kPer + 1) <= 32, "survivor bitmask is 32 bits");
    typedef uint32_t mask_t;
    mask_t bits = 0;
    // Positions owned by this wavefront: rel in [lo, hi). The span's
    // positions belong to it, the chunk after the span only to the last
    // wavefront; with the 3-token filter positions 0 and 1 are left out (a
    // match ending there has fewer than 3 tokens, below n_min).
    const int32_t lo = FILTER3 ? (t0 < 2 ? 2 - (int32_t)t0 : 0) : 0;
    const int32_t span_end = rq0 + 4 * (kHaloChunks + kSpan);
    const int32_t hi = last_wave ? nrel : (span_end < nrel ? span_end : nrel);
    const int32_t ell0 = FILTER3 ? 3 : 1;  // tokens known to match for a survivor
    // two adjacent suffix tokens as one 64-bit value (earlier token low)
    const u64 q21 = (u64)(uint32_t)p2 | (u64)(uint32_t)p1 << 32;
    const u64 q32 = (u64)(uint32_t)p3 | (u64)(uint32_t)p2 << 32;
#pragma unroll
    for (int k = 0; k < kPer; ++k) {
        const int32_t r0 = rq0 + 4 * (kHaloChunks + k * kWave + lane);  // rel of token 0
        bool c[4];
        if constexpr (FILTER3) {
            // the two tokens before this chunk: lane l - 1's last two, by a
            // wavefront shift; lane 0, which has no source lane and keeps
            // the shift's `old` operand, gets lane 63 of the previous slot
            // (rotated to lane 0) or the halo's last chunk
            const int32_t oz = k > 0 ? __builtin_amdgcn_mov_dpp(v[k - 1].z, 0x13c /* wave_ror:1 */, 0xf, 0xf, false)
                                     : __builtin_amdgcn_readlane(v[kPer].z, kHaloChunks - 1);
            const int32_t ow = k > 0 ? __builtin_amdgcn_mov_dpp(v[k - 1].w, 0x13c /* wave_ror:1 */, 0xf, 0xf, false)
                                     : __builtin_amdgcn_readlane(v[kPer].w, kHaloChunks - 1);
            const int32_t pz = __builtin_amdgcn_update_dpp(oz, v[k].z, 0x138 /* wave_shr:1 */, 0xf, 0xf, false);
            const int32_t pw = __builtin_amdgcn_update_dpp(ow, v[k].w, 0x138 /* wave_shr:1 */, 0xf, 0xf, false);
            // each position's three tokens as a 64-bit pair and one token
            const u64 xy = (u64)(uint32_t)v[k].x | (u64)(uint32_t)v[k].y << 32;
            const u64 zw = (u64)(uint32_t)v[k].z | (u64)(uint32_t)v[k].w << 32;
            const u64 zwp = (u64)(uint32_t)pz | (u64)(uint32_t)pw << 32;
            c[0] = zwp == q32 && v[k].x == p1;
            c[1] = xy == q21 && pw == p3;
            c[2] = xy == q32 && v[k].z == p1;
            c[3] = zw == q21 && v[k].y == p3;
        } else {
#pragma unroll
            for (int i = 0; i < 4; ++i)
                c[i] = comp(v[k], i) == p1;
        }
        // inside an interior tile only wavefront 0's first chunk can hold
        // positions outside [lo, hi) (the delta tokens before t0)
        if (CHECKED || k == 0) {
#pragma unroll
            for (int i = 0; i < 4; ++i)
                c[i] = c[i] && r0 + i >= lo && (!CHECKED || r0 + i < hi);
        }
        bits |= ((mask_t)c[0] | (mask_t)c[1] << 1 | (mask_t)c[2] << 2 | (mask_t)c[3] << 3) << (4 * k);
    }
    // the chunk after the span holds the tile's last positions (those of
    // them the last wavefront owns): tested on the first token only
    if (last_wave && lane == kHaloChunks) {
        const int32_t r0 = rq0 + 4 * qx;
#pragma unroll
        for (int i = 0; i < 4; ++i)
            bits |= (mask_t)(r0 + i >= lo && r0 + i < hi && comp(v[kPer], i) == p1) << (4 * kPer + i);
    }

    // 4. survivors extend backwards from LDS. Most wavefronts have none and
    // skip this with one branch. With a few survivors (at most kWaveExt
    // lanes holding one each, the usual case) the whole wavefront extends
    // each in one LDS round trip: lane j compares the token j before the
    // candidate's end with suffix token j, and the first mismatch (or
    // j = lim) is the match length. Otherwise each lane walks its own
    // bitmask, kExtBlock tokens in its first round trip per survivor and
    // 2 * kExtBlock in each later one.
    u64 best = 0;
    if (__any(bits != 0)) {
        if constexpr (TAIL) {
            // a last tile's span runs past its candidates (the suffix itself,
            // zero blocks and bytes past the row can pass the test there):
            // keep the positions below hi. The extra chunk was range-checked
            // when it was tested.
            mask_t keep = (mask_t)0xf << (4 * kPer);
#pragma unroll
            for (int k = 0; k < kPer; ++k) {
                const int32_t r0 = rq0 + 4 * (kHaloChunks + k * kWave + lane);
                const int32_t n = hi - r0 < 0 ? 0 : (hi - r0 > 4 ? 4 : hi - r0);
                keep |= (mask_t)((1u << n) - 1u) << (4 * k);
            }
            bits &= keep;
        }
        const int32_t *wt = (const int32_t *)win;
        // lowest rel an extension may reach: position 0 (first tile) or the halo
        const int32_t floor_rel = t0 < kHalo ? -(int32_t)t0 : -kHalo;
        const u64 holders = __ballot(bits != 0);
        if (__popcll(holders) <= kWaveExt && !__any((bits & (bits - 1)) != 0)) {
            u64 hl = holders;  // the same in every lane, as is wb
            u64 wb = 0;
            while (hl) {
                const int src = __builtin_ctzll(hl);
                hl &= hl - 1;
                const uint32_t sb = __builtin_amdgcn_readlane(bits, src);
                const int bit = __builtin_ctz(sb);
                const int k = bit >> 2, i = bit & 3;
                // only the last wavefront's lane kHaloChunks tests the extra chunk
                const int q = k < kPer ? kHaloChunks + k * kWave + src : kHaloChunks + kSpan;
                const int32_t slot = 4 * q + i;
                const int32_t rel = rq0 + slot;
                const int32_t lim = (!CHECKED || rel - mhat + 1 >= floor_rel) ? mhat : rel - floor_rel + 1;
                const bool in = lane < lim;
                const int32_t tk = in ? wt[slot - lane] : 0;
                const int32_t pt = in ? pat[mhat - 1 - lane] : 0;
                const u64 miss = __ballot(!in || tk != pt);
                const int32_t ell = miss ? __builtin_ctzll(miss) : kWave;
                if (ell >= a.n_min) {
                    const u64 key = ((u64)(uint32_t)ell << 32) | (uint32_t)(t0 + rel);
                    wb = key > wb ? key : wb;
                }
            }
            return wb;
        }
        while (bits) {
            const int bit = __builtin_ctz(bits);
            bits &= bits - 1;
            const int k = bit >> 2, i = bit & 3;
            const int q = k < kPer ? kHaloChunks + k * kWave + lane : qx;
            const int32_t slot = 4 * q + i;
            const int32_t rel = rq0 + slot;
            int32_t ell = k < kPer ? ell0 : 1;
            ell = ell < mhat ? ell : mhat;
            // each round trip's reads are independent; a mismatch mask marks
            // the first token that differs (or lies past m or before
            // position 0)
            const int32_t lim = (!CHECKED || rel - mhat + 1 >= floor_rel) ? mhat : rel - floor_rel + 1;
            // the first round trip compares kExtBlock tokens (most survivors
            // fail there); a candidate that passes it is likely a long match,
            // and the following rounds compare twice as many
            if (ell < lim) {
                int32_t tk[kExtBlock], pt[kExtBlock];
#pragma unroll
                for (int u = 0; u < kExtBlock; ++u) {
                    const int32_t j = ell + u < lim ? ell + u : ell;
                    tk[u] = wt[slot - j];
                    pt[u] = pat[mhat - 1 - j];
                }
                uint32_t miss = 1u << kExtBlock;
#pragma unroll
                for (int u = 0; u < kExtBlock; ++u)
                    miss |= (uint32_t)((tk[u] != pt[u]) | (ell + u >= lim)) << u;
                const int run = __builtin_ctz(miss);
                ell += run;
                if (run == kExtBlock) {
                    while (ell < lim) {
                        // all reads first (indices clamped into range, no
                        // branches), then the comparisons
                        int32_t tk2[2 * kExtBlock], pt2[2 * kExtBlock];
#pragma unroll
                        for (int u = 0; u < 2 * kExtBlock; ++u) {
                            const int32_t j = ell + u < lim ? ell + u : ell;
                            tk2[u] = wt[slot - j];
                            pt2[u] = pat[mhat - 1 - j];
                        }
                        uint32_t miss2 = 1u << (2 * kExtBlock);
#pragma unroll
                        for (int u = 0; u < 2 * kExtBlock; ++u)
                            miss2 |= (uint32_t)((tk2[u] != pt2[u]) | (ell + u >= lim)) << u;
                        const int run2 = __builtin_ctz(miss2);
                        ell += run2;
                        if (run2 < 2 * kExtBlock)
                            break;
                    }
                }
            }
            if (ell >= a.n_min) {
                const u64 key = ((u64)(uint32_t)ell << 32) | (uint32_t)(t0 + rel);
                best = key > best ? key : best;
            }
        }
    }
    return best;
}

// The fields needed first are separate leading arguments so that they can be
// preloaded into SGPRs at wave launch; the rest come in `args`.
//
// STRIDED batches (row b at base + b * stride) know every tile's address
// from those arguments alone. A tile that lies inside every row by the
// caller's bound min_len (checked against each length on the device) then
// issues its loads at once, before its length is read from memory; other
// tiles, and row-table batches, read the length and row first.
//
// APPEND (a strided batch over the context's store, fused gather): row b
// first gains counts[b] tokens, as pld_append would add them. Positions at
// or past the old length are read from the append's source, so no
// workgroup depends on the copy, which the request's last tile makes. The
// new length is stored by the workgroup that emits the draft, and every
// workgroup of the request (those without candidates too) counts itself in
// before that, so none of them can read the new length as its old one.
template <int TILE, int THREADS, bool STRIDED, bool FUSE, bool CONTROL, bool APPEND>
__global__ __launch_bounds__(THREADS) void pld_scan(const void *rows, const int32_t *lengths,
                                                    int32_t batch, int32_t max_len,
                                                    int32_t n_min, int32_t n_max, int64_t stride,
                                                    int32_t min_len, DraftArgs args)
{
    DraftArgs a = args;
    if constexpr (STRIDED) {
        a.base = (const int32_t *)rows;
        a.stride = stride;
        a.min_len = min_len;
    } else {
        a.histories = (const int32_t *const *)rows;
        a.stride = 0;
    }
    a.lengths = lengths;
    a.batch = batch;
    a.max_len = max_len;
    a.n_min = n_min;
    a.n_max = n_max;
    static_assert(THREADS % kWave == 0, "whole wavefronts");
    static_assert(TILE % (4 * THREADS) == 0, "whole chunks per lane");
    constexpr int kWaves = THREADS / kWave;
    constexpr int kWinW = kHaloChunks + TILE / 4 / kWaves + 1;
    constexpr int kPer = WaveGeom<TILE, THREADS>::kPer;
    static_assert(kWave >= PLD_N_MAX_LIMIT, "one suffix token per lane");

    __shared__ int4 win[kWaves * kWinW];
    __shared__ int32_t pat[kWaves * kWave];
    __shared__ u64 wbest[kWaves];

    const int tid = threadIdx.x;
    // grid: x = request, y = tile (and z, when a request has more tiles than
    // the y dimension holds: y is then exactly kGridY tiles, and tile =
    // z * kGridY + y). Workgroups are dispatched x-fastest, so consecutive
    // ones hold the same tile of consecutive requests.
    const int tile = (int)(blockIdx.z * kGridY + blockIdx.y);
    const int b = blockIdx.x;
    const int64_t t0 = (int64_t)tile * TILE;
    // tiles per request (the grid may hold a few more when split over z)
    const int32_t req_tiles = a.max_len > 1 ? (int32_t)(((int64_t)a.max_len - 1 + TILE - 1) / TILE) : 1;
    if (APPEND && tile >= req_tiles)
        return;  // past every request's tiles: counts in nowhere, reads nothing

    int4 v[kPer + 1];
    bool ahead = false;
    if constexpr (STRIDED && !APPEND) {
        // interior for every row of length >= min_len
        ahead = t0 >= kHalo + 4 && t0 + TILE + 4 <= (int64_t)min_len - 1;
        const int4 *arow = (const int4 *)(a.base + (int64_t)b * stride);
        // a tile not loaded ahead re-reads the row's first chunk in every lane
        load_interior<TILE, THREADS>(arow, t0, ahead, arow, v);
    }

    const Req r = load_req<APPEND>(a, b, TILE);
    // the fusion's per-request inputs, issued with the request's length.
    // (Issued late, before the arrival add, as the controller's are below,
    // they measured slower on a batch of 8 requests of 25,000 tokens.)
    FusePre pre{};
    if constexpr (FUSE)
        pre = fuse_preload(a.fuse, b, tid & (kWave - 1));
    // workgroups counted in by the fused gather: the tiles that hold
    // candidates, or with APPEND every tile of the request
    const int32_t arrive = APPEND ? req_tiles : r.ntiles;
    if (!APPEND && tile >= r.ntiles)
        return;  // this request has no candidates in this tile
    if (r.err && tid == 0 && (!APPEND || tile == 0))
        atomicOr(a.err, r.err);
    if constexpr (APPEND) {
        if (tile == 0 && tid == 0) {
            if (r.app_err)
                atomicOr(a.err, r.app_err);
        }
        // the copy; no workgroup of this launch reads these positions of the row
        if (tile == r.ntiles - 1) {
            int32_t *dst = a.app_store + (int64_t)b * a.stride + r.split;
            for (int t = tid; t < r.add; t += THREADS)
                dst[t] = gld(r.src + t);
        }
    }

    const int32_t mhat = r.L - 1 < a.n_max ? r.L - 1 : a.n_max;
    u64 best = 0;
    if ((!APPEND || tile < r.ntiles) && mhat >= a.n_min) {
        // interior: halo and the chunk after the tile lie inside the row (below
        // the old length with APPEND) and every position of the tile is a
        // candidate
        const bool interior = t0 >= kHalo + 4 && t0 + TILE + 4 <= (int64_t)(APPEND ? r.split : r.L) - 1;
        // a request's last tile that is not also its first runs the interior
        // tests: its window's blocks past the row load as zeros, and its
        // positions past the candidates are dropped from the survivors
        const bool tail = !APPEND && !interior && t0 >= kHalo + 4;
        const bool f3 = a.n_min >= 3;
        if (STRIDED && !APPEND && ahead && r.err == 0)
            best = f3 ? scan_wave<TILE, THREADS, false, true, true, false>(a, r, t0, mhat, win, pat, v)
                      : scan_wave<TILE, THREADS, false, false, true, false>(a, r, t0, mhat, win, pat, v);
        else if (interior)
            best = f3 ? scan_wave<TILE, THREADS, false, true, false, APPEND>(a, r, t0, mhat, win, pat, v)
                      : scan_wave<TILE, THREADS, false, false, false, APPEND>(a, r, t0, mhat, win, pat, v);
        else if (tail)
            best = f3 ? scan_wave<TILE, THREADS, false, true, false, false, true>(a, r, t0, mhat, win, pat, v)
                      : scan_wave<TILE, THREADS, false, false, false, false, true>(a, r, t0, mhat, win, pat, v);
        else
            best = f3 ? scan_wave<TILE, THREADS, true, true, false, APPEND>(a, r, t0, mhat, win, pat, v)
                      : scan_wave<TILE, THREADS, true, false, false, APPEND>(a, r, t0, mhat, win, pat, v);
    }
    // 5. wavefront maximum by DPP (only where the lanes hold different values),
    // then lane 0 merges it: into the request's slot (separate gather
    // kernel) or, fused, into the workgroup's maximum (one LDS word per
    // wavefront and a single barrier, after which wavefront 0 alone goes on).
    {
        // a value every lane already holds (no match, or the wavefront-level
        // extension's result) needs no reduction
        const u64 first = ((u64)(uint32_t)__builtin_amdgcn_readfirstlane((int)(uint32_t)(best >> 32)) << 32) |
                          (uint32_t)__builtin_amdgcn_readfirstlane((int)(uint32_t)best);
        if (__any(best != first))
            best = wave_max_u64(best);
        else
            best = first;
    }
    const bool found = best != 0;
    const bool leader = (tid & (kWave - 1)) == 0;
    if (!a.fused) {
        // the gather kernel reads the request's slot after this kernel ends
        if (found && leader)
            __hip_atomic_fetch_max(&a.slots[b].key, best, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        return;
    }
    // one LDS word per wavefront, one barrier; then wavefront 0 alone
    // merges, and emits if it is the last to arrive
    u64 m = best;
    bool premerged = false;  // m is the workgroup's increase of the request's key
    if constexpr (kWaves > 1) {
        // With several workgroups per request, a wavefront with a match takes
        // its atomicMax as soon as its own tests end, and leaves the increase
        // it made; the workgroup adds the sum with its arrival.
        u64 word = found ? best : 0ull;
        if (arrive > 1 && found && leader) {
            const u64 old = __hip_atomic_fetch_max(&a.slots[b].key, best, __ATOMIC_RELAXED,
                                                   __HIP_MEMORY_SCOPE_AGENT);
            word = best > old ? best - old : 0ull;
        }
        if (leader)
            wbest[tid / kWave] = word;
        __syncthreads();
        if (tid >= kWave)
            return;
        m = wbest[0];
        if (arrive > 1) {
            premerged = true;
#pragma unroll
            for (int w = 1; w < kWaves; ++w)
                m += wbest[w];
        } else {
#pragma unroll
            for (int w = 1; w < kWaves; ++w)
                m = wbest[w] > m ? wbest[w] : m;
        }
    } else if (!found) {
        m = 0;
    }

    // 6. fused gather: the last workgroup of the request to arrive emits the
    // draft. Only atomic read-modify-writes at agent scope cross
    // workgroups: each is performed at the location's single point of
    // coherence. A wavefront with a match takes its atomicMax's return
    // before the barrier, and its workgroup adds the increases made to the
    // maximum together with its arrival; the increases of all atomicMax
    // calls sum to the final maximum, so the workgroup that counts last
    // reads it from its own add (and clears the slot).
    // the controller's per-request inputs, issued before the arrival add so
    // that they land within its round trip
    CtlPre cpre{};
    if constexpr (CONTROL)
        cpre = control_preload(a.control, b, tid & (kWave - 1));
    int last = 1;
    if (arrive > 1) {
        if (tid == 0) {
            // this workgroup's increase of the maximum (0 without a match),
            // known once its atomicMax calls return, is added with its arrival
            u64 inc = premerged ? m : 0ull;
            if (!premerged && m) {
                const u64 old = __hip_atomic_fetch_max(&a.slots[b].key, m, __ATOMIC_RELAXED,
                                                       __HIP_MEMORY_SCOPE_AGENT);
                inc = m > old ? m - old : 0;
            }
            const u64 prev = __hip_atomic_fetch_add(&a.slots[b].acc, (inc << 24) + 1,
                                                    __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
            last = (uint32_t)(prev & 0xffffffu) == (uint32_t)(arrive - 1);
            if (last) {
                // every other workgroup's increase is in `prev`: their maxima
                // returned before they counted in
                m = (prev >> 24) + inc;
                __hip_atomic_store(&a.slots[b].key, 0ull, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
                __hip_atomic_store(&a.slots[b].acc, 0ull, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
            }
        }
        // lane 0's results to the whole wavefront
        last = __builtin_amdgcn_readfirstlane(last);
        m = ((u64)(uint32_t)__builtin_amdgcn_readfirstlane((int)(uint32_t)(m >> 32)) << 32) |
            (uint32_t)__builtin_amdgcn_readfirstlane((int)(uint32_t)m);
    }
    if (!last)
        return;
    if constexpr (APPEND) {
        emit<true>(a, b, r, m, tid, kWave);
        if (tid == 0 && r.add > 0)
            a.app_lengths[b] = r.L;
    } else {
        emit_request<FUSE, CONTROL>(a, b, r, m, tid, kWave, pre, cpre);
    }
}

__global__ __launch_bounds__(kWave) void pld_gather(DraftArgs a)
{
    const int b = blockIdx.x;
    const Req r = load_req(a, b, 1);
    const u64 key = a.slots[b].key;
    if (a.do_fuse)
        emit_request<true, false>(a, b, r, r.err ? 0ull : key, threadIdx.x, kWave,
                                  fuse_preload(a.fuse, b, threadIdx.x), CtlPre{});
    else if (a.do_control)
        emit_request<false, true>(a, b, r, r.err ? 0ull : key, threadIdx.x, kWave, FusePre{},
                                  control_preload(a.control, b, threadIdx.x));
    else
        emit_request<false, false>(a, b, r, r.err ? 0ull : key, threadIdx.x, kWave, FusePre{},
                                   CtlPre{});
    __syncthreads();
    if (threadIdx.x == 0 && key != 0)
        a.slots[b].key = 0;
}

// One workgroup per request: append counts[b] tokens to store row b.
__global__ __launch_bounds__(256) void pld_append_kernel(AppendArgs a)
{
    __shared__ int32_t s_len;
    __shared__ int s_ok;
    const int b = blockIdx.x;
    if (threadIdx.x == 0) {
        const int32_t len = a.lengths[b];
        // a length outside [0, max_len] (the array is the caller's to write
        // through pld_histories) rejects the append like an overflow
        const uint32_t e = append_error(len, a.counts[b], a.max_len);
        if (e)
            atomicOr(a.err, e);
        s_len = len;
        s_ok = e == 0;
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

// pld_fuse: one wavefront per request, lookup drafts read from the caller's
// buffers.
__global__ __launch_bounds__(kWave) void pld_fuse_kernel(FuseArgs a)
{
    const int b = blockIdx.x;
    const int t = threadIdx.x;
    const int32_t d = a.lookup_len[b];
    const int32_t m = a.lookup_match[b];
    const int32_t lk = d >= 0 && d <= a.lookup_k && t < d ? a.lookup[(int64_t)b * a.lookup_k + t]
                                                          : -1;
    fuse_request(a, b, t, d, m, lk, fuse_preload(a, b, t));
}

template <int TILE, int THREADS>
hipError_t launch_scan(const DraftArgs &a, int64_t tiles_per_req, hipStream_t s)
{
    // y holds at most kGridY tiles; more go on in z
    const unsigned ty = tiles_per_req < kGridY ? (unsigned)tiles_per_req : kGridY;
    const dim3 grid((unsigned)a.batch, ty, (unsigned)((tiles_per_req + ty - 1) / ty));
    if (a.stride && (a.do_fuse || a.do_control))
        return hipErrorInvalidValue;  // no entry point fuses a strided batch
    if (a.do_fuse && a.do_control)
        return hipErrorInvalidValue;  // no entry point does both
    if (a.do_append && (!a.stride || a.min_len != 0 || !a.fused || a.do_fuse || a.do_control))
        return hipErrorInvalidValue;  // an append runs with the store's strided scan only
    if (a.do_append)
        hipLaunchKernelGGL((pld_scan<TILE, THREADS, true, false, false, true>),
                           grid, dim3(THREADS), 0, s, (const void *)a.base,
                           a.lengths, a.batch, a.max_len, a.n_min, a.n_max, a.stride, 0, a);
    else if (a.stride)
        hipLaunchKernelGGL((pld_scan<TILE, THREADS, true, false, false, false>),
                           grid, dim3(THREADS), 0, s, (const void *)a.base,
                           a.lengths, a.batch, a.max_len, a.n_min, a.n_max, a.stride, a.min_len,
                           a);
    else if (a.do_fuse && a.fused)
        hipLaunchKernelGGL((pld_scan<TILE, THREADS, false, true, false, false>),
                           grid, dim3(THREADS), 0, s, (const void *)a.histories,
                           a.lengths, a.batch, a.max_len, a.n_min, a.n_max, (int64_t)0, 0, a);
    else if (a.do_control && a.fused)
        hipLaunchKernelGGL((pld_scan<TILE, THREADS, false, false, true, false>),
                           grid, dim3(THREADS), 0, s, (const void *)a.histories,
                           a.lengths, a.batch, a.max_len, a.n_min, a.n_max, (int64_t)0, 0, a);
    else
        hipLaunchKernelGGL((pld_scan<TILE, THREADS, false, false, false, false>),
                           grid, dim3(THREADS), 0, s, (const void *)a.histories,
                           a.lengths, a.batch, a.max_len, a.n_min, a.n_max, (int64_t)0, 0, a);
    return hipGetLastError();
}

}  // namespace

}  // namespace pld

// The no-allocation entry point's reduction state: one copy per GPU, held
// from the moment the library's code object is loaded until the process
// ends. Host code never names this array's address directly (the name is a
// host-side stand-in); it uses the device address static_scratch() looks up.
static __device__ __align__(256) unsigned char scratch[sizeof(pld::StaticScratch)];

namespace pld {

hipError_t static_scratch(StaticScratch **out, hipStream_t s)
{
    constexpr int kMaxDevices = 64;
    static std::mutex mu;
    static void *ptr[kMaxDevices];
    static bool cleared[kMaxDevices];
    int dev = 0;
    hipError_t e = hipGetDevice(&dev);
    if (e != hipSuccess)
        return e;
    if (dev < 0 || dev >= kMaxDevices)
        return hipErrorInvalidDevice;
    std::lock_guard<std::mutex> lock(mu);
    if (!ptr[dev]) {
        void *p = nullptr;
        e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
        if (e != hipSuccess)
            return e;
        ptr[dev] = p;
    }
    if (!cleared[dev]) {
        // the slots and the zero block must start at zero; a fill kernel
        // rather than a memset, so that a captured first call replays cleanly
        e = launch_fill((int32_t *)ptr[dev], (int64_t)(sizeof(StaticScratch) / 4), 0, s);
        if (e != hipSuccess)
            return e;
        cleared[dev] = true;
    }
    *out = (StaticScratch *)ptr[dev];
    return hipSuccess;
}

hipError_t launch_draft(const DraftArgs &a, int tile_tokens, hipStream_t s)
{
    const int64_t tiles = a.max_len > 1 ? ((int64_t)a.max_len - 1 + tile_tokens - 1) / tile_tokens : 1;
    hipError_t e;
    switch (tile_tokens) {
    // every size keeps 4 chunks (16 tokens) per lane, except the smallest
    case 256: e = launch_scan<256, 64>(a, tiles, s); break;
    case 1024: e = launch_scan<1024, 64>(a, tiles, s); break;
    case 2048: e = launch_scan<2048, 128>(a, tiles, s); break;
    case 4096: e = launch_scan<4096, 256>(a, tiles, s); break;
    case 8192: e = launch_scan<8192, 512>(a, tiles, s); break;
    case 16384: e = launch_scan<16384, 1024>(a, tiles, s); break;
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

hipError_t launch_fuse(const FuseArgs &a, int32_t batch, hipStream_t s)
{
    if (batch <= 0)
        return hipSuccess;
    hipLaunchKernelGGL(pld_fuse_kernel, dim3((unsigned)batch), dim3(kWave), 0, s, a);
    return hipGetLastError();
}

}  // namespace pld
