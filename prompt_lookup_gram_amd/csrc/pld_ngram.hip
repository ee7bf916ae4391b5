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
// `cap` 32-byte slots (a power of two at least twice max_len, so at most half
// full and every probe sequence reaches an empty slot). Word 0 of a slot is
// (count << 32 | end + 1), `end` the end position of the occurrence that
// claimed it (0 = empty); words 2 and 3 hold its first 4 tokens.
//  - the pair table holds one slot per (n + 1)-gram of the history (its 5th
//    token, for n = 4, in the low half of word 1); count is how often its
//    first n tokens were followed by its last one;
//  - the gram table holds one slot per n-gram that was followed at least
//    once: count is its occurrences followed by a token, word 1 (`top`) the
//    packed maximum of (successor count << 32 | ~order(token)) over its
//    successors.
// The maximum over packed words is the most frequent successor, the
// smaller token on a tie (order() maps signed order onto unsigned). Counts
// only grow, and each increment of a pair's count offers (new count,
// token) to the gram's maximum, so after an append the maximum is exactly
// the one over final counts whatever order the atomics ran in. Nothing is
// approximate: slots are identified by their full tokens, so the drafts
// equal those of a brute-force recount.
//
// Inserts: appending token p (p >= 1) adds, for each n <= min(n_max, p), one
// occurrence of the n-gram h[p - n .. p) followed by h[p]. One thread per
// (p, n) loads a 4-slot window of both tables' probe sequences at once and
// finds, in each, the first slot that is empty or holds its tokens: a slot
// claimed by an earlier append is compared with the tokens stored in it; one
// claimed during this append (its tokens may not be stored yet) with the
// history at its end position (old tokens from the store, new ones from the
// append's source row). Then both atomics go out together: a
// compare-and-swap claims an empty slot with count 1, an add counts a held
// one. Only the pair's new count is waited for; the gram's add and the
// maximum of its top word are not. A claim that loses a race re-examines
// the slot it lost.
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
constexpr int kVerifySlots = 4;  // lanes per round when verifying along an occurrence
constexpr int kVerifyRounds = kWave / kVerifySlots;
constexpr int kSlotWords = 4;    // 64-bit words per slot of either table
constexpr u64 kOne = 1ull << 32; // count 1 in a slot's first word

__device__ __forceinline__ u64 *gram_table(const NgramArgs &a, int b, int n)
{
    return a.grams + ((int64_t)b * a.n_max + (n - 1)) * a.cap * kSlotWords;
}

__device__ __forceinline__ u64 *pair_table(const NgramArgs &a, int b, int n)
{
    return a.pairs + ((int64_t)b * a.n_max + (n - 1)) * a.cap * kSlotWords;
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

constexpr int kProbe = 4;  // slots an insert loads per table per round trip

struct Window {
    ulonglong2 head[kProbe];  // words 0, 1
    ulonglong2 key[kProbe];   // words 2, 3
};

__device__ __forceinline__ void load_window(const u64 *tab, int64_t cap, int64_t slot, Window &w)
{
    for (int i = 0; i < kProbe; ++i) {
        const u64 *s = tab + ((slot + i) & (cap - 1)) * kSlotWords;
        w.head[i] = *(const ulonglong2 *)s;
        w.key[i] = *(const ulonglong2 *)(s + 2);
    }
}

// Does a held slot (words w0, w1, key) count the nk tokens tk? `fresh_from`
// is the first end position this append can claim: a slot claimed before it
// has its tokens stored, a newer one is compared with the history.
__device__ __forceinline__ bool stored_equal(u64 w1, ulonglong2 key, int nk, const int32_t *tk)
{
    return (int32_t)(uint32_t)key.x == tk[0] && (nk < 2 || (int32_t)(key.x >> 32) == tk[1]) &&
           (nk < 3 || (int32_t)(uint32_t)key.y == tk[2]) &&
           (nk < 4 || (int32_t)(key.y >> 32) == tk[3]) &&
           (nk < 5 || (int32_t)(uint32_t)w1 == tk[4]);
}

template <typename Tok>
__device__ bool holds(u64 w0, u64 w1, ulonglong2 key, int nk, const int32_t *tk,
                      int64_t fresh_from, const Tok &tok)
{
    const int64_t r = (int64_t)(uint32_t)w0 - 1;
    if (r < fresh_from)
        return stored_equal(w1, key, nk, tk);
    bool same = true;
    for (int j = 0; j < nk; ++j)
        same = same && tok(r - nk + 1 + j) == tk[j];
    return same;
}

// What a loaded window says without further loads, one bit per slot:
// empty, holding tk by its stored tokens, or claimed during this append
// (to be compared with the history).
struct Marks {
    uint32_t empty, match, fresh;
};

__device__ __forceinline__ Marks mark(const Window &w, int nk, const int32_t *tk,
                                      int64_t fresh_from)
{
    Marks m{0, 0, 0};
    for (int i = 0; i < kProbe; ++i) {
        const u64 w0 = w.head[i].x;
        const bool occ = (uint32_t)w0 != 0;
        const bool old = (int64_t)(uint32_t)w0 - 1 < fresh_from;
        m.empty |= (uint32_t)!occ << i;
        m.match |= (uint32_t)(occ && old && stored_equal(w.head[i].y, w.key[i], nk, tk)) << i;
        m.fresh |= (uint32_t)(occ && !old) << i;
    }
    return m;
}

// The first slot at or after `slot` in probe order that is empty (*empty) or
// holds tk, starting from the loaded window `w` and its marks.
template <typename Tok>
__device__ int64_t locate(const u64 *tab, int64_t cap, int64_t slot, Window &w, Marks m, int nk,
                          const int32_t *tk, int64_t fresh_from, const Tok &tok, bool *empty)
{
    for (int64_t probed = 0; probed < cap; probed += kProbe) {
        for (int i = 0; i < kProbe; ++i) {
            const bool hit = ((m.empty | m.match) >> i) & 1u ||
                             (((m.fresh >> i) & 1u) &&
                              holds(w.head[i].x, 0, ulonglong2{0, 0}, nk, tk, fresh_from, tok));
            if (hit) {
                *empty = (m.empty >> i) & 1u;
                return (slot + i) & (cap - 1);
            }
        }
        slot = (slot + kProbe) & (cap - 1);
        load_window(tab, cap, slot, w);
        m = mark(w, nk, tk, fresh_from);
    }
    *empty = false;
    return -1;  // not reached: a table is at most half full
}

// After a lost claim at `slot` (the winner's word 0 in w0): the slot to
// count in, found again from there.
template <typename Tok>
__device__ int64_t after_lost_claim(const u64 *tab, int64_t cap, int64_t slot, u64 w0, int nk,
                                    const int32_t *tk, int64_t fresh_from, const Tok &tok,
                                    bool *empty)
{
    // (the winner normally claimed during this append, and holds() then
    // compares the history; an older claim is compared with its stored tokens)
    u64 w1 = 0;
    ulonglong2 key{0, 0};
    if ((int64_t)(uint32_t)w0 - 1 < fresh_from) {
        const u64 *s = tab + slot * kSlotWords;
        w1 = s[1];
        key = *(const ulonglong2 *)(s + 2);
    }
    if (holds(w0, w1, key, nk, tk, fresh_from, tok)) {
        *empty = false;
        return slot;
    }
    Window w;
    load_window(tab, cap, (slot + 1) & (cap - 1), w);
    return locate(tab, cap, (slot + 1) & (cap - 1), w, mark(w, nk, tk, fresh_from), nk, tk,
                  fresh_from, tok, empty);
}

// Stores a freshly claimed slot's tokens (words 2, 3; the 5th in word 1).
__device__ __forceinline__ void store_key(u64 *s, int nk, const int32_t *tk)
{
    s[2] = (uint32_t)tk[0] | (nk > 1 ? (u64)(uint32_t)tk[1] << 32 : 0);
    if (nk > 2)
        s[3] = (uint32_t)tk[2] | (nk > 3 ? (u64)(uint32_t)tk[3] << 32 : 0);
    if (nk > 4)
        s[1] = (uint32_t)tk[4];
}

__device__ __forceinline__ bool claim(u64 *s, u64 word, u64 *cur)
{
    *cur = 0;
    return __hip_atomic_compare_exchange_strong(s, cur, word, __ATOMIC_RELAXED, __ATOMIC_RELAXED,
                                                __HIP_MEMORY_SCOPE_AGENT);
}

// The checks pld_append_kernel makes, in the same words.
__device__ __forceinline__ bool append_ok(const NgramArgs &a, int32_t old_len, int32_t c)
{
    return c >= 0 && old_len >= 0 && (int64_t)old_len + c <= a.max_len;
}

// Counts position p at length n: the n-gram tk[0..n) (ending at p - 1) was
// followed by tk[n] = h[p]. Tokens are read through `tok` (LDS or memory);
// old_len is the request's length before the append.
template <typename Tok>
__device__ void insert_one(const NgramArgs &a, int b, int32_t old_len, const Tok &tok, int64_t p,
                           int n)
{
    int32_t tk[5];
    u64 h = kHashSeed;
    for (int j = 0; j < n; ++j) {
        tk[j] = tok(p - n + j);
        h = hstep(h, tk[j]);
    }
    tk[n] = tok(p);
    const int64_t cap = a.cap;
    u64 *ptab = pair_table(a, b, n), *gtab = gram_table(a, b, n);
    const int64_t ph = (int64_t)(hfinal(hstep(h, tk[n])) & (u64)(cap - 1));
    const int64_t gh = (int64_t)(hfinal(h) & (u64)(cap - 1));
    Window wp, wg;
    load_window(ptab, cap, ph, wp);
    load_window(gtab, cap, gh, wg);
    // pairs end at p, grams at p - 1: the first ends this append can claim
    const int64_t p_fresh = old_len, g_fresh = (int64_t)old_len - 1;
    // both windows are marked before either walk, so their loads are in
    // flight together
    const Marks mp = mark(wp, n + 1, tk, p_fresh), mg = mark(wg, n, tk, g_fresh);
    bool pe, ge;
    int64_t ps = locate(ptab, cap, ph, wp, mp, n + 1, tk, p_fresh, tok, &pe);
    int64_t gs = locate(gtab, cap, gh, wg, mg, n, tk, g_fresh, tok, &ge);
    const u64 pword = kOne | (uint32_t)(p + 1), gword = kOne | (uint32_t)p;

    // the gram: claim or count (the count's return is not needed)
    for (;;) {
        u64 *s = gtab + gs * kSlotWords;
        if (!ge) {
            __hip_atomic_fetch_add(s, kOne, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
            break;
        }
        u64 cur;
        if (claim(s, gword, &cur)) {
            store_key(s, n, tk);
            break;
        }
        gs = after_lost_claim(gtab, cap, gs, cur, n, tk, g_fresh, tok, &ge);
    }
    // the pair: claim (count 1) or count, with the new count returned
    uint32_t count;
    for (;;) {
        u64 *s = ptab + ps * kSlotWords;
        if (!pe) {
            count = (uint32_t)(__hip_atomic_fetch_add(s, kOne, __ATOMIC_RELAXED,
                                                      __HIP_MEMORY_SCOPE_AGENT) >> 32) + 1;
            break;
        }
        u64 cur;
        if (claim(s, pword, &cur)) {
            store_key(s, n + 1, tk);
            count = 1;
            break;
        }
        ps = after_lost_claim(ptab, cap, ps, cur, n + 1, tk, p_fresh, tok, &pe);
    }
    __hip_atomic_fetch_max(gtab + gs * kSlotWords + 1, pack_top(count, tk[n]), __ATOMIC_RELAXED,
                           __HIP_MEMORY_SCOPE_AGENT);
}

// Inserts items i0, i0 + step, ... of one append: item i is position
// old_len + i / 4 and context length 1 + i % 4 (lengths above n_max are
// skipped).
template <typename Tok>
__device__ void insert_items(const NgramArgs &a, int b, int32_t old_len, const Tok &tok,
                             int32_t c, int64_t i0, int64_t step)
{
    const int64_t items = (int64_t)c * a.n_max;
    for (int64_t i = i0; i < items; i += step) {
        const int64_t p = old_len + i / a.n_max;
        const int n = 1 + (int)(i % a.n_max);
        if (p - n >= 0)
            insert_one(a, b, old_len, tok, p, n);
    }
}

struct MemTok {
    AppendView v;
    __device__ __forceinline__ int32_t operator()(int64_t q) const { return v.at(q); }
};

// Tokens q0 .. of the request staged in LDS.
struct LdsTok {
    const int32_t *w;
    int64_t q0;
    __device__ __forceinline__ int32_t operator()(int64_t q) const { return w[q - q0]; }
};
// History tokens during a fused append and draft: the append's LDS window
// from q0 on, the store below it.
struct WindowTok {
    const int32_t *row;
    const int32_t *w;
    int64_t q0;
    __device__ __forceinline__ int32_t operator()(int64_t q) const
    {
        return q >= q0 ? w[q - q0] : row[q];
    }
};
// LDS tokens of a one-workgroup append: its new tokens and the 4 before
// them, which hold every token its inserts read (longer appends read
// memory).
constexpr int kAppendWindow = 1024 + 4;

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
    insert_items(a, b, old_len, MemTok{v}, c, (int64_t)blockIdx.y * blockDim.x + threadIdx.x,
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
    const int64_t q0 = old_len > 4 ? old_len - 4 : 0;
    const int64_t nw = (int64_t)old_len + c - q0;
    const bool staged = nw <= kAppendWindow;
    if (staged) {
        for (int64_t i = threadIdx.x; i < nw; i += blockDim.x)
            win[i] = v.at(q0 + i);
        __syncthreads();
    }
    // the copy first, so that its stores complete under the inserts (which
    // read new tokens from the window or the source row, never from it)
    if (staged)
        insert_items(a, b, old_len, LdsTok{win, q0}, c, threadIdx.x, blockDim.x);
    else
        insert_items(a, b, old_len, MemTok{v}, c, threadIdx.x, blockDim.x);
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

// Thresholds of context length n: the followed count needed (at least 1)
// and the top successor's share in percent.
__device__ __forceinline__ void thresholds(const NgramDraftArgs &d, int n, int64_t *need,
                                           int64_t *pct)
{
    const int32_t c = by_length(n, d.min_count[0], d.min_count[1], d.min_count[2],
                                d.min_count[3]);
    *need = c > 1 ? c : 1;
    *pct = by_length(n, d.min_percent[0], d.min_percent[1], d.min_percent[2], d.min_percent[3]);
}

__device__ __forceinline__ int32_t pick4(int m, int32_t t0, int32_t t1, int32_t t2, int32_t t3)
{
    return m == 0 ? t0 : m == 1 ? t1 : m == 2 ? t2 : t3;
}

// Bits 0, 4, 8, ..., 60 of x, packed into bits 0..15.
__device__ __forceinline__ uint32_t every4th(u64 x)
{
    x &= 0x1111111111111111ull;
    x = (x | (x >> 3)) & 0x0303030303030303ull;
    x = (x | (x >> 6)) & 0x000f000f000f000full;
    x = (x | (x >> 12)) & 0x000000ff000000ffull;
    x = (x | (x >> 24)) & 0xffffull;
    return (uint32_t)x;
}

__device__ __forceinline__ bool key_is(ulonglong2 key, int n, int32_t c0, int32_t c1, int32_t c2,
                                       int32_t c3)
{
    return (int32_t)(uint32_t)key.x == c0 && (n < 2 || (int32_t)(key.x >> 32) == c1) &&
           (n < 3 || (int32_t)(uint32_t)key.y == c2) && (n < 4 || (int32_t)(key.y >> 32) == c3);
}

// One wavefront per request; the draft is built token by token.
//
// An exact round: lanes 16(n - 1) .. 16n - 1 look up context length n, lane
// w of the group reading slot w of the current 16-slot window of the probe
// sequence. The first slot in probe order that is empty or holds the
// context's tokens ends the group's search; the longest length that passes
// its thresholds proposes the token.
//
// Verification along an occurrence: when a round's token came from the
// longest length (n_max) and the occurrence that created the chosen slot (its
// stored end) was followed by that same token, the following history tokens
// y_1, y_2, ... are taken as the hypothesis for the next draft tokens. One
// load fetches them; then lanes 4i .. 4i + 3 read the first 8 slots of the
// probe sequence of round i's n_max-gram (the context the stream has if the
// hypothesis held for the i tokens before it), 16 rounds at once. The
// rounds are then taken in order while each one's n_max-gram is found in
// those slots and passes its thresholds (so the longest length proposes the
// round's token, as an exact round would decide); the walk stops at a draft
// token that differs from the hypothesis (that token is kept: its own
// context was right) or at a round the longest length does not decide, and
// exact rounds continue from there.
// A slot's words 0, 1 (head) and 2, 3 (key). COHERENT reads them with
// agent-scope atomic loads, past this compute unit's cache (after this
// kernel's own inserts, whose window loads may have cached older copies).
template <bool COHERENT>
__device__ __forceinline__ void load_slot(const u64 *sp, ulonglong2 &head, ulonglong2 &key)
{
    if (COHERENT) {
        head.x = __hip_atomic_load(sp, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        head.y = __hip_atomic_load(sp + 1, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        key.x = __hip_atomic_load(sp + 2, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        key.y = __hip_atomic_load(sp + 3, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    } else {
        head = *(const ulonglong2 *)sp;
        key = *(const ulonglong2 *)(sp + 2);
    }
}

// The draft of request b, whose history has length L and ends with tokens
// t0..t3 (oldest first), by one wavefront. tok(q) reads history token q.
template <bool COHERENT, typename Tok>
__device__ void draft_request(const NgramArgs &a, const NgramDraftArgs &d, int b, int lane,
                              int32_t L, const Tok &tok_at, int32_t t0, int32_t t1, int32_t t2,
                              int32_t t3)
{
    // exact rounds: group g looks up length n
    const int g = lane >> 4, w = lane & (kWindow - 1), n = g + 1;
    int64_t need, pct;
    thresholds(d, n, &need, &pct);
    const u64 *tab = n <= a.n_max ? gram_table(a, b, n) : a.grams;
    // verification: lane (si, sj) reads slot sj of round si's probe sequence
    // for length n_max
    const int si = lane / kVerifySlots, sj = lane % kVerifySlots;
    int64_t vneed, vpct;
    thresholds(d, d.n_max, &vneed, &vpct);
    const u64 *vtab = gram_table(a, b, d.n_max);

    int32_t *draft_row = d.out_draft + (int64_t)b * d.k_max;
    int32_t *level_row = d.out_levels ? d.out_levels + (int64_t)b * d.k_max : nullptr;
    int64_t len = L;
    int32_t s = 0;
    bool ended = false;
    auto emit = [&](int32_t tok, int level) {
        if (lane == 0) {
            draft_row[s] = tok;
            if (level_row)
                level_row[s] = level;
        }
        t0 = t1;
        t1 = t2;
        t2 = t3;
        t3 = tok;
        ++len;
        ++s;
    };
    while (s < d.k_max && !ended) {
        // ---- an exact round ----
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
                const u64 *sp = tab + ((home + it + w) & (a.cap - 1)) * kSlotWords;
                ulonglong2 head, key;
                load_slot<COHERENT>(sp, head, key);
                w0 = head.x;
                w1 = head.y;
                const bool empty = (uint32_t)w0 == 0;
                hit = !empty && key_is(key, n, c0, c1, c2, t3);
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
        if (leaders == 0) {
            ended = true;
            break;
        }
        const int best = 63 - __builtin_clzll(leaders);  // the longest passing length
        const int level = best / kWindow + 1;
        const int32_t tok = top_token(readlane64(top, best));
        const int64_t ref = (int64_t)(uint32_t)readlane64(word, best);  // claim's successor
        emit(tok, level);
        if (s >= d.k_max || level != d.n_max)
            continue;

        // ---- verification along the occurrence that claimed the slot ----
        const int32_t y = ref + lane < L ? tok_at(ref + lane) : 0;
        if (__builtin_amdgcn_readlane(y, 0) != tok)
            continue;
        // round i (draft token s + i) assumes y_1 .. y_i, so it needs ref + i < L
        int64_t span = (int64_t)L - ref;
        if (span > d.k_max - s)
            span = d.k_max - s;
        if (span > kVerifyRounds)
            span = kVerifyRounds;
        // round si's context of length n_max: the last n_max of t0..t3, y_1..y_si
        const int nm = d.n_max;
        int32_t v[4];
        for (int j = 0; j < 4; ++j) {
            const int m = 4 + si - nm + j;
            const int32_t from_y = __shfl(y, m - 3 > 0 ? m - 3 : 0);
            v[j] = m < 4 ? pick4(m < 0 ? 0 : m, t0, t1, t2, t3) : from_y;
        }
        u64 vh = hstep(kHashSeed, v[0]);
        for (int j = 1; j < 4; ++j)
            if (j < nm)
                vh = hstep(vh, v[j]);
        const bool von = si < span;
        // lane sj reads slots sj and sj + 4 of the round's probe sequence
        bool vstop[2] = {false, false}, vhit[2] = {false, false};
        u64 vw0[2] = {0, 0}, vw1[2] = {0, 0};
        if (von) {
            ulonglong2 head[2], key[2];
            for (int l = 0; l < 2; ++l) {
                const int64_t vslot =
                    (int64_t)((hfinal(vh) + (u64)(sj + l * kVerifySlots)) & (u64)(a.cap - 1));
                load_slot<COHERENT>(vtab + vslot * kSlotWords, head[l], key[l]);
            }
            for (int l = 0; l < 2; ++l) {
                vw0[l] = head[l].x;
                vw1[l] = head[l].y;
                const bool empty = (uint32_t)vw0[l] == 0;
                vhit[l] = !empty && key_is(key[l], nm, v[0], v[1], v[2], v[3]);
                vstop[l] = empty || vhit[l];
            }
        }
        // the round's first stopping slot in probe order: its first 4 slots,
        // then the next 4
        const uint32_t near = (uint32_t)(__ballot(vstop[0]) >> (si * kVerifySlots)) & 0xfu;
        const uint32_t far = (uint32_t)(__ballot(vstop[1]) >> (si * kVerifySlots)) & 0xfu;
        const int layer = near ? 0 : 1;
        const uint32_t vmine = near ? near : far;
        const int vsrc = si * kVerifySlots + (vmine ? __builtin_ctz(vmine) : 0);
        const bool h0 = __shfl((int)vhit[0], vsrc) != 0, h1 = __shfl((int)vhit[1], vsrc) != 0;
        const u64 a0 = __shfl(vw0[0], vsrc), a1 = __shfl(vw0[1], vsrc);
        const u64 b0 = __shfl(vw1[0], vsrc), b1 = __shfl(vw1[1], vsrc);
        const bool rhit = layer ? h1 : h0;
        const u64 rw0 = layer ? a1 : a0, rw1 = layer ? b1 : b0;
        // round si is decided here when its n_max-gram is found and passes;
        // it keeps the hypothesis when its token is y_(si + 1)
        const int64_t rcount = (int64_t)(rw0 >> 32), rtopc = (int64_t)(rw1 >> 32);
        const bool rpass = von && vmine && rhit && len + si >= nm && rcount >= vneed &&
                           100 * rtopc >= vpct * rcount;
        const int32_t vt = top_token(rw1);
        const int32_t hyp = __shfl(y, si + 1);
        const uint32_t dec = every4th(__ballot(rpass && sj == 0));
        const uint32_t keep = every4th(__ballot(rpass && sj == 0 && vt == hyp));
        // rounds 0 .. c - 1 are decided and keep the hypothesis; round c is
        // taken too when it is decided (its own context was right)
        const int c = __builtin_ctz(~keep);
        const int taken = c + (int)((dec >> c) & 1u);
        if (taken > 0) {
            const int32_t mine = __shfl(vt, lane < kVerifyRounds ? kVerifySlots * lane : 0);
            if (lane < taken) {
                draft_row[s + lane] = mine;
                if (level_row)
                    level_row[s + lane] = nm;
            }
            // the stream's last 4 tokens: the old ones, then the taken ones
            const int32_t u0 = taken >= 4 ? __builtin_amdgcn_readlane(mine, taken - 4)
                               : pick4(taken, t0, t1, t2, t3);
            const int32_t u1 = taken >= 3 ? __builtin_amdgcn_readlane(mine, taken - 3)
                               : pick4(taken + 1, t0, t1, t2, t3);
            const int32_t u2 = taken >= 2 ? __builtin_amdgcn_readlane(mine, taken - 2)
                               : pick4(taken + 2, t0, t1, t2, t3);
            t3 = __builtin_amdgcn_readlane(mine, taken - 1);
            t0 = u0;
            t1 = u1;
            t2 = u2;
            len += taken;
            s += taken;
        }
    }
    for (int32_t i = s + lane; i < d.k_max; i += kWave) {
        draft_row[i] = -1;
        if (level_row)
            level_row[i] = 0;
    }
    if (lane == 0)
        d.out_len[b] = s;
}

struct RowTok {
    const int32_t *row;
    __device__ __forceinline__ int32_t operator()(int64_t q) const { return row[q]; }
};

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
    draft_request<false>(a, d, b, lane, L, RowTok{row}, __builtin_amdgcn_readlane(tl, 0),
                         __builtin_amdgcn_readlane(tl, 1), __builtin_amdgcn_readlane(tl, 2),
                         __builtin_amdgcn_readlane(tl, 3));
}

// One decode step of request b in one workgroup: the append (counts, copy,
// new length) as pld_append_ngram, then wave 0 drafts from the cache as
// pld_ngram_draft, reading slots past this compute unit's cache. An append
// that is rejected leaves the row as it was, and the row is drafted as it
// stands.
__global__ __launch_bounds__(256) void pld_append_draft_ngram(NgramArgs a, const int32_t *tokens,
                                                              int64_t tokens_stride,
                                                              const int32_t *counts,
                                                              NgramDraftArgs d)
{
    __shared__ int s_ok;
    __shared__ int32_t win[kAppendWindow];
    const int b = blockIdx.x;
    int32_t old_len = a.lengths[b];
    const int32_t c = counts[b];
    if (threadIdx.x == 0) {
        const bool ok = append_ok(a, old_len, c);
        if (!ok)
            atomicOr(a.err, c < 0 ? kErrAppendNegative : kErrAppendCapacity);
        s_ok = ok;
    }
    __syncthreads();
    int32_t *row = a.store + (int64_t)b * a.pitch;
    const int32_t *src = tokens + (int64_t)b * tokens_stride;
    const bool ok = s_ok != 0;
    const int32_t add = ok ? c : 0;
    if (old_len < 0 || old_len > a.max_len)
        old_len = 0;  // a corrupt length: the append was rejected above
    const int32_t L = old_len + add;
    AppendView v{row, src, old_len};
    const int64_t q0 = old_len > 4 ? old_len - 4 : 0;
    const int64_t nw = (int64_t)L - q0;
    const bool staged = nw <= kAppendWindow;
    if (staged) {
        for (int64_t i = threadIdx.x; i < nw; i += blockDim.x)
            win[i] = v.at(q0 + i);
        __syncthreads();
    }
    if (add > 0) {
        if (staged)
            insert_items(a, b, old_len, LdsTok{win, q0}, add, threadIdx.x, blockDim.x);
        else
            insert_items(a, b, old_len, MemTok{v}, add, threadIdx.x, blockDim.x);
        for (int32_t t = threadIdx.x; t < add; t += blockDim.x)
            row[old_len + t] = src[t];
    }
    // the draft below reads what these inserts wrote, past this compute
    // unit's cache: every thread's stores and atomics complete before the
    // barrier
    __builtin_amdgcn_s_waitcnt(0);
    __syncthreads();
    if (threadIdx.x >= kWave)
        return;
    const int lane = threadIdx.x;
    if (lane == 0 && add > 0)
        a.lengths[b] = L;
    // the draft reads history tokens through the same reader: a position at
    // or past the old length is in the window, or in the source row
    int32_t tl = 0;
    if (lane < 4 && L - 4 + lane >= 0)
        tl = staged ? win[L - 4 + lane - q0] : row[L - 4 + lane];
    const int32_t t0 = __builtin_amdgcn_readlane(tl, 0), t1 = __builtin_amdgcn_readlane(tl, 1);
    const int32_t t2 = __builtin_amdgcn_readlane(tl, 2), t3 = __builtin_amdgcn_readlane(tl, 3);
    if (staged)
        draft_request<true>(a, d, b, lane, L, WindowTok{row, win, q0}, t0, t1, t2, t3);
    else
        draft_request<true>(a, d, b, lane, L, RowTok{row}, t0, t1, t2, t3);
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

hipError_t launch_append_draft_ngram(const NgramArgs &a, const int32_t *tokens,
                                     int64_t tokens_stride, const int32_t *counts,
                                     const NgramDraftArgs &d, hipStream_t s)
{
    if (d.batch <= 0)
        return hipSuccess;
    hipLaunchKernelGGL(pld_append_draft_ngram, dim3((unsigned)d.batch), dim3(256), 0, s, a, tokens,
                       tokens_stride, counts, d);
    return hipGetLastError();
}

hipError_t launch_ngram_clear(const NgramArgs &a, int32_t batch, hipStream_t s)
{
    const int64_t slots = (int64_t)batch * a.n_max * a.cap;
    hipError_t e = fill_zero(a.grams, slots * kSlotWords, s);
    if (e == hipSuccess)
        e = fill_zero(a.pairs, slots * kSlotWords, s);
    return e;
}

}  // namespace pld
