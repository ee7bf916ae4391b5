/*
 * libpld: batched prompt-lookup (n-gram) drafting on AMD Instinct MI355X.
 *
 * The operation (HyperQwen lookup-drafting page, "lookup drafting: the
 * three-step principle", step 1): for every request of a batch, find the
 * longest suffix of its own int32 token history, between n_min and n_max
 * tokens, that occurred earlier in that history (the earlier occurrence may
 * overlap the suffix); among occurrences of that length take the most recent;
 * the tokens that followed it, at most k_max of them (the verify-block bound
 * of step 2 on the same page, and of section 4 of the Strata prompt-lookup
 * page), are the draft.
 *
 * Exactly, for a history h[0..L) (this is the contract the kernels meet):
 *   S = { (m, j) : n_min <= m <= n_max, 0 <= j, j + m <= L - 1,
 *                  h[j .. j+m) == h[L-m .. L) }
 *   S empty     -> draft_len = 0, match_len = 0, start = -1, row all -1
 *   otherwise   -> (m, j) = maximum of S by m first, then j;
 *                  d = min(k_max, L - (j + m));
 *                  row[0..d) = h[j+m .. j+m+d), row[d..k_max) = -1;
 *                  draft_len = d, match_len = m, start = j.
 * The suffix never matches itself (j = L - m is excluded) and an occurrence
 * is always followed by at least one token. Tokens are compared as raw 32-bit
 * integers. Matches longer than n_max are reported as n_max.
 *
 * Conventions for every entry point:
 *  - Pointers named "device" are HIP device memory of the device that was
 *    current when the context was created; call with that device current.
 *  - Calls taking a stream enqueue work on it and return without waiting;
 *    results are ready when the stream's work up to that point is done.
 *    Caller buffers must stay valid until then.
 *  - Host-side argument checks run before anything is enqueued; a failed
 *    check returns PLD_EINVAL and enqueues nothing. pld_last_error() then
 *    names the argument.
 *  - Problems only visible on the device (a bad per-request length or row
 *    pointer, an append past capacity) do not stop the call: the affected
 *    request is written as "no match" (or its append is dropped) and a sticky
 *    flag is set, which pld_sync() reports and clears. Nothing is ever cut
 *    to fit: the Strata engine review (chapter 05, on using the engine)
 *    reports a context longer than the model's limit as an error instead of
 *    truncating it, and a history or append past max_len is handled the
 *    same way here.
 *  - Only the pld_create* calls allocate. No other entry point allocates
 *    memory (pld_draft_batch_noalloc needs no context at all).
 *  - A context must not be used from two host threads at once, and two
 *    draft or append calls on one context must not overlap in time on the
 *    device (they share the context's per-request reduction slots): issue them
 *    on one stream, or order the streams.
 */
#ifndef PLD_H_
#define PLD_H_

#include <stdint.h>

#include <hip/hip_runtime_api.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef struct pld_ctx pld_ctx; /* opaque; owned by the library */

typedef enum pld_status {
    PLD_OK = 0,
    PLD_EINVAL = 1,    /* bad argument, or bad per-request input seen on device */
    PLD_ENOMEM = 2,    /* device allocation failed in pld_create */
    PLD_EHIP = 3,      /* a HIP runtime call or kernel launch failed */
    PLD_ECAPACITY = 4  /* a history longer than max_len, or an append past it */
} pld_status;

/* Largest n_max accepted (the kernels keep n_max - 1 tokens of left context
   per tile). The page's own setting is n_max = 12. */
#define PLD_N_MAX_LIMIT 64

/*
 * Create a context for batches of up to max_batch requests whose histories
 * are at most max_len tokens (1 <= max_len <= 2^31 - 1: a position must fit
 * the low 32 bits of the packed key the scan reduces).
 *
 * The context holds 256 bytes of reduction state per request, a sticky error
 * word and, when own_store != 0, a history store of max_batch rows of
 * max_len tokens (row pitch rounded up to 64 tokens) with a length per row,
 * all lengths starting at 0 (fed by pld_append; the Strata prompt-lookup page,
 * section 4, keeps its history index growing by O(1) appends).
 *
 * out:    receives the context (unchanged on failure).
 * stream: the context's memory is cleared by work enqueued on this stream
 *         (NULL: the null stream); the call waits for that work.
 * Errors: PLD_EINVAL (bad sizes, null out; max_len >= 2^31), PLD_ENOMEM,
 * PLD_EHIP. The only entry points that allocate are the pld_create* calls.
 */
pld_status pld_create(pld_ctx **out, int32_t max_batch, int64_t max_len,
                      int32_t own_store, hipStream_t stream);

/*
 * pld_create with a store (own_store = 1) and an incremental n-gram index
 * over it, for lengths n_min..n_max (1 <= n_min <= n_max <= PLD_N_MAX_LIMIT).
 *
 * The Strata prompt-lookup page (section 4) keeps an index from n-grams to
 * history positions that grows by O(1) work per appended token. Here, for
 * each request and each indexed length n, an open-addressed table maps every
 * n-gram of the history to the end of its most recent occurrence that can be
 * drafted from. pld_append keeps it current; pld_draft_store answers from it
 * with exactly the results pld_draft_batch gives on the same store.
 * Memory: max_batch * (n_max - n_min + 1) tables of 8-byte slots, each table
 * a power of two >= 2 * max_len slots (576 MB for 64 requests of 49,152
 * tokens and lengths 4..12).
 * Errors: as pld_create (max_len and stream as there); PLD_EINVAL for a
 * bad length range.
 */
pld_status pld_create_indexed(pld_ctx **out, int32_t max_batch, int64_t max_len,
                              int32_t n_min, int32_t n_max, hipStream_t stream);

/* Free everything the context owns. Waits for the device to finish work
   first. NULL is a no-op. */
pld_status pld_destroy(pld_ctx *ctx);

/*
 * Tuning controls. They never change results, only how the scan is split:
 *  tile_tokens: candidate positions per workgroup, one of 256, 1024, 2048,
 *               4096, 8192, 16384; -1 restores the default, chosen per call:
 *               4096 when max_len fits one tile of 4096, else the largest of
 *               4096, 2048 and 1024 that gives the scan at least 1024
 *               workgroups (batch x tiles of max_len); 0 keeps the current
 *               value.
 *  fused_gather: 1 (default) lets the last workgroup of each request emit
 *               its draft inside the scan kernel; 0 emits drafts with a
 *               second kernel; -1 keeps the current value.
 * Errors: PLD_EINVAL for other values.
 */
pld_status pld_configure(pld_ctx *ctx, int32_t tile_tokens, int32_t fused_gather);

/*
 * The scan's tile for a draft call of `batch` requests on this context: the
 * candidate positions each workgroup covers, as pld_configure fixed it or as
 * the automatic rule picks it. Reporting only; the tile never changes
 * results.
 *  tile_tokens: host out-param.
 * Errors: PLD_EINVAL (null ctx or out, batch outside [1, max_batch]).
 */
pld_status pld_scan_tile(pld_ctx *ctx, int32_t batch, int32_t *tile_tokens);

/*
 * Streaming append into the context's own store (own_store != 0).
 *
 * The Strata prompt-lookup page (section 4, prompt lookup) keeps the
 * history it drafts from current by appending each accepted token in O(1);
 * here an append is O(count) work for the appended tokens only, whatever
 * the row's length, and never re-reads the stored history.
 *
 * For b < batch: tokens[b * tokens_stride + t] for t < counts[b] are appended
 * to row b, whose length grows by counts[b].
 *  tokens: device int32, row b at tokens + b * tokens_stride;
 *          tokens_stride >= 0 tokens.
 *  counts: device int32[batch], each 0 <= counts[b].
 * A row whose append would pass max_len, or whose count is negative, is left
 * unchanged and sets the sticky flag (PLD_ECAPACITY / PLD_EINVAL at
 * pld_sync); so is a row whose stored length is outside [0, max_len] (the
 * length array is reachable through pld_histories), as PLD_ECAPACITY.
 * batch == 0 is a no-op. With an index (pld_create_indexed) the
 * n-grams that the append makes draftable are inserted first, in a second
 * kernel on the same stream. With a successor-count cache
 * (pld_create_ngram) the appended tokens' n-grams are counted in the same
 * launch as the copy when 0 < tokens_stride <= 1024, otherwise in a kernel
 * before it.
 * Errors: PLD_EINVAL (no store, batch outside [0, max_batch], null pointers,
 * negative stride), PLD_EHIP.
 */
pld_status pld_append(pld_ctx *ctx, const int32_t *tokens, int64_t tokens_stride,
                      const int32_t *counts, int32_t batch, hipStream_t stream);

/*
 * Device views of the context's store, to pass to pld_draft_batch (the
 * HyperQwen page, step 1, drafts each request from its own history; these
 * are those histories as the appends left them):
 *  *histories: device array of max_batch row pointers (host out-param);
 *  *lengths:   device int32[max_batch] current row lengths (host out-param).
 * Both stay owned by the context. Errors: PLD_EINVAL (no store, null out).
 */
pld_status pld_histories(pld_ctx *ctx, const int32_t *const **histories,
                           const int32_t **lengths);

/* Set every store row's length to 0, and empty the n-gram index if there is
   one (stream-ordered). Errors: PLD_EINVAL (no store), PLD_EHIP. */
pld_status pld_store_reset(pld_ctx *ctx, hipStream_t stream);

/*
 * Draft every request of a batch (the operation stated at the top).
 *
 *  histories: device array of batch row pointers; row b holds lengths[b]
 *             int32 tokens, 4-byte aligned (any offset; 16-byte alignment is
 *             fastest). Rows may alias each other and the store.
 *  lengths:   device int32[batch], 0 <= lengths[b] <= max_len.
 *  batch:     0 <= batch <= max_batch; 0 is a no-op.
 *  n_min, n_max: 1 <= n_min <= n_max <= PLD_N_MAX_LIMIT.
 *  k_max:     >= 1.
 *  out_draft: device int32[batch * k_max], row-major, row b at b * k_max.
 *  out_len:   device int32[batch], draft lengths.
 *  out_match: device int32[batch], match lengths (0 = no match).
 * A request whose length is outside [0, max_len], or whose row pointer is
 * null (with a nonzero length) or not 4-byte aligned, is written as no match
 * and sets the sticky flag.
 * Errors: PLD_EINVAL, PLD_EHIP.
 */
pld_status pld_draft_batch(pld_ctx *ctx, const int32_t *const *histories,
                           const int32_t *lengths, int32_t batch, int32_t n_min,
                           int32_t n_max, int32_t k_max, int32_t *out_draft,
                           int32_t *out_len, int32_t *out_match,
                           hipStream_t stream);

/* pld_draft_batch plus out_pos: device int32[batch], the occurrence start j
   (-1 when no match). */
pld_status pld_draft_batch_pos(pld_ctx *ctx, const int32_t *const *histories,
                               const int32_t *lengths, int32_t batch,
                               int32_t n_min, int32_t n_max, int32_t k_max,
                               int32_t *out_draft, int32_t *out_len,
                               int32_t *out_match, int32_t *out_pos,
                               hipStream_t stream);

/*
 * For callers that cannot allocate (code under HIP graph capture, tight
 * serving loops, harnesses that forbid allocation): pld_draft_batch_pos
 * without a context. The per-request reduction state lives in a static
 * device array of the library instead of a context: 256 bytes for each of
 * at most PLD_NOALLOC_MAX_BATCH requests (1 MiB per GPU, held from the
 * library's load until the process ends). This call never allocates; its
 * first call on a device looks the array up and clears it (a fill kernel on
 * `stream`). Every call on a GPU shares that GPU's array, which the kernels
 * leave cleared after each call: calls that overlap in time on one GPU
 * (other streams, other host threads) race and must be ordered by the
 * caller. The tile is chosen as pld_configure's automatic rule does, with the
 * fused gather.
 *
 *  max_len:  bound on every length, 1 <= max_len <= 2^31 - 1 (as in
 *            pld_create); it sizes the launch.
 *  batch:    0 <= batch <= PLD_NOALLOC_MAX_BATCH; larger batches are refused.
 *  out_pos:  device int32[batch] (not NULL).
 *  out_err:  device uint32 or NULL: bits are OR-ed into it (never cleared
 *            by the call) when a request's length lies outside [0, max_len]
 *            or its row pointer is null or misaligned; such requests are
 *            written as no match. NULL drops the report.
 *  Other arguments and results exactly as in pld_draft_batch_pos.
 * Errors: PLD_EINVAL (bad sizes or pointers, batch above the maximum),
 * PLD_EHIP.
 */
#define PLD_NOALLOC_MAX_BATCH 4096
pld_status pld_draft_batch_noalloc(const int32_t *const *histories, const int32_t *lengths,
                                   int32_t batch, int64_t max_len, int32_t n_min, int32_t n_max,
                                   int32_t k_max, int32_t *out_draft, int32_t *out_len,
                                   int32_t *out_match, int32_t *out_pos, uint32_t *out_err,
                                   hipStream_t stream);

/*
 * pld_draft_batch for histories laid out at a fixed stride: row b starts at
 * base + b * stride (a padded [batch, stride] int32 buffer, such as the
 * context's own store). Tiles that lie inside every row by the caller's
 * bound min_len start reading before their row's length is known, which
 * shortens the call; pass min_len = 0 when no bound is known.
 *
 *  base:     device int32, 16-byte aligned.
 *  stride:   tokens between row starts, a multiple of 4, >= 4.
 *  lengths:  device int32[batch], min_len <= lengths[b] <= min(max_len, stride).
 *  min_len:  0 <= min_len <= min(max_len, stride).
 *  out_pos:  device int32[batch] or NULL (as in pld_draft_batch_pos).
 *  Other arguments as in pld_draft_batch. A request whose length is outside
 *  [min_len, min(max_len, stride)] is written as no match and sets the
 *  sticky flag (PLD_EINVAL below min_len, PLD_ECAPACITY above). Only bytes
 *  inside rows' [0, stride) spans are read.
 * Errors: PLD_EINVAL, PLD_EHIP.
 */
pld_status pld_draft_batch_strided(pld_ctx *ctx, const int32_t *base, int64_t stride,
                                   const int32_t *lengths, int32_t min_len, int32_t batch,
                                   int32_t n_min, int32_t n_max, int32_t k_max,
                                   int32_t *out_draft, int32_t *out_len, int32_t *out_match,
                                   int32_t *out_pos, hipStream_t stream);

/*
 * Fingerprint bits the index keeps (default 32). Two n-grams whose hashes
 * agree in these bits share a slot; a query that lands on such a shared slot
 * is answered by an exact scan of that request's history, so results never
 * change, only speed. Fewer bits make that path common, for testing it.
 * Takes effect for inserts and queries issued afterwards; change it only on
 * an empty index (after pld_store_reset) so that all entries agree.
 * Errors: PLD_EINVAL (no index, bits outside [0, 32]).
 */
pld_status pld_index_fingerprint_bits(pld_ctx *ctx, int32_t bits);

/*
 * pld_draft_batch over the first `batch` rows of the context's store,
 * answered from the n-gram index instead of a scan of the histories: one
 * probe per length n in [n_min, n_max], in parallel; the longest hit is
 * confirmed against the stored tokens (a shared-fingerprint slot that does
 * not confirm sends that request to an exact scan of its row). Results are
 * identical to pld_draft_batch_pos on pld_histories (same outputs, same
 * padding).
 *  n_min, n_max: within the indexed lengths of pld_create_indexed.
 *  out_pos: device int32[batch] or NULL.
 * Errors: PLD_EINVAL (no index, lengths outside it, bad sizes), PLD_EHIP.
 */
pld_status pld_draft_store(pld_ctx *ctx, int32_t batch, int32_t n_min, int32_t n_max,
                           int32_t k_max, int32_t *out_draft, int32_t *out_len,
                           int32_t *out_match, int32_t *out_pos, hipStream_t stream);

/*
 * One decode step on the context's store: pld_append (tokens, tokens_stride,
 * counts, batch as there), then the draft of the first `batch` rows of the
 * new histories (n_min, n_max, k_max and outputs as in pld_draft_store or,
 * without an index, pld_draft_batch_pos on pld_histories; out_pos may be
 * NULL). On an indexed context n_min, n_max must lie inside the indexed
 * lengths. With 0 < tokens_stride <= 1024 both steps run in one launch:
 * on an indexed context one workgroup per request; on a context with a
 * plain store (no index, no successor-count cache) and the fused gather
 * (the default of pld_configure), inside the scan's own launch, which reads
 * the appended positions from `tokens`. Otherwise they run as two calls.
 * Results, the store and the reported errors are the same either way. A
 * rejected append (see pld_append) leaves its row as it was, and that row is
 * drafted as it stands. All arguments are checked before anything is
 * enqueued.
 * Errors: those of pld_append and of the draft call.
 */
pld_status pld_append_draft_store(pld_ctx *ctx, const int32_t *tokens, int64_t tokens_stride,
                                  const int32_t *counts, int32_t batch, int32_t n_min,
                                  int32_t n_max, int32_t k_max, int32_t *out_draft,
                                  int32_t *out_len, int32_t *out_match, int32_t *out_pos,
                                  hipStream_t stream);

/*
 * Draft fusion and long-block scheduling (HyperQwen lookup-drafting page,
 * "lookup drafting: the three-step principle", steps 2 and 3).
 *
 * Before each verify step the lookup draft and a small drafter's proposal
 * are merged into the block of draft positions the target model verifies:
 *  - scheduling (step 3): a long block of positions_long draft positions runs
 *    only while the request is copying: it starts on a step whose lookup
 *    match is >= tail_min with a draft covering all positions_long
 *    positions, when the entry_steps steps before it were near-full
 *    (accepted >= their positions - near_full_slack); it is held sticky
 *    further steps after that condition fails. Otherwise the block has the
 *    drafter's head positions.
 *  - fusion (step 2): head positions 0 .. head-1 hold the drafter's tokens;
 *    the lookup draft replaces them (where it has tokens) when its match is
 *    >= replace_min, or >= agree_min with the drafter's first agree_tokens
 *    tokens equal to the lookup's. In a long block, tail positions
 *    head .. positions_long-1 take the lookup's tokens when its match is
 *    >= tail_min, up to the end of the lookup draft; the block ends at the
 *    first tail position the lookup does not cover.
 * Readings of points the page leaves open: near-full, the run of two, the
 * tail test, the hold re-armed by every entry step, a partial head
 * replacement, a gap ending the block (the same in pld_fuse's contract and
 * the test oracle).
 */
typedef struct pld_fuse_params {
    int32_t head;            /* drafter positions; the page: 7 */
    int32_t positions_long;  /* draft positions of a long block (<= 64); 15 */
    int32_t replace_min;     /* head: match length that replaces outright; 8 */
    int32_t agree_min;       /* head: match length that replaces on agreement; 6 */
    int32_t agree_tokens;    /* head: leading tokens that must agree; 2 */
    int32_t tail_min;        /* tail: match length that fills it; 4 */
    int32_t entry_steps;     /* near-full steps in a row before a long block; 2 */
    int32_t sticky;          /* steps a long block is held; 3 */
    int32_t near_full_slack; /* a near-full step misses at most this many; 1 */
} pld_fuse_params;

/* int32 words of per-request state: long flag, hold left, near-full run,
   draft positions of the previous block. All zero before a request's first
   step (and to restart it). */
#define PLD_FUSE_STATE_WORDS 4
#define PLD_FUSE_MAX_POSITIONS 64

/* The page's values: 7, 15, 8, 6, 2, 4, 2, 3, and slack 1 (a reading).
   Errors: PLD_EINVAL (null). */
pld_status pld_fuse_params_default(pld_fuse_params *params);

/*
 * One fused step for a batch.
 *
 *  params:       host struct; 1 <= head <= positions_long <= 64,
 *                1 <= agree_tokens <= head, replace_min, agree_min,
 *                tail_min >= 1, entry_steps, sticky, near_full_slack >= 0.
 *  lookup:       device int32[batch * lookup_k]: row b holds request b's
 *                lookup draft (pld_draft_batch's out_draft with k_max =
 *                lookup_k >= 1).
 *  lookup_len, lookup_match: device int32[batch]: its draft and match
 *                lengths (out_len, out_match).
 *  drafter:      device int32[batch * head], the drafter's proposals.
 *  accepted:     device int32[batch]: draft tokens the verifier accepted at
 *                the request's previous step (read only when it had one).
 *  state:        device int32[batch * PLD_FUSE_STATE_WORDS], read and
 *                updated; row b belongs to request b.
 *  out_block:    device int32[batch * positions_long]: the fused block, -1
 *                past its draft positions.
 *  out_positions: device int32[batch]: draft positions to verify.
 *  out_src:      device uint64[batch] or NULL: bit t set when block
 *                position t came from the lookup (the positions a sampler
 *                turns into point masses on the proposed token).
 * Device-side input errors (lookup_len outside [0, lookup_k], a negative
 * match, accepted outside [0, previous positions], a state row no step
 * could have written) give that request the drafter's head, reset its
 * state to zero and set the sticky flag (PLD_EINVAL at pld_sync).
 * Errors: PLD_EINVAL (bad params, sizes or null pointers), PLD_EHIP.
 */
pld_status pld_fuse(pld_ctx *ctx, const pld_fuse_params *params, const int32_t *lookup,
                    int32_t lookup_k, const int32_t *lookup_len, const int32_t *lookup_match,
                    const int32_t *drafter, const int32_t *accepted, int32_t *state,
                    int32_t batch, int32_t *out_block, int32_t *out_positions,
                    uint64_t *out_src, hipStream_t stream);

/*
 * pld_draft_batch followed by pld_fuse on its outputs, in one launch: the
 * workgroup that emits a request's lookup draft also fuses it with the
 * drafter's proposal (lookup_k = k_max). Outputs of both calls are written;
 * arguments and errors are those of the two calls.
 */
pld_status pld_draft_fuse_batch(pld_ctx *ctx, const int32_t *const *histories,
                                const int32_t *lengths, int32_t batch, int32_t n_min,
                                int32_t n_max, int32_t k_max, int32_t *out_draft,
                                int32_t *out_len, int32_t *out_match,
                                const pld_fuse_params *params, const int32_t *drafter,
                                const int32_t *accepted, int32_t *state, int32_t *out_block,
                                int32_t *out_positions, uint64_t *out_src, hipStream_t stream);

/*
 * Online cost/benefit controller (Strata prompt-lookup page, section 5).
 *
 * Per request and step it chooses between the lookup draft, the model's own
 * draft layer (MTP) and plain decoding, from running estimates of each
 * one's committed tokens per unit of verify time: the lookup's acceptance
 * in 4 match-length buckets, MTP's acceptance, and each source's round
 * time, all exponential moving averages of measured outcomes. The lookup
 * draft is chosen only when its estimate is at least `margin` times MTP's
 * (the page: 5% better); otherwise MTP when it beats plain decoding, else
 * plain decoding. Readings where the page gives no number or formula:
 * acceptance is accepted / drafted tokens of a round; a round commits its
 * accepted tokens plus one; the moving averages weigh a new measurement by
 * alpha (acceptance) and beta (time); estimates start at prior_accept and
 * prior_time; the buckets start at match lengths 0, bucket_edge[0..2]; ties
 * go to the draft. Arithmetic is IEEE double with each operation rounded on
 * its own, so decisions do not depend on the compiler.
 */
typedef struct pld_control_params {
    double alpha;          /* weight of a new acceptance fraction; 0.1 */
    double beta;           /* weight of a new round time; 0.1 */
    double margin;         /* the lookup needs margin x MTP's rate; the page: 1.05 */
    double prior_accept;   /* first acceptance estimate; 0.5 */
    double prior_time;     /* first round-time estimate, caller's unit; 1.0 */
    int32_t mtp_tokens;    /* MTP draft tokens per round; the page: 3 */
    int32_t bucket_edge[3];/* first match length of buckets 1..3; 6, 8, 12 */
} pld_control_params;

/* doubles of per-request controller state (zeros before the first step) */
#define PLD_CONTROL_STATE_WORDS 11
/* sources */
#define PLD_SOURCE_PLAIN 0
#define PLD_SOURCE_MTP 1
#define PLD_SOURCE_LOOKUP 2

/* The defaults above. Errors: PLD_EINVAL (null). */
pld_status pld_control_params_default(pld_control_params *params);

/*
 * One controller step for a batch: fold in each request's previous round,
 * then choose its source for this round.
 *  accepted:     device int32[batch]: draft tokens the verifier accepted in
 *                the previous round (read when the request had one).
 *  round_time:   device double[batch]: that round's measured time (> 0).
 *  lookup_len, lookup_match: device int32[batch]: this round's lookup draft
 *                (pld_draft_batch's out_len and out_match; 0 = none).
 *  state:        device double[batch * PLD_CONTROL_STATE_WORDS], updated.
 *  out_source:   device int32[batch]: PLD_SOURCE_*.
 *  out_rates:    device double[batch * 3] or NULL: the estimates the choice
 *                used (plain, MTP, lookup; 0 for a missing lookup draft).
 * An outcome out of range (accepted above the round's draft tokens or
 * negative, a time not > 0) or a negative lookup input is not folded in
 * and sets the sticky flag (PLD_EINVAL at pld_sync); the choice is still
 * made.
 * Errors: PLD_EINVAL (bad params, sizes, pointers), PLD_EHIP.
 */
pld_status pld_control(pld_ctx *ctx, const pld_control_params *params, const int32_t *accepted,
                       const double *round_time, const int32_t *lookup_len,
                       const int32_t *lookup_match, double *state, int32_t batch,
                       int32_t *out_source, double *out_rates, hipStream_t stream);

/*
 * Successor-count n-gram drafting (llama.cpp page, the section on what
 * prompt lookup decoding is: its context cache).
 *
 * The drafter keeps statistics of the n-grams of sizes 1..4 of the current
 * token stream and of the tokens that followed them, and builds a draft one
 * token at a time, each token one lookup of the tokens before it, proposing
 * a context's most frequent successor when fixed thresholds pass (the
 * page's example: a 4-gram seen at least once whose most frequent successor
 * holds at least half of its occurrences). Computed per request, for each
 * draft token s < k_max:
 *  - the context of length n is the last n tokens of the history followed
 *    by draft tokens 0..s-1 (drafted tokens are never counted);
 *  - n runs from n_max down to n_min; its statistics are over the history
 *    h[0..L): count = the positions i in [n, L) with h[i-n..i) equal to the
 *    context, and the most frequent h[i] among them (the smaller token, as
 *    a signed integer, on a tie) with `top` occurrences;
 *  - the first n with count >= max(1, min_count[n-1]) and
 *    100 * top >= min_percent[n-1] * count proposes that token;
 *  - the draft ends at the first token no length proposes.
 * Defaults (pld_ngram_params_default): n 1..4, min_count 1 and min_percent
 * 50 for every length (the page gives these for the 4-gram).
 */
#define PLD_NGRAM_MAX_N 4

typedef struct pld_ngram_params {
    int32_t n_min;                        /* shortest context tried, >= 1 */
    int32_t n_max;                        /* longest, <= the context's cache */
    int32_t min_count[PLD_NGRAM_MAX_N];   /* per length n at [n-1], >= 0 */
    int32_t min_percent[PLD_NGRAM_MAX_N]; /* per length n at [n-1], 0..100 */
} pld_ngram_params;

/* Fills *params with the defaults above. Errors: PLD_EINVAL (null). */
pld_status pld_ngram_params_default(pld_ngram_params *params);

/*
 * pld_create with a store (own_store = 1) and a successor-count cache over
 * it for context lengths 1..n_max (1 <= n_max <= PLD_NGRAM_MAX_N).
 * pld_append keeps it current (O(n_max) work per appended token) and
 * pld_store_reset empties it. Per request and length: a table of n-gram
 * slots and one of successor-pair slots, 32 bytes each, each a power of two
 * >= max(16, 2 * max_len) slots (2.15 GB for 64 requests of 49,152 tokens
 * and n_max 4). A context has either this cache or an index, not both.
 * Errors: as pld_create (max_len and stream as there); PLD_EINVAL for n_max
 * out of range.
 */
pld_status pld_create_ngram(pld_ctx **out, int32_t max_batch, int64_t max_len, int32_t n_max,
                            hipStream_t stream);

/*
 * Drafts for the first `batch` rows of the context's store from its
 * successor-count cache, by the rule above. One wavefront per request looks
 * up all lengths of a draft token in one round trip; results are exact
 * (n-grams are compared by their tokens, never by hash alone).
 *  params: host pointer; n_max at most the cache's.
 *  out_draft: device int32[batch * k_max], row-major, -1 past out_len[b].
 *  out_len: device int32[batch], the draft lengths.
 *  out_levels: device int32[batch * k_max] or NULL: the context length
 *              behind each draft token, 0 past out_len[b].
 * Errors: PLD_EINVAL (no cache, bad params, sizes, pointers), PLD_EHIP.
 */
pld_status pld_draft_ngram(pld_ctx *ctx, const pld_ngram_params *params, int32_t batch,
                           int32_t k_max, int32_t *out_draft, int32_t *out_len,
                           int32_t *out_levels, hipStream_t stream);

/*
 * One decode step on a successor-count context: pld_append (tokens,
 * tokens_stride, counts, batch as there), then pld_draft_ngram of the first
 * `batch` rows (params, k_max and outputs as there). With
 * 0 < tokens_stride <= 1024 both steps run in one launch, one workgroup per
 * request (the draft starts from the appended tokens it already holds);
 * otherwise as the two calls. Results are the same either way. A rejected
 * append leaves its row as it was, and that row is drafted as it stands.
 * All arguments are checked before anything is enqueued.
 * Errors: those of pld_append and pld_draft_ngram.
 */
pld_status pld_append_draft_ngram(pld_ctx *ctx, const int32_t *tokens, int64_t tokens_stride,
                                  const int32_t *counts, int32_t batch,
                                  const pld_ngram_params *params, int32_t k_max,
                                  int32_t *out_draft, int32_t *out_len, int32_t *out_levels,
                                  hipStream_t stream);

/*
 * pld_draft_batch and pld_control in one launch: the workgroup that emits a
 * request's lookup draft also runs its controller step, with this call's
 * draft length and match length as the step's lookup draft. Arguments as in
 * pld_draft_batch (no out_pos) and pld_control (no lookup_len,
 * lookup_match: they are out_len, out_match). Results are identical to the
 * two calls in a row.
 * Errors: those of pld_draft_batch and pld_control.
 */
pld_status pld_draft_control_batch(pld_ctx *ctx, const int32_t *const *histories,
                                   const int32_t *lengths, int32_t batch, int32_t n_min,
                                   int32_t n_max, int32_t k_max, int32_t *out_draft,
                                   int32_t *out_len, int32_t *out_match,
                                   const pld_control_params *params, const int32_t *accepted,
                                   const double *round_time, double *state, int32_t *out_source,
                                   double *out_rates, hipStream_t stream);

/*
 * Wait for the device (the given stream and every other stream), then
 * report and clear the sticky device-side flag. The flag exists so that a
 * bad request is reported and never silently cut short (the Strata engine
 * review, chapter 05: an over-long context is an error, not a truncation).
 * Statuses:
 * PLD_OK when clear; PLD_ECAPACITY when a history exceeded max_len (or its
 * row's stride) or an append overflowed; PLD_EINVAL when a length or count
 * was negative, a length was below a strided call's min_len, a row pointer
 * was null or misaligned, pld_fuse saw inconsistent per-request inputs, or
 * pld_control an outcome out of range (capacity wins when both are set).
 * Errors: PLD_EINVAL (null ctx), PLD_EHIP.
 */
pld_status pld_sync(pld_ctx *ctx, hipStream_t stream);

/* Static description of a status code. Never NULL. */
const char *pld_strerror(pld_status status);

/* Details of the last failed call on this host thread ("" if none). */
const char *pld_last_error(void);

#ifdef __cplusplus
}
#endif

#endif /* PLD_H_ */
