/*
 * Draft fusion and long-block scheduling oracle.
 *
 * TEST INFRASTRUCTURE ONLY. The test suite, the package's smoke check and the
 * bench's CPU-baseline leg are the only code that may load this library. The
 * HIP library never links, loads or calls it, and the two share no source,
 * header, table or helper: this file includes nothing but libc headers.
 *
 * What is computed (HyperQwen lookup-drafting page, "lookup drafting: the
 * three-step principle", steps 2 and 3). Before each verify step of one
 * request, the lookup draft (step 1) and the small drafter's proposal are
 * merged into the block of draft positions the target model verifies:
 *
 *  Step 3, scheduling. Extra verify positions cost attention time, so the long
 *  block (positions_long draft positions, 15 on the page) runs only while the
 *  request is copying; otherwise the block has the drafter's `head` positions
 *  (7 on the page). The long block starts when the lookup can fill every
 *  tail position and the previous steps were near-full, two in a row on the
 *  page (one saturated step happens by chance in ordinary text). Once on, it
 *  is kept for `sticky` further steps (3 on the page) after that condition
 *  fails, because the signal drops out briefly for incidental reasons.
 *
 *  Step 2, fusion (the lookup never overwrites blindly). Head positions
 *  (0 .. head-1) already hold drafter tokens: the lookup's tokens replace
 *  them only when its match is at least replace_min tokens (8), or at least
 *  agree_min tokens (6) and the drafter's first agree_tokens (2) tokens equal
 *  the lookup's, two independent sources agreeing. Tail positions
 *  (head .. positions_long-1) have no other proposal; in a long block the
 *  lookup fills them whenever its match is at least tail_min tokens (4).
 *
 * Written in that order for one request and one step: update the run of
 * near-full steps with the previous step's result, decide the block size,
 * then fill the head, then the tail.
 *
 * Readings where the page is silent (each one a choice of the plainest form):
 *  - "near-full": a step is near-full when the verifier accepted at least
 *    (its block's draft positions - near_full_slack) tokens, slack 1;
 *  - "two in a row": the two steps before this one were near-full
 *    (entry_steps = 2); the first step of a request has no history;
 *  - "can fill the tail": match >= tail_min and the lookup draft covers
 *    every tail position (draft length >= positions_long);
 *  - the sticky hold is re-armed to `sticky` steps on every step whose entry
 *    condition holds, and counts down on each step that is long only by
 *    the hold;
 *  - a replaced head takes the lookup token at each head position the
 *    lookup draft covers and keeps the drafter's token after it;
 *  - a tail position the lookup does not cover ends the block there (a
 *    verify block has no gaps); the tail is filled position by position
 *    from the lookup draft even when the head kept the drafter's tokens;
 *  - block slots past the block's draft positions hold -1;
 *  - the block size of a step is its number of filled draft positions, and
 *    that is what the next step's near-full test compares against.
 *
 * Parity status: pinned (hand-derived cases of every head and tail rule, a
 * hand-derived multi-step schedule trace, invariants over random inputs,
 * special cases that reduce to drafter-only and lookup-only drafting, and
 * planted-mistake mutants that the pins reject).
 */

#include <stddef.h>
#include <stdint.h>

#define FUSE_ORACLE_OK 0
#define FUSE_ORACLE_EINVAL 1

/* Parameters, in the order the page states them. */
typedef struct fuse_oracle_params {
    int32_t head;            /* drafter positions (7) */
    int32_t positions_long;  /* draft positions of a long block (15) */
    int32_t replace_min;     /* head: match length that replaces outright (8) */
    int32_t agree_min;       /* head: match length that replaces on agreement (6) */
    int32_t agree_tokens;    /* head: leading tokens that must agree (2) */
    int32_t tail_min;        /* tail: match length that fills it (4) */
    int32_t entry_steps;     /* near-full steps in a row before a long block (2) */
    int32_t sticky;          /* steps a long block is held after its condition fails (3) */
    int32_t near_full_slack; /* a near-full step misses at most this many (1) */
} fuse_oracle_params;

/* Per-request state carried from step to step; all zero before the first. */
enum { ST_LONG = 0, ST_HOLD = 1, ST_STREAK = 2, ST_PREV_POSITIONS = 3, ST_WORDS = 4 };

static int params_ok(const fuse_oracle_params *p)
{
    return p->head >= 1 && p->positions_long >= p->head && p->positions_long <= 64 &&
           p->replace_min >= 1 && p->agree_min >= 1 && p->agree_tokens >= 1 &&
           p->agree_tokens <= p->head && p->tail_min >= 1 && p->entry_steps >= 0 &&
           p->sticky >= 0 && p->near_full_slack >= 0;
}

/*
 * One request, one step.
 *  lookup[0..lookup_k): the lookup draft row, of which the first d tokens are
 *      the draft (d <= lookup_k), with match length m (0 = no match);
 *  drafter[0..head): the drafter's proposal;
 *  accepted: draft tokens the verifier accepted at the previous step (read
 *      only when state[ST_PREV_POSITIONS] > 0; must be in [0, that]);
 *  state[ST_WORDS]: updated in place;
 *  block[0..positions_long): the fused block, -1 past *positions;
 *  *positions: draft positions to verify; *src: bit t set when block[t]
 *      came from the lookup.
 */
int fuse_oracle_step(const fuse_oracle_params *p, const int32_t *lookup, int32_t lookup_k,
                     int32_t d, int32_t m, const int32_t *drafter, int32_t accepted,
                     int32_t *state, int32_t *block, int32_t *positions, uint64_t *src)
{
    if (!params_ok(p) || lookup_k < 1 || d < 0 || d > lookup_k || m < 0)
        return FUSE_ORACLE_EINVAL;
    int32_t prev_positions = state[ST_PREV_POSITIONS];
    if (prev_positions > 0 && (accepted < 0 || accepted > prev_positions))
        return FUSE_ORACLE_EINVAL;

    /* step 3: the run of near-full steps ending at the previous step */
    int32_t streak = state[ST_STREAK];
    if (prev_positions > 0) {
        int near_full = accepted >= prev_positions - p->near_full_slack;
        streak = near_full ? streak + 1 : 0;
        if (streak > p->entry_steps)
            streak = p->entry_steps; /* only "at least entry_steps" matters */
    }

    /* step 3: block size */
    int fills_tail = m >= p->tail_min && d >= p->positions_long;
    int entry = fills_tail && streak >= p->entry_steps;
    int is_long;
    int32_t hold = state[ST_HOLD];
    if (entry) {
        is_long = 1;
        hold = p->sticky;
    } else if (state[ST_LONG] && hold > 0) {
        is_long = 1;
        hold = hold - 1;
    } else {
        is_long = 0;
        hold = 0;
    }

    /* step 2: the head */
    int agree = d >= p->agree_tokens;
    for (int32_t t = 0; agree && t < p->agree_tokens; t++) {
        if (drafter[t] != lookup[t])
            agree = 0;
    }
    int replace_head = m >= p->replace_min || (m >= p->agree_min && agree);
    uint64_t bits = 0;
    for (int32_t t = 0; t < p->head; t++) {
        if (replace_head && t < d) {
            block[t] = lookup[t];
            bits |= (uint64_t)1 << t;
        } else {
            block[t] = drafter[t];
        }
    }
    int32_t n = p->head;

    /* step 2: the tail, in a long block only, up to the first gap */
    if (is_long && m >= p->tail_min) {
        while (n < p->positions_long && n < d) {
            block[n] = lookup[n];
            bits |= (uint64_t)1 << n;
            n++;
        }
    }
    for (int32_t t = n; t < p->positions_long; t++)
        block[t] = -1;

    state[ST_LONG] = is_long;
    state[ST_HOLD] = hold;
    state[ST_STREAK] = streak;
    state[ST_PREV_POSITIONS] = n;
    *positions = n;
    *src = bits;
    return FUSE_ORACLE_OK;
}

/*
 * A batch, one request after another. Row b of lookup is
 * lookup[b * lookup_k ..], of drafter drafter[b * head ..], of state
 * state[b * ST_WORDS ..] and of block block[b * positions_long ..].
 */
int fuse_oracle_batch(const fuse_oracle_params *p, int32_t batch, const int32_t *lookup,
                      int32_t lookup_k, const int32_t *lookup_len, const int32_t *lookup_match,
                      const int32_t *drafter, const int32_t *accepted, int32_t *state,
                      int32_t *block, int32_t *positions, uint64_t *src)
{
    if (batch < 0 || !params_ok(p))
        return FUSE_ORACLE_EINVAL;
    for (int32_t b = 0; b < batch; b++) {
        int rc = fuse_oracle_step(p, lookup + (int64_t)b * lookup_k, lookup_k, lookup_len[b],
                                  lookup_match[b], drafter + (int64_t)b * p->head, accepted[b],
                                  state + (int64_t)b * ST_WORDS,
                                  block + (int64_t)b * p->positions_long, positions + b, src + b);
        if (rc != FUSE_ORACLE_OK)
            return rc;
    }
    return FUSE_ORACLE_OK;
}
