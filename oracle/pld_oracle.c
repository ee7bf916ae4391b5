/*
 * Prompt-lookup drafting oracle.
 *
 * TEST INFRASTRUCTURE ONLY. The test suite, the package's smoke check and the
 * bench's CPU-baseline leg are the only code that may load this library. The
 * HIP library never links, loads or calls it, and the two share no source,
 * header, table or helper: this file includes nothing but libc headers.
 *
 * What is computed (HyperQwen lookup-drafting page, "lookup drafting: the
 * three-step principle", step 1): before each decode step, each request's own
 * token history is searched for the most recent earlier occurrence of its
 * longest just-generated suffix, between n_min and n_max tokens long (4..12 on
 * that page); the tokens that followed that occurrence become the draft. The
 * occurrence may overlap the suffix itself, so a periodic tail matches at its
 * own period. The draft is bounded by the verify block (HyperQwen page, step
 * 2: 15 draftable positions in a 16-token block; Strata prompt-lookup page,
 * section 4: at most 5 tokens), here the parameter k_max.
 *
 * Written as a plain search in the order the rule is stated: lengths from the
 * longest allowed down to n_min, and for each length start positions from the
 * most recent down to 0; the first hit is the answer.
 *
 * Readings where the page is silent (each one a choice of the plainest form):
 *  - the suffix matching itself (start j = L - m) does not count, and an
 *    occurrence must be followed by at least one token: j + m <= L - 1;
 *  - overlap is unrestricted: any j <= L - m - 1, including j = L - m - 1;
 *  - the continuation stops at the end of the history:
 *    d = min(k_max, L - (j + m)); it does not wrap into itself;
 *  - among occurrences of the longest length the most recent (largest j)
 *    wins, even if an older one would give a longer draft;
 *  - matches longer than n_max count as n_max (the search never looks further);
 *  - with L - 1 < n_min there is no match;
 *  - no match: draft length 0, match length 0, start -1, row all -1;
 *  - draft slots past the draft length hold -1;
 *  - tokens are compared as raw 32-bit integers.
 *
 * Parity status: pinned (exhaustive brute force over the set definition, a
 * reversed-history Z-function cross-check, a linear-time certificate checker,
 * the periodic-tail closed form, hand-derived planted-copy examples, the
 * continuation invariant, and planted-mistake mutants that the pins reject).
 */

#include <stddef.h>
#include <stdint.h>

#define PLD_ORACLE_OK 0
#define PLD_ORACLE_EINVAL 1

/* 1 when the n tokens at a and at b are equal. */
static int same_tokens(const int32_t *a, const int32_t *b, int64_t n)
{
    for (int64_t i = 0; i < n; i++) {
        if (a[i] != b[i])
            return 0;
    }
    return 1;
}

/*
 * One request. h[0..L) is the history. Writes k_max draft slots, the draft
 * length, the match length and the occurrence start j (-1 when none).
 */
int pld_oracle_draft_one(const int32_t *h, int64_t L, int32_t n_min,
                         int32_t n_max, int32_t k_max, int32_t *draft,
                         int32_t *out_len, int32_t *out_match, int64_t *out_pos)
{
    if (n_min < 1 || n_max < n_min || k_max < 1 || L < 0)
        return PLD_ORACLE_EINVAL;
    if (L > 0 && h == NULL)
        return PLD_ORACLE_EINVAL;

    for (int32_t t = 0; t < k_max; t++)
        draft[t] = -1;
    *out_len = 0;
    *out_match = 0;
    *out_pos = -1;

    /* the longest suffix that can still have an earlier occurrence followed
       by at least one token */
    int64_t m_top = (L - 1 < (int64_t)n_max) ? L - 1 : (int64_t)n_max;

    for (int64_t m = m_top; m >= n_min; m--) {
        const int32_t *suffix = h + (L - m);
        for (int64_t j = L - m - 1; j >= 0; j--) {
            if (same_tokens(h + j, suffix, m)) {
                int64_t follow = L - (j + m);
                int64_t d = follow < (int64_t)k_max ? follow : (int64_t)k_max;
                for (int64_t t = 0; t < d; t++)
                    draft[t] = h[j + m + t];
                *out_len = (int32_t)d;
                *out_match = (int32_t)m;
                *out_pos = j;
                return PLD_ORACLE_OK;
            }
        }
    }
    return PLD_ORACLE_OK;
}

/*
 * A batch: histories[b] points at request b's lengths[b] tokens. Output row b
 * of out_draft is out_draft[b * k_max .. (b + 1) * k_max). Requests are done
 * one after another on the calling thread.
 */
int pld_oracle_draft_batch(const int32_t *const *histories,
                           const int64_t *lengths, int32_t batch,
                           int32_t n_min, int32_t n_max, int32_t k_max,
                           int32_t *out_draft, int32_t *out_len,
                           int32_t *out_match, int64_t *out_pos)
{
    if (batch < 0)
        return PLD_ORACLE_EINVAL;
    for (int32_t b = 0; b < batch; b++) {
        int rc = pld_oracle_draft_one(histories[b], lengths[b], n_min, n_max,
                                      k_max, out_draft + (int64_t)b * k_max,
                                      out_len + b, out_match + b, out_pos + b);
        if (rc != PLD_ORACLE_OK)
            return rc;
    }
    return PLD_ORACLE_OK;
}
