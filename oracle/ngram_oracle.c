/*
 * Successor-count ("context cache") n-gram drafting oracle.
 *
 * TEST INFRASTRUCTURE ONLY. The test suite, the package's smoke check and the
 * bench's CPU-baseline leg are the only code that may load this library. The
 * HIP library never links, loads or calls it, and the two share no source,
 * header, table or helper: this file includes nothing but libc headers.
 *
 * What is computed (llama.cpp page, the section that explains what prompt
 * lookup decoding is). The drafter keeps, over the current token stream,
 * statistics of the n-grams of sizes 1 to 4 and of the tokens that followed
 * each of them. A draft is built one token at a time: each drafted token
 * costs one lookup of the tokens just before it. Fixed acceptance thresholds
 * decide whether a lookup may propose its most frequent successor; the
 * page's example for the context cache is a 4-gram seen at least once whose
 * most frequent successor accounts for at least half of its occurrences.
 * The page's later sections (sorted successor vectors, checking the
 * thresholds on the top successor before scoring the rest) change how fast
 * this is answered, not what.
 *
 * Here the statistics are not cached: for every draft token and context
 * length they are recounted from the history by brute force (every position
 * is compared; the successors found are sorted and the longest run of equal
 * tokens is the most frequent one). That is the definition written out.
 *
 * Readings where the page is silent (each one a choice of the plainest form):
 *  - the statistics of an n-gram g are taken over every position i of the
 *    history h[0..L) with n <= i < L and h[i-n..i) == g: its count is the
 *    number of such i, and h[i] is a successor (an occurrence at the very end
 *    has no successor and is not counted);
 *  - the context of draft token s is the last n tokens of the history
 *    followed by the s tokens drafted so far; drafted tokens are not counted
 *    in the statistics (they are not part of the stream yet);
 *  - lengths are tried from n_max (4) down to n_min (1); the first length
 *    whose statistics pass its thresholds proposes the token ("queried in
 *    priority order", the most specific context first);
 *  - thresholds per length n: count >= max(1, min_count[n-1]) and
 *    100 * top >= min_percent[n-1] * count, with top the most frequent
 *    successor's count; the page gives the 4-gram's (1 and 50) and, by
 *    default, every length uses the same;
 *  - among successors with the same top count the smaller token (as a
 *    signed 32-bit integer) is proposed;
 *  - drafting stops at the first token that no length can propose, or at
 *    k_max tokens; the draft row is padded with -1 and the per-token context
 *    length with 0.
 *
 * Parity status: pinned (hand-derived golden cases, an independent
 * incremental-dictionary drafter in the tests, periodic streams whose
 * drafts have a closed form, threshold special cases, and planted-mistake
 * mutants that the pins reject).
 */

#include <stddef.h>
#include <stdint.h>
#include <stdlib.h>

#define NGRAM_ORACLE_OK 0
#define NGRAM_ORACLE_EINVAL 1
#define NGRAM_ORACLE_ENOMEM 2
#define NGRAM_ORACLE_MAX_N 4

typedef struct ngram_oracle_params {
    int32_t n_min;                           /* shortest context tried (1) */
    int32_t n_max;                           /* longest context tried (4) */
    int32_t min_count[NGRAM_ORACLE_MAX_N];   /* per n (index n-1): occurrences needed (1) */
    int32_t min_percent[NGRAM_ORACLE_MAX_N]; /* per n: top successor's share, percent (50) */
} ngram_oracle_params;

static int params_ok(const ngram_oracle_params *p)
{
    if (p->n_min < 1 || p->n_max < p->n_min || p->n_max > NGRAM_ORACLE_MAX_N)
        return 0;
    for (int i = 0; i < NGRAM_ORACLE_MAX_N; i++) {
        if (p->min_count[i] < 0 || p->min_percent[i] < 0 || p->min_percent[i] > 100)
            return 0;
    }
    return 1;
}

static int cmp_i32(const void *a, const void *b)
{
    int32_t x = *(const int32_t *)a, y = *(const int32_t *)b;
    return (x > y) - (x < y);
}

/* Statistics of the n-gram ctx[0..n) over the history: *count occurrences
   followed by a token, the most frequent successor *tok with *top of them
   (smallest token on a tie). succ has room for L tokens. */
static void successor_stats(const int32_t *h, int64_t L, const int32_t *ctx, int n,
                            int32_t *succ, int64_t *count, int64_t *top, int32_t *tok)
{
    int64_t c = 0;
    for (int64_t i = n; i < L; i++) {
        int eq = 1;
        for (int t = 0; t < n; t++) {
            if (h[i - n + t] != ctx[t]) {
                eq = 0;
                break;
            }
        }
        if (eq)
            succ[c++] = h[i];
    }
    *count = c;
    *top = 0;
    *tok = -1;
    if (c == 0)
        return;
    qsort(succ, (size_t)c, sizeof(int32_t), cmp_i32);
    /* longest run of equal tokens; runs are visited in increasing token
       order and only a strictly longer run replaces the best, so a tie keeps
       the smaller token */
    int64_t run_start = 0;
    for (int64_t i = 1; i <= c; i++) {
        if (i == c || succ[i] != succ[run_start]) {
            if (i - run_start > *top) {
                *top = i - run_start;
                *tok = succ[run_start];
            }
            run_start = i;
        }
    }
}

/*
 * One request.
 *  h[0..L): the history; k_max >= 1 draft tokens at most;
 *  draft[k_max]: the draft, -1 past *draft_len;
 *  levels[k_max]: the context length that proposed each token, 0 past it.
 */
int ngram_oracle_draft_one(const ngram_oracle_params *p, const int32_t *h, int64_t L,
                           int32_t k_max, int32_t *draft, int32_t *draft_len, int32_t *levels)
{
    if (!params_ok(p) || L < 0 || k_max < 1)
        return NGRAM_ORACLE_EINVAL;
    for (int32_t s = 0; s < k_max; s++) {
        draft[s] = -1;
        levels[s] = 0;
    }
    *draft_len = 0;
    if (L == 0)
        return NGRAM_ORACLE_OK;
    int32_t *succ = (int32_t *)malloc((size_t)L * sizeof(int32_t));
    if (!succ)
        return NGRAM_ORACLE_ENOMEM;
    for (int32_t s = 0; s < k_max; s++) {
        /* the stream so far: the history, then draft[0..s) */
        int64_t len = L + s;
        int32_t chosen = 0, tok = -1;
        for (int n = p->n_max; n >= p->n_min && !chosen; n--) {
            if (len < n)
                continue;
            int32_t ctx[NGRAM_ORACLE_MAX_N];
            for (int t = 0; t < n; t++) {
                int64_t q = len - n + t;
                ctx[t] = q < L ? h[q] : draft[q - L];
            }
            int64_t count, top;
            int32_t best;
            successor_stats(h, L, ctx, n, succ, &count, &top, &best);
            int64_t need = p->min_count[n - 1] > 1 ? p->min_count[n - 1] : 1;
            if (count >= need && 100 * top >= (int64_t)p->min_percent[n - 1] * count) {
                chosen = n;
                tok = best;
            }
        }
        if (!chosen)
            break;
        draft[s] = tok;
        levels[s] = chosen;
        *draft_len = s + 1;
    }
    free(succ);
    return NGRAM_ORACLE_OK;
}

/* A batch, one request after another: histories[b] with lengths[b]; rows b
   of draft and levels start at b * k_max. */
int ngram_oracle_draft_batch(const ngram_oracle_params *p, const int32_t *const *histories,
                             const int64_t *lengths, int32_t batch, int32_t k_max,
                             int32_t *draft, int32_t *draft_len, int32_t *levels)
{
    if (batch < 0 || k_max < 1 || !params_ok(p))
        return NGRAM_ORACLE_EINVAL;
    for (int32_t b = 0; b < batch; b++) {
        int rc = ngram_oracle_draft_one(p, histories[b], lengths[b], k_max,
                                        draft + (int64_t)b * k_max, draft_len + b,
                                        levels + (int64_t)b * k_max);
        if (rc != NGRAM_ORACLE_OK)
            return rc;
    }
    return NGRAM_ORACLE_OK;
}
