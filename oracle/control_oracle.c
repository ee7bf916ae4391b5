/*
 * Online cost/benefit controller oracle.
 *
 * TEST INFRASTRUCTURE ONLY. The test suite, the package's smoke check and the
 * bench's CPU-baseline leg are the only code that may load this library. The
 * HIP library never links, loads or calls it, and the two share no source,
 * header, table or helper: this file includes nothing but libc headers.
 *
 * What is computed (Strata prompt-lookup page, section 5, the online
 * cost/benefit controller). No fixed threshold decides whether a lookup
 * draft is used; the policy learns online. At every step the controller
 * estimates, for the model's own draft layer (MTP) and for the lookup draft,
 * the expected number of committed tokens per unit of verify time. The
 * acceptance of lookup drafts is estimated online by an exponential moving
 * average (EMA) in 4 buckets of match length; the verify cost comes from
 * measured round times. The lookup draft is used only when its expected
 * gain beats the MTP draft's by at least 5%; otherwise the controller falls
 * back to the MTP draft or, when that does not pay either, to plain
 * decoding. The MTP layer proposes 3 tokens per round (same page, section 1).
 *
 * Written in that order for one request and one step: fold the previous
 * round's measured outcome into the estimates of the source that was used,
 * then estimate each source's committed tokens per unit time for this
 * round and choose.
 *
 * Readings where the page is silent (each one a choice of the plainest form):
 *  - "acceptance" is the fraction of a round's draft tokens the verifier
 *    accepted; committed tokens = accepted + 1 (the verifier's own token),
 *    so a source expected to accept a fraction p of d draft tokens commits
 *    1 + p * d;
 *  - plain decoding commits 1 token per round;
 *  - the 4 match-length buckets start at match lengths 0, edge[0], edge[1],
 *    edge[2] (defaults 6, 8, 12: below 6, 6..7, 8..11, 12 and up, the
 *    HyperQwen page's thresholds for trusting a lookup match);
 *  - one EMA of round time per source (plain, MTP, lookup), weight beta for
 *    a new measurement; acceptance EMAs weight alpha (both 0.1);
 *  - every estimate starts from a prior (acceptance 0.5, time 1.0 in the
 *    caller's unit) and only the source that ran is updated;
 *  - "beats by 5%": rate_lookup >= 1.05 * rate_mtp; a step without a lookup
 *    draft cannot choose it; MTP is chosen when rate_mtp >= rate_plain;
 *  - arithmetic in IEEE double, each operation rounded on its own (no fused
 *    multiply-add), in the order written here.
 *
 * Parity status: pinned (the closed form of an EMA under constant inputs,
 * hand-derived decisions at and around each boundary, invariants of the
 * update, special cases, and planted-mistake mutants that the pins reject).
 */

#include <stddef.h>
#include <stdint.h>

#define CONTROL_ORACLE_OK 0
#define CONTROL_ORACLE_EINVAL 1

typedef struct control_oracle_params {
    double alpha;        /* EMA weight of a new acceptance fraction (0.1) */
    double beta;         /* EMA weight of a new round time (0.1) */
    double margin;       /* lookup needs rate >= margin * MTP's rate (1.05) */
    double prior_accept; /* first acceptance estimate (0.5) */
    double prior_time;   /* first round-time estimate (1.0) */
    int32_t mtp_tokens;  /* MTP draft tokens per round (3) */
    int32_t edge[3];     /* first match length of buckets 1, 2, 3 (6, 8, 12) */
} control_oracle_params;

/* Sources. */
enum { SRC_NONE = -1, SRC_PLAIN = 0, SRC_MTP = 1, SRC_LOOKUP = 2 };

/* State, 11 doubles per request: acceptance per lookup bucket (4), MTP
   acceptance, round time of plain, MTP and lookup rounds, then what the
   last decision was (source, lookup bucket, draft tokens); a state of all
   zeros is "never decided" (the priors are taken then). */
enum {
    ST_ACC0 = 0, ST_ACC_MTP = 4, ST_T_PLAIN = 5, ST_T_MTP = 6, ST_T_LOOKUP = 7,
    ST_LAST_SRC = 8, ST_LAST_BUCKET = 9, ST_LAST_DRAFTED = 10, ST_WORDS = 11
};

static int params_ok(const control_oracle_params *p)
{
    return p->alpha >= 0.0 && p->alpha <= 1.0 && p->beta >= 0.0 && p->beta <= 1.0 &&
           p->margin > 0.0 && p->prior_accept >= 0.0 && p->prior_accept <= 1.0 &&
           p->prior_time > 0.0 && p->mtp_tokens >= 0 && p->edge[0] <= p->edge[1] &&
           p->edge[1] <= p->edge[2];
}

static int bucket_of(const control_oracle_params *p, int32_t match)
{
    int b = 0;
    for (int i = 0; i < 3; i++) {
        if (match >= p->edge[i])
            b = i + 1;
    }
    return b;
}

/*
 * One request, one step.
 *  accepted, round_time: the previous round's outcome (read when a decision
 *      was made before: state[ST_LAST_SRC] encodes it, see below);
 *  lookup_len, lookup_match: this round's lookup draft (0 = none);
 *  state[ST_WORDS]: updated in place; a fresh request has all zeros;
 *  *source: the choice; rates[3]: committed tokens per unit time estimated
 *      for plain, MTP and lookup (the lookup's is 0 without a draft).
 * The last source is stored as source + 1 so that 0 means none.
 */
int control_oracle_step(const control_oracle_params *p, int32_t accepted, double round_time,
                        int32_t lookup_len, int32_t lookup_match, double *state,
                        int32_t *source, double *rates)
{
    if (!params_ok(p) || lookup_len < 0 || lookup_match < 0)
        return CONTROL_ORACLE_EINVAL;
    int last = (int)state[ST_LAST_SRC] - 1;
    if (last == SRC_NONE && state[ST_T_PLAIN] == 0.0) {
        /* a fresh request: every estimate at its prior */
        for (int i = 0; i < 4; i++)
            state[ST_ACC0 + i] = p->prior_accept;
        state[ST_ACC_MTP] = p->prior_accept;
        state[ST_T_PLAIN] = p->prior_time;
        state[ST_T_MTP] = p->prior_time;
        state[ST_T_LOOKUP] = p->prior_time;
    }

    /* fold in the previous round's outcome, for the source that ran */
    if (last != SRC_NONE) {
        int32_t drafted = (int32_t)state[ST_LAST_DRAFTED];
        if (accepted < 0 || accepted > drafted || !(round_time > 0.0))
            return CONTROL_ORACLE_EINVAL;
        if (last == SRC_PLAIN) {
            state[ST_T_PLAIN] = p->beta * round_time + (1.0 - p->beta) * state[ST_T_PLAIN];
        } else if (last == SRC_MTP) {
            double frac = drafted > 0 ? (double)accepted / (double)drafted : 0.0;
            state[ST_ACC_MTP] = p->alpha * frac + (1.0 - p->alpha) * state[ST_ACC_MTP];
            state[ST_T_MTP] = p->beta * round_time + (1.0 - p->beta) * state[ST_T_MTP];
        } else {
            int bk = (int)state[ST_LAST_BUCKET];
            double frac = (double)accepted / (double)drafted;
            state[ST_ACC0 + bk] = p->alpha * frac + (1.0 - p->alpha) * state[ST_ACC0 + bk];
            state[ST_T_LOOKUP] = p->beta * round_time + (1.0 - p->beta) * state[ST_T_LOOKUP];
        }
    }

    /* expected committed tokens per unit time, per source */
    double r_plain = 1.0 / state[ST_T_PLAIN];
    double r_mtp = (1.0 + state[ST_ACC_MTP] * (double)p->mtp_tokens) / state[ST_T_MTP];
    int bk = bucket_of(p, lookup_match);
    double r_lookup = 0.0;
    if (lookup_len > 0)
        r_lookup = (1.0 + state[ST_ACC0 + bk] * (double)lookup_len) / state[ST_T_LOOKUP];

    int choice;
    int32_t drafted;
    if (lookup_len > 0 && r_lookup >= p->margin * r_mtp) {
        choice = SRC_LOOKUP;
        drafted = lookup_len;
    } else if (r_mtp >= r_plain) {
        choice = SRC_MTP;
        drafted = p->mtp_tokens;
    } else {
        choice = SRC_PLAIN;
        drafted = 0;
    }
    state[ST_LAST_SRC] = (double)(choice + 1);
    state[ST_LAST_BUCKET] = (double)bk;
    state[ST_LAST_DRAFTED] = (double)drafted;
    *source = choice;
    rates[0] = r_plain;
    rates[1] = r_mtp;
    rates[2] = r_lookup;
    return CONTROL_ORACLE_OK;
}

/* A batch, one request after another; row b of state is state[b * 11 ..],
   of rates rates[b * 3 ..]. */
int control_oracle_batch(const control_oracle_params *p, int32_t batch, const int32_t *accepted,
                         const double *round_time, const int32_t *lookup_len,
                         const int32_t *lookup_match, double *state, int32_t *source,
                         double *rates)
{
    if (batch < 0 || !params_ok(p))
        return CONTROL_ORACLE_EINVAL;
    for (int32_t b = 0; b < batch; b++) {
        int rc = control_oracle_step(p, accepted[b], round_time[b], lookup_len[b],
                                     lookup_match[b], state + (int64_t)b * ST_WORDS, source + b,
                                     rates + (int64_t)b * 3);
        if (rc != CONTROL_ORACLE_OK)
            return rc;
    }
    return CONTROL_ORACLE_OK;
}
