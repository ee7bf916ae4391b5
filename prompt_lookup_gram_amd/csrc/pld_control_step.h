// One request's step of the online cost/benefit controller, shared by the
// controller's own kernel and the lookup scan's emit (device code only).
//
// Strata prompt-lookup page, section 5: no fixed threshold decides whether a
// lookup draft is used. Every step the controller estimates, for the
// model's own draft layer (MTP, 3 tokens per round per section 1 of the same
// page) and for the lookup draft, the expected committed tokens per unit of
// verify time; lookup acceptance is an exponential moving average in 4
// match-length buckets, verify cost a moving average of measured round
// times. The lookup draft runs only when it beats MTP by the margin (5%);
// otherwise MTP, or plain decoding when MTP does not pay either.
//
// In this order: the previous round's measured outcome updates the
// estimates of the source that ran (its acceptance fraction, accepted /
// drafted, and its round time); then each source's rate is estimated
// (committed tokens = 1 + acceptance * draft tokens, 1 for plain decoding,
// over its round time) and the best by the rule is chosen and remembered.
// Arithmetic is IEEE double with every operation rounded on its own (no
// fused multiply-add), so a decision never depends on how the compiler
// schedules the arithmetic.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "pld_kernels.h"

namespace pld {

// state words per request
constexpr int kCtlAcc0 = 0, kCtlAccMtp = 4, kCtlTPlain = 5, kCtlTMtp = 6, kCtlTLookup = 7;
constexpr int kCtlLastSrc = 8, kCtlLastBucket = 9, kCtlLastDrafted = 10, kCtlWords = 11;
constexpr int kCtlPlain = 0, kCtlMtp = 1, kCtlLookup = 2;

typedef double ctl_double4 __attribute__((ext_vector_type(4)));

// A request's 11 state words in registers: the 4 bucket estimates as one
// vector (a runtime bucket index is then an element select, never a memory
// access), the rest as scalars.
struct CtlState {
    ctl_double4 acc;                  // lookup acceptance per match-length bucket
    double acc_mtp;                   // MTP acceptance
    double t_plain, t_mtp, t_lookup;  // round time per source
    double last_src, last_bucket, last_drafted;  // the last decision (source + 1)
};

__device__ __forceinline__ CtlState ctl_load(const double *row)
{
    CtlState s;
    s.acc = ctl_double4{row[kCtlAcc0], row[kCtlAcc0 + 1], row[kCtlAcc0 + 2], row[kCtlAcc0 + 3]};
    s.acc_mtp = row[kCtlAccMtp];
    s.t_plain = row[kCtlTPlain];
    s.t_mtp = row[kCtlTMtp];
    s.t_lookup = row[kCtlTLookup];
    s.last_src = row[kCtlLastSrc];
    s.last_bucket = row[kCtlLastBucket];
    s.last_drafted = row[kCtlLastDrafted];
    return s;
}

__device__ __forceinline__ void ctl_store(double *row, const CtlState &s)
{
    row[kCtlAcc0] = s.acc.x;
    row[kCtlAcc0 + 1] = s.acc.y;
    row[kCtlAcc0 + 2] = s.acc.z;
    row[kCtlAcc0 + 3] = s.acc.w;
    row[kCtlAccMtp] = s.acc_mtp;
    row[kCtlTPlain] = s.t_plain;
    row[kCtlTMtp] = s.t_mtp;
    row[kCtlTLookup] = s.t_lookup;
    row[kCtlLastSrc] = s.last_src;
    row[kCtlLastBucket] = s.last_bucket;
    row[kCtlLastDrafted] = s.last_drafted;
}

struct ControlResult {
    int choice;
    double r_plain, r_mtp, r_lookup;
    bool bad;  // an input was out of range (the outcome is not folded in)
};

// st: the request's state, updated in place; acc, t: the previous round's
// outcome; d, match: this round's lookup draft length and match.
__device__ __forceinline__ ControlResult control_step(const ControlArgs &a, CtlState &st,
                                                      int32_t acc, double t, int32_t d,
                                                      int32_t match)
{
#pragma clang fp contract(off)
    ControlResult res;
    res.bad = d < 0 || match < 0;
    if (d < 0)
        d = 0;
    const int last = (int)st.last_src - 1;
    if (last < 0 && st.t_plain == 0.0) {
        // a fresh request: every estimate at its prior
        st.acc = ctl_double4{a.prior_accept, a.prior_accept, a.prior_accept, a.prior_accept};
        st.acc_mtp = a.prior_accept;
        st.t_plain = a.prior_time;
        st.t_mtp = a.prior_time;
        st.t_lookup = a.prior_time;
    }
    if (last >= 0) {
        const int32_t drafted = (int32_t)st.last_drafted;
        if (acc < 0 || acc > drafted || !(t > 0.0)) {
            res.bad = true;  // the outcome is not folded in
        } else if (last == kCtlPlain) {
            st.t_plain = a.beta * t + (1.0 - a.beta) * st.t_plain;
        } else if (last == kCtlMtp) {
            const double frac = drafted > 0 ? (double)acc / (double)drafted : 0.0;
            st.acc_mtp = a.alpha * frac + (1.0 - a.alpha) * st.acc_mtp;
            st.t_mtp = a.beta * t + (1.0 - a.beta) * st.t_mtp;
        } else {
            const double sb = st.last_bucket;
            const int bk = sb >= 3.0 ? 3 : (sb >= 0.0 ? (int)sb : 0);  // a corrupt row stays in bounds
            const double frac = (double)acc / (double)drafted;
            st.acc[bk] = a.alpha * frac + (1.0 - a.alpha) * st.acc[bk];
            st.t_lookup = a.beta * t + (1.0 - a.beta) * st.t_lookup;
        }
    }

    res.r_plain = 1.0 / st.t_plain;
    res.r_mtp = (1.0 + st.acc_mtp * (double)a.mtp_tokens) / st.t_mtp;
    int bk = 0;
    for (int i = 0; i < 3; ++i)
        if (match >= a.edge[i])
            bk = i + 1;
    res.r_lookup = 0.0;
    if (d > 0)
        res.r_lookup = (1.0 + st.acc[bk] * (double)d) / st.t_lookup;
    int32_t drafted;
    if (d > 0 && res.r_lookup >= a.margin * res.r_mtp) {
        res.choice = kCtlLookup;
        drafted = d;
    } else if (res.r_mtp >= res.r_plain) {
        res.choice = kCtlMtp;
        drafted = a.mtp_tokens;
    } else {
        res.choice = kCtlPlain;
        drafted = 0;
    }
    st.last_src = (double)(res.choice + 1);
    st.last_bucket = (double)bk;
    st.last_drafted = (double)drafted;
    return res;
}

// Writes one request's choice and (when asked) its estimated rates.
__device__ __forceinline__ void control_write(const ControlArgs &a, int64_t b,
                                              const ControlResult &res)
{
    a.out_source[b] = res.choice;
    if (a.out_rates) {
        a.out_rates[b * 3 + 0] = res.r_plain;
        a.out_rates[b * 3 + 1] = res.r_mtp;
        a.out_rates[b * 3 + 2] = res.r_lookup;
    }
    if (res.bad)
        atomicOr(a.err, kErrControlInput);
}

}  // namespace pld
