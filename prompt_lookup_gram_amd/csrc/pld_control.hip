// Online cost/benefit controller for a batch of requests, for gfx950
// (MI355X): one thread per request.
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
// Per request and step, in this order: the previous round's measured
// outcome updates the estimates of the source that ran (its acceptance
// fraction, accepted / drafted, and its round time); then each source's
// rate is estimated (committed tokens = 1 + acceptance * draft tokens,
// 1 for plain decoding, over its round time) and the best by the rule is
// chosen and remembered. Arithmetic is IEEE double with every operation
// rounded on its own (no fused multiply-add), so a decision never depends
// on how the compiler schedules the arithmetic.

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "pld_kernels.h"

namespace pld {

namespace {

// state words per request
constexpr int kAcc0 = 0, kAccMtp = 4, kTPlain = 5, kTMtp = 6, kTLookup = 7;
constexpr int kLastSrc = 8, kLastBucket = 9, kLastDrafted = 10, kWords = 11;
constexpr int kPlain = 0, kMtp = 1, kLookup = 2;

__global__ __launch_bounds__(256) void pld_control_kernel(ControlArgs a)
{
#pragma clang fp contract(off)
    const int64_t b = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
    if (b >= a.batch)
        return;
    double st[kWords];
    double *row = a.state + b * kWords;
    for (int i = 0; i < kWords; ++i)
        st[i] = row[i];
    int32_t d = a.lookup_len[b];
    const int32_t match = a.lookup_match[b];
    bool bad = d < 0 || match < 0;
    if (d < 0)
        d = 0;

    const int last = (int)st[kLastSrc] - 1;
    if (last < 0 && st[kTPlain] == 0.0) {
        // a fresh request: every estimate at its prior
        for (int i = 0; i < 4; ++i)
            st[kAcc0 + i] = a.prior_accept;
        st[kAccMtp] = a.prior_accept;
        st[kTPlain] = a.prior_time;
        st[kTMtp] = a.prior_time;
        st[kTLookup] = a.prior_time;
    }
    if (last >= 0) {
        const int32_t drafted = (int32_t)st[kLastDrafted];
        const int32_t acc = a.accepted[b];
        const double t = a.round_time[b];
        if (acc < 0 || acc > drafted || !(t > 0.0)) {
            bad = true;  // the outcome is not folded in
        } else if (last == kPlain) {
            st[kTPlain] = a.beta * t + (1.0 - a.beta) * st[kTPlain];
        } else if (last == kMtp) {
            const double frac = drafted > 0 ? (double)acc / (double)drafted : 0.0;
            st[kAccMtp] = a.alpha * frac + (1.0 - a.alpha) * st[kAccMtp];
            st[kTMtp] = a.beta * t + (1.0 - a.beta) * st[kTMtp];
        } else {
            const double sb = st[kLastBucket];
            const int bk = sb >= 3.0 ? 3 : (sb >= 0.0 ? (int)sb : 0);  // a corrupt row stays in bounds
            const double frac = (double)acc / (double)drafted;
            st[kAcc0 + bk] = a.alpha * frac + (1.0 - a.alpha) * st[kAcc0 + bk];
            st[kTLookup] = a.beta * t + (1.0 - a.beta) * st[kTLookup];
        }
    }

    const double r_plain = 1.0 / st[kTPlain];
    const double r_mtp = (1.0 + st[kAccMtp] * (double)a.mtp_tokens) / st[kTMtp];
    int bk = 0;
    for (int i = 0; i < 3; ++i)
        if (match >= a.edge[i])
            bk = i + 1;
    double r_lookup = 0.0;
    if (d > 0)
        r_lookup = (1.0 + st[kAcc0 + bk] * (double)d) / st[kTLookup];
    int choice;
    int32_t drafted;
    if (d > 0 && r_lookup >= a.margin * r_mtp) {
        choice = kLookup;
        drafted = d;
    } else if (r_mtp >= r_plain) {
        choice = kMtp;
        drafted = a.mtp_tokens;
    } else {
        choice = kPlain;
        drafted = 0;
    }
    st[kLastSrc] = (double)(choice + 1);
    st[kLastBucket] = (double)bk;
    st[kLastDrafted] = (double)drafted;
    for (int i = 0; i < kWords; ++i)
        row[i] = st[i];
    a.out_source[b] = choice;
    if (a.out_rates) {
        a.out_rates[b * 3 + 0] = r_plain;
        a.out_rates[b * 3 + 1] = r_mtp;
        a.out_rates[b * 3 + 2] = r_lookup;
    }
    if (bad)
        atomicOr(a.err, kErrControlInput);
}

}  // namespace

hipError_t launch_control(const ControlArgs &a, hipStream_t s)
{
    if (a.batch <= 0)
        return hipSuccess;
    const unsigned blocks = (unsigned)((a.batch + 255) / 256);
    hipLaunchKernelGGL(pld_control_kernel, dim3(blocks), dim3(256), 0, s, a);
    return hipGetLastError();
}

}  // namespace pld
