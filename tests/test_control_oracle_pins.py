"""Pins for the online cost/benefit controller oracle (Strata prompt-lookup
page, section 5), ``oracle/control_oracle.c``.

- The closed form of an exponential moving average under constant inputs,
  x_k = x + (x_0 - x)(1 - w)^k, against the oracle's step-by-step updates.
- Hand-derived decisions from a fresh state, at and around each boundary
  (lookup against 1.05 x MTP, MTP against plain decoding), worked out from
  the page's rule with the stated readings.
- Which estimates a round's outcome may change (only its source's; a lookup
  round only its match-length bucket), over random traces.
- Special cases: no learning (weights 0), last-value estimates (weights 1),
  a margin no lookup can meet, a margin every lookup meets.
"""

from __future__ import annotations

import numpy as np
import pytest

import oracle

P = oracle.ControlParams
PLAIN, MTP, LOOKUP = oracle.SRC_PLAIN, oracle.SRC_MTP, oracle.SRC_LOOKUP
W = oracle.CONTROL_STATE_WORDS


def fresh(batch=1):
    return np.zeros((batch, W), np.float64)


def step(params, state, accepted, t, d, m, lib=None):
    src, rates, st = oracle.control(params, np.atleast_1d(accepted), np.atleast_1d(t),
                                    np.atleast_1d(d), np.atleast_1d(m), state, lib=lib)
    return int(src[0]), rates[0], st


# ---------------------------------------------------------------------------
# hand-derived decisions
# ---------------------------------------------------------------------------
#
# Fresh state, defaults: every acceptance estimate 0.5, every round time 1.0.
#   rate_plain = 1 / 1.0 = 1.0
#   rate_mtp = (1 + 0.5 * 3) / 1.0 = 2.5, so the lookup needs >= 2.625
#   rate_lookup(d) = (1 + 0.5 * d) / 1.0
# d = 3: 2.5 < 2.625 -> MTP (2.5 >= 1.0); d = 4: 3.0 >= 2.625 -> LOOKUP;
# d = 0: no lookup draft -> MTP.

HAND_DECISIONS = [
    # (draft length, match length, expected source, expected rates)
    (0, 0, MTP, (1.0, 2.5, 0.0)),
    (3, 12, MTP, (1.0, 2.5, 2.5)),
    (4, 12, LOOKUP, (1.0, 2.5, 3.0)),
    (16, 4, LOOKUP, (1.0, 2.5, 9.0)),
]


@pytest.mark.parametrize("d,m,want,rates", HAND_DECISIONS)
def test_fresh_decisions(d, m, want, rates):
    src, r, st = step(P(), fresh(), 0, 1.0, d, m)
    assert src == want
    assert r.tolist() == list(rates)
    # the decision is remembered: source + 1, lookup bucket, draft tokens
    bucket = {0: 0, 4: 0, 12: 3}[m]
    drafted = {LOOKUP: d, MTP: 3, PLAIN: 0}[want]
    assert st[0, 8:].tolist() == [want + 1, bucket, drafted]


def test_plain_when_mtp_does_not_pay():
    """prior acceptance 0: rate_mtp = (1 + 0) / 1 = 1.0 = rate_plain -> MTP
    (ties go to the draft). One MTP round of time 2.0 accepting 0 of 3:
    time 0.1 * 2.0 + 0.9 * 1.0 = 1.1, rate_mtp = 1 / 1.1 < 1.0 -> PLAIN;
    then plain rounds of time 1.0 leave rate_plain at 1.0 and keep PLAIN."""
    p = P(prior_accept=0.0)
    src, r, st = step(p, fresh(), 0, 1.0, 0, 0)
    assert src == MTP and r.tolist() == [1.0, 1.0, 0.0]
    src, r, st = step(p, st, 0, 2.0, 0, 0)
    assert src == PLAIN
    assert st[0, 6] == 0.1 * 2.0 + 0.9 * 1.0
    assert r[1] == 1.0 / (0.1 * 2.0 + 0.9 * 1.0)
    src, r, st = step(p, st, 0, 1.0, 0, 0)
    assert src == PLAIN and st[0, 5] == 0.1 * 1.0 + 0.9 * 1.0


def test_margin_boundary():
    """rate_lookup at exactly margin * rate_mtp chooses the lookup (the rule
    is ">= 5% better"). margin 1.5 (exact in binary): rate_mtp 2.5, the
    lookup needs 3.75 = 1 + 0.5 d, d >= 5.5: d = 5 gives 3.5 -> MTP, d = 6
    gives 4.0 -> LOOKUP. margin 1.6: 1.6 * 2.5 is 4.0000000000000002 before
    rounding and 4.0 after (the next double up is 4 + 8.9e-16), so d = 6
    (rate 4.0) ties and takes the lookup."""
    p = P(margin=1.5)
    assert step(p, fresh(), 0, 1.0, 5, 12)[0] == MTP
    assert step(p, fresh(), 0, 1.0, 6, 12)[0] == LOOKUP
    assert step(P(margin=1.6), fresh(), 0, 1.0, 6, 12)[0] == LOOKUP
    assert step(P(margin=1.61), fresh(), 0, 1.0, 6, 12)[0] == MTP


BUCKETS = [(0, 0), (5, 0), (6, 1), (7, 1), (8, 2), (11, 2), (12, 3), (64, 3)]


@pytest.mark.parametrize("m,bucket", BUCKETS)
def test_lookup_outcome_updates_its_bucket(m, bucket):
    """A lookup round's acceptance goes to its match length's bucket
    (edges 6, 8, 12): fraction 4/8 = 0.5 -> unchanged; 8/8 -> 0.1 + 0.45."""
    p = P(margin=0.01)          # every lookup draft is taken
    src, _, st = step(p, fresh(), 0, 1.0, 8, m)
    assert src == LOOKUP
    _, _, st2 = step(p, st, 8, 1.0, 8, m)
    want = [0.5] * 4
    want[bucket] = 0.1 * 1.0 + 0.9 * 0.5
    assert st2[0, :4].tolist() == want
    assert st2[0, 4] == 0.5                      # MTP's estimate untouched
    assert st2[0, 7] == 0.1 * 1.0 + 0.9 * 1.0    # lookup round time


# ---------------------------------------------------------------------------
# closed form of the moving averages
# ---------------------------------------------------------------------------


@pytest.mark.parametrize("alpha,beta,frac,t", [(0.1, 0.1, 0.75, 2.0), (0.3, 0.05, 0.2, 0.4),
                                              (0.9, 0.5, 1.0, 7.5)])
def test_ema_closed_form(alpha, beta, frac, t):
    """k lookup rounds that each accept a fraction `frac` of 8 tokens in time
    t: estimate_k = frac + (0.5 - frac)(1 - alpha)^k, time_k = t + (1 - t)(1 -
    beta)^k."""
    p = P(alpha=alpha, beta=beta, margin=1e-9)
    st = fresh()
    src, _, st = step(p, st, 0, 1.0, 8, 12)
    acc = int(round(frac * 8))
    frac = acc / 8          # the fraction the rounds actually accept
    for k in range(1, 61):
        src, _, st = step(p, st, acc, t, 8, 12)
        assert src == LOOKUP
        a_k = frac + (0.5 - frac) * (1 - alpha) ** k
        t_k = t + (1.0 - t) * (1 - beta) ** k
        assert st[0, 3] == pytest.approx(a_k, rel=1e-12, abs=1e-14)
        assert st[0, 7] == pytest.approx(t_k, rel=1e-12, abs=1e-14)


# ---------------------------------------------------------------------------
# random traces: what an outcome may change
# ---------------------------------------------------------------------------


def random_trace(seed, batch=16, steps=80, lib=None, params=None):
    rng = np.random.default_rng([7201, seed])
    p = params or P(alpha=float(rng.uniform(0, 1)), beta=float(rng.uniform(0, 1)),
                    margin=float(rng.uniform(0.5, 2.0)),
                    prior_accept=float(rng.uniform(0, 1)),
                    prior_time=float(rng.uniform(0.5, 2)), mtp_tokens=int(rng.integers(0, 6)),
                    edge=tuple(sorted(rng.integers(1, 16, 3).tolist())))
    st = np.zeros((batch, W))
    drafted = np.zeros(batch, np.int64)
    rows = []
    for _ in range(steps):
        acc = np.array([rng.integers(0, k + 1) for k in drafted], np.int32)
        t = rng.uniform(0.2, 3.0, batch)
        d = np.where(rng.random(batch) < 0.7, rng.integers(1, 17, batch), 0).astype(np.int32)
        m = np.where(d > 0, rng.integers(1, 20, batch), 0).astype(np.int32)
        src, rates, st2 = oracle.control(p, acc, t, d, m, st, lib=lib)
        rows.append((acc, t, d, m, src, rates, st.copy(), st2.copy()))
        drafted = st2[:, 10].astype(np.int64)
        st = st2
    return p, rows


def outcome_errors(seed, lib=None):
    """First violated property of a random trace, or None."""
    p, rows = random_trace(seed, lib=lib)
    for i, (acc, t, d, m, src, rates, before, after) in enumerate(rows):
        for b in range(len(src)):
            if i == 0:
                continue  # first step: priors
            last = int(before[b, 8]) - 1
            changed = np.nonzero(before[b, :8] != after[b, :8])[0].tolist()
            allowed = {0: [5], 1: [4, 6], 2: [int(before[b, 9]), 7]}[last]
            if not set(changed) <= set(allowed):
                return (i, b, "changed", changed, allowed)
            if not (0.0 <= after[b, :5]).all() or not (after[b, :5] <= 1.0).all():
                return (i, b, "acceptance outside [0, 1]")
            if not (after[b, 5:8] > 0).all():
                return (i, b, "time not positive")
            # the choice is the best by the rule stated on the page
            r_p, r_m, r_l = rates[b]
            if d[b] > 0 and r_l >= p.margin * r_m:
                want = LOOKUP
            elif r_m >= r_p:
                want = MTP
            else:
                want = PLAIN
            if src[b] != want:
                return (i, b, "choice", int(src[b]), want)
            if src[b] == LOOKUP and d[b] == 0:
                return (i, b, "lookup without a draft")
    return None


@pytest.mark.parametrize("seed", range(10))
def test_outcomes_touch_only_their_source(seed):
    assert outcome_errors(seed) is None


def test_no_learning_and_last_value():
    """alpha = beta = 0: estimates stay at the priors; alpha = beta = 1:
    they equal the last round's fraction and time."""
    _, rows = random_trace(3, params=P(alpha=0.0, beta=0.0))
    for *_, after in rows:
        assert (after[:, :5] == 0.5).all() and (after[:, 5:8] == 1.0).all()
    p = P(alpha=1.0, beta=1.0, margin=1e-9)
    st = fresh()
    _, _, st = step(p, st, 0, 1.0, 10, 9)
    _, _, st = step(p, st, 3, 0.25, 10, 9)
    assert st[0, 2] == 0.3 and st[0, 7] == 0.25


def test_unreachable_margin_and_free_lookup():
    _, rows = random_trace(4, params=P(margin=1e30))
    assert all((r[4] != LOOKUP).all() for r in rows)
    _, rows = random_trace(5, params=P(margin=1e-30))
    for acc, t, d, m, src, *_ in rows:
        assert ((src == LOOKUP) == (d > 0)).all()


def test_rejects_bad_outcomes():
    _, _, st = step(P(), fresh(), 0, 1.0, 4, 12)       # lookup of 4 chosen
    with pytest.raises(oracle.OracleError):
        step(P(), st, 5, 1.0, 4, 12)                   # accepted > drafted
    with pytest.raises(oracle.OracleError):
        step(P(), st, 2, 0.0, 4, 12)                   # non-positive time
    with pytest.raises(oracle.OracleError):
        step(P(alpha=1.5), fresh(), 0, 1.0, 4, 12)
