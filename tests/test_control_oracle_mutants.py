"""Planted mistakes in the controller oracle must be caught by its pins.

Each mutant is a copy of ``oracle/control_oracle.c`` with one plausible slip
in a rule of the Strata prompt-lookup page's section 5 (a weight on the
wrong side, a dropped term, a boundary off by one, the wrong estimate
updated), compiled with gcc into a temporary library on the CPU. The
hand-derived decisions, the moving-average closed form and the update
invariants are run against it; at least one must fail.
"""

from __future__ import annotations

import os

import numpy as np
import pytest

import oracle
import test_control_oracle_pins as pins

HERE = os.path.dirname(oracle.__file__)
SRC = os.path.join(HERE, "control_oracle.c")

MUTANTS = {
    "ema_weight_on_old": ("state[ST_ACC0 + bk] = p->alpha * frac + (1.0 - p->alpha) * state[ST_ACC0 + bk];",
                          "state[ST_ACC0 + bk] = (1.0 - p->alpha) * frac + p->alpha * state[ST_ACC0 + bk];"),
    "time_uses_alpha": ("state[ST_T_LOOKUP] = p->beta * round_time + (1.0 - p->beta) * state[ST_T_LOOKUP];",
                        "state[ST_T_LOOKUP] = p->alpha * round_time + (1.0 - p->alpha) * state[ST_T_LOOKUP];"),
    "no_bonus_token": ("r_lookup = (1.0 + state[ST_ACC0 + bk] * (double)lookup_len) / state[ST_T_LOOKUP];",
                       "r_lookup = (state[ST_ACC0 + bk] * (double)lookup_len) / state[ST_T_LOOKUP];"),
    "margin_on_lookup": ("r_lookup >= p->margin * r_mtp", "p->margin * r_lookup >= r_mtp"),
    "margin_strict": ("r_lookup >= p->margin * r_mtp", "r_lookup > p->margin * r_mtp"),
    "plain_beats_ties": ("} else if (r_mtp >= r_plain) {", "} else if (r_mtp > r_plain) {"),
    "bucket_edge_exclusive": ("if (match >= p->edge[i])", "if (match > p->edge[i])"),
    "mtp_rate_ignores_tokens": ("double r_mtp = (1.0 + state[ST_ACC_MTP] * (double)p->mtp_tokens) / state[ST_T_MTP];",
                                "double r_mtp = (1.0 + state[ST_ACC_MTP]) / state[ST_T_MTP];"),
    "mtp_updates_lookup_time": ("state[ST_T_MTP] = p->beta * round_time + (1.0 - p->beta) * state[ST_T_MTP];",
                                "state[ST_T_LOOKUP] = p->beta * round_time + (1.0 - p->beta) * state[ST_T_LOOKUP];"),
    "lookup_updates_bucket_zero": ("int bk = (int)state[ST_LAST_BUCKET];", "int bk = 0;"),
    "fraction_counts_bonus": ("double frac = (double)accepted / (double)drafted;",
                              "double frac = (double)(accepted + 1) / (double)(drafted + 1);"),
    # (taking the lookup without a draft would be an equivalent mutant: its
    # rate is then 0 and the MTP rate is always positive)
    "rate_without_draft": ("    if (lookup_len > 0)\n        r_lookup",
                           "    if (lookup_len >= 0)\n        r_lookup"),
    "remembers_wrong_drafted": ("        drafted = p->mtp_tokens;", "        drafted = 0;"),
    "plain_rate_from_mtp_time": ("double r_plain = 1.0 / state[ST_T_PLAIN];",
                                 "double r_plain = 1.0 / state[ST_T_MTP];"),
}


def _pins_fail(lib) -> bool:
    checks = []

    def hand_case(d, m, want, rates):
        src, r, st = pins.step(oracle.ControlParams(), pins.fresh(), 0, 1.0, d, m, lib=lib)
        bucket = {0: 0, 4: 0, 12: 3}[m]
        drafted = {pins.LOOKUP: d, pins.MTP: 3, pins.PLAIN: 0}[want]
        return (src == want and r.tolist() == list(rates) and
                st[0, 8:].tolist() == [want + 1, bucket, drafted])

    for case in pins.HAND_DECISIONS:
        checks.append(lambda case=case: hand_case(*case))
    P = oracle.ControlParams

    def plain_case():
        p = P(prior_accept=0.0)
        src, r, st = pins.step(p, pins.fresh(), 0, 1.0, 0, 0, lib=lib)
        src2, r2, st2 = pins.step(p, st, 0, 2.0, 0, 0, lib=lib)
        src3, r3, st3 = pins.step(p, st2, 0, 1.0, 0, 0, lib=lib)
        return (src, src2, src3) == (pins.MTP, pins.PLAIN, pins.PLAIN) and \
            st2[0, 6] == 0.1 * 2.0 + 0.9 * 1.0 and st3[0, 5] == 1.0

    def margin_case():
        f = pins.fresh()
        return (pins.step(P(margin=1.5), f, 0, 1.0, 5, 12, lib=lib)[0] == pins.MTP and
                pins.step(P(margin=1.5), f, 0, 1.0, 6, 12, lib=lib)[0] == pins.LOOKUP and
                pins.step(P(margin=1.6), f, 0, 1.0, 6, 12, lib=lib)[0] == pins.LOOKUP)

    def bucket_case():
        for m, bucket in pins.BUCKETS:
            p = P(margin=0.01)
            _, _, st = pins.step(p, pins.fresh(), 0, 1.0, 8, m, lib=lib)
            _, _, st2 = pins.step(p, st, 8, 1.0, 8, m, lib=lib)
            want = [0.5] * 4
            want[bucket] = 0.1 * 1.0 + 0.9 * 0.5
            if st2[0, :4].tolist() != want or st2[0, 7] != 0.1 + 0.9:
                return False
        return True

    def ema_case():
        p = P(alpha=0.3, beta=0.05, margin=1e-9)
        _, _, st = pins.step(p, pins.fresh(), 0, 1.0, 8, 12, lib=lib)
        for k in range(1, 30):
            _, _, st = pins.step(p, st, 6, 2.0, 8, 12, lib=lib)
            if abs(st[0, 3] - (0.75 + (0.5 - 0.75) * 0.7 ** k)) > 1e-12:
                return False
            if abs(st[0, 7] - (2.0 + (1.0 - 2.0) * 0.95 ** k)) > 1e-12:
                return False
        return True

    checks += [plain_case, margin_case, bucket_case, ema_case]
    for c in checks:
        try:
            if not c():
                return True
        except oracle.OracleError:
            return True
    for seed in range(10):
        try:
            if pins.outcome_errors(seed, lib=lib) is not None:
                return True
        except oracle.OracleError:
            return True
    return False


@pytest.mark.parametrize("name", sorted(MUTANTS))
def test_control_mutant_is_caught(name, tmp_path):
    src = open(SRC).read()
    old, new = MUTANTS[name]
    assert old in src, f"mutation site for {name} no longer in the oracle"
    c = tmp_path / "control_oracle.c"
    c.write_text(src.replace(old, new, 1))
    so = tmp_path / f"{name}.so"
    oracle.compile_lib(str(so), oracle.sources({"control_oracle.c": str(c)}), strict=False)
    assert _pins_fail(oracle.load(str(so))), f"mutant {name} passed every pin"


def test_unmutated_control_oracle_passes_same_pins():
    assert not _pins_fail(oracle.load())
