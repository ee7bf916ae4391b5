"""Planted mistakes in the oracle must be caught by the pins.

Each mutant is a copy of ``oracle/pld_oracle.c`` with one plausible slip
(an off-by-one bound, a dropped term, a wrong index, a flipped comparison),
compiled with gcc into a temporary library on the CPU. The exhaustive
set-definition brute force, the hand-derived worked examples and the
periodic closed form are then run against it; at least one must fail. This
shows the pins are strong enough to catch mistakes of that kind in the oracle
itself.
"""

from __future__ import annotations

import os

import numpy as np
import pytest

import oracle
from checkers import all_histories, brute_force_set
from test_oracle_pins import read_golden

SRC = os.path.join(os.path.dirname(oracle.__file__), "pld_oracle.c")

MUTANTS = {
    "self_match_allowed": ("for (int64_t j = L - m - 1; j >= 0; j--)",
                           "for (int64_t j = L - m; j >= 0; j--)"),
    "skips_start_zero": ("j >= 0; j--", "j > 0; j--"),
    "oldest_first": ("for (int64_t j = L - m - 1; j >= 0; j--)",
                     "for (int64_t j = 0; j <= L - m - 1; j++)"),
    "shortest_first": ("for (int64_t m = m_top; m >= n_min; m--)",
                       "for (int64_t m = n_min; m <= m_top; m++)"),
    "n_min_exclusive": ("m >= n_min; m--", "m > n_min; m--"),
    # (capping at L instead of L - 1 would be an equivalent mutant: a suffix
    # of L tokens has no admissible start, so that loop never runs)
    "m_top_too_small": ("(L - 1 < (int64_t)n_max) ? L - 1",
                        "(L - 2 < (int64_t)n_max) ? L - 2"),
    "ignores_n_max": ("(L - 1 < (int64_t)n_max) ? L - 1 : (int64_t)n_max",
                      "L - 1"),
    "continuation_off_by_one": ("draft[t] = h[j + m + t];",
                                "draft[t] = h[j + m + t - 1];"),
    "draft_len_short": ("int64_t follow = L - (j + m);",
                        "int64_t follow = L - (j + m) - 1;"),
    "compare_one_token_short": ("same_tokens(h + j, suffix, m)",
                                "same_tokens(h + j, suffix, m - 1)"),
    "padding_zero": ("draft[t] = -1;", "draft[t] = 0;"),
    "match_reports_draft_len": ("*out_match = (int32_t)m;",
                                "*out_match = (int32_t)d;"),
    "no_k_max_cap": ("int64_t d = follow < (int64_t)k_max ? follow : (int64_t)k_max;",
                     "int64_t d = follow;"),
}


def _pins_fail(lib) -> bool:
    for case in read_golden():
        h = np.array(case.get("history", []), dtype=np.int32)
        n_min, n_max, k_max = case["params"]
        try:
            d, dl, ml, pos = oracle.draft([h], n_min, n_max, k_max, lib=lib)
        except oracle.OracleError:
            return True
        if ((int(ml[0]), int(pos[0]), int(dl[0])) != tuple(case["expect"])
                or d[0].tolist() != case["draft"]):
            return True
    for params in [(1, 3, 2), (2, 4, 3), (1, 9, 9)]:
        for L in range(0, 8):
            H = all_histories(3, L)
            want = brute_force_set(H, *params)
            got = oracle.draft(list(H), *params, lib=lib)
            if not all(np.array_equal(np.asarray(a), np.asarray(b))
                       for a, b in zip(want, (got[0], got[1], got[2], got[3]))):
                return True
    return False


@pytest.mark.parametrize("name", sorted(MUTANTS))
def test_mutant_is_caught(name, tmp_path):
    src = open(SRC).read()
    old, new = MUTANTS[name]
    assert old in src, f"mutation site for {name} no longer in the oracle"
    mutated = src.replace(old, new, 1)
    c = tmp_path / f"{name}.c"
    so = tmp_path / f"{name}.so"
    c.write_text(mutated)
    oracle.compile_lib(str(so), oracle.sources({"pld_oracle.c": str(c)}), strict=False)
    lib = oracle.load(str(so))
    assert _pins_fail(lib), f"mutant {name} passed every pin"


def test_unmutated_oracle_passes_same_pins():
    assert not _pins_fail(oracle.load())
