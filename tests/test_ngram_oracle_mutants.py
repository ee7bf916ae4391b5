"""Planted mistakes in the n-gram drafting oracle must be caught by its pins.

Each mutant is a copy of ``oracle/ngram_oracle.c`` with one plausible slip
in a rule of the llama.cpp page's context cache or in a reading of it (a
range off by one, a tie the wrong way, the lengths tried in the wrong order,
a threshold strict where it is not, drafted tokens left out of the
context), compiled with gcc into a temporary library on the CPU. The golden
cases, the comparison with the dictionary drafter and the closed forms are
run against it; at least one must fail.
"""

from __future__ import annotations

import itertools
import os

import numpy as np
import pytest

import oracle
import test_ngram_oracle_pins as pins

HERE = os.path.dirname(oracle.__file__)
SRC = os.path.join(HERE, "ngram_oracle.c")

MUTANTS = {
    "skips_first_position": ("for (int64_t i = n; i < L; i++)", "for (int64_t i = n + 1; i < L; i++)"),
    "successor_is_gram_end": ("succ[c++] = h[i];", "succ[c++] = h[i - 1];"),
    "tie_takes_larger": ("if (i - run_start > *top)", "if (i - run_start >= *top)"),
    "shortest_first": ("for (int n = p->n_max; n >= p->n_min && !chosen; n--)",
                       "for (int n = p->n_min; n <= p->n_max && !chosen; n++)"),
    "share_strict": ("100 * top >= (int64_t)p->min_percent[n - 1] * count",
                     "100 * top > (int64_t)p->min_percent[n - 1] * count"),
    "count_strict": ("if (count >= need &&", "if (count > need &&"),
    "unseen_context_passes": ("int64_t need = p->min_count[n - 1] > 1 ? p->min_count[n - 1] : 1;",
                              "int64_t need = p->min_count[n - 1];"),
    "share_of_length_one": ("(int64_t)p->min_percent[n - 1] * count",
                            "(int64_t)p->min_percent[0] * count"),
    "count_of_length_one": ("int64_t need = p->min_count[n - 1] > 1 ? p->min_count[n - 1] : 1;",
                            "int64_t need = p->min_count[0] > 1 ? p->min_count[0] : 1;"),
    "context_ignores_draft": ("ctx[t] = q < L ? h[q] : draft[q - L];",
                              "ctx[t] = h[q < L ? q : L - 1];"),
    "context_off_by_one": ("int64_t q = len - n + t;", "int64_t q = len - n + t - 1;"),
    "level_off_by_one": ("levels[s] = chosen;", "levels[s] = chosen - 1;"),
    "gap_instead_of_stop": ("        if (!chosen)\n            break;",
                            "        if (!chosen)\n            continue;"),
    "unsigned_tie_order": ("return (x > y) - (x < y);",
                           "return ((uint32_t)x > (uint32_t)y) - ((uint32_t)x < (uint32_t)y);"),
}


def _pins_fail(lib) -> bool:
    try:
        for case in pins.CASES:
            d, n, lv = oracle.ngram_draft(case["params"], [case["history"]], case["k"], lib=lib)
            if d[0].tolist() != case["draft"] or lv[0].tolist() != case["levels"]:
                return True
        hs = [np.array(t, np.int32) for L in range(8)
              for t in itertools.product(range(3), repeat=L)]
        for p in pins.EXHAUSTIVE_PARAMS:
            d, n, lv = oracle.ngram_draft(p, hs, 5, lib=lib)
            for b, h in enumerate(hs):
                wd, wn, wl = pins.dict_draft(h, p, 5)
                if d[b].tolist() != wd or int(n[b]) != wn or lv[b].tolist() != wl:
                    return True
        block = np.array([7 * i - 20 for i in range(5)], np.int32)
        for L in range(9, 20):
            d, n, lv = oracle.ngram_draft(pins.P(), [np.resize(block, L)], 16, lib=lib)
            if d[0].tolist() != [int(block[(L + s) % 5]) for s in range(16)] or (lv != 4).any():
                return True
    except oracle.OracleError:
        return True
    return False


@pytest.mark.parametrize("name", sorted(MUTANTS))
def test_ngram_mutant_is_caught(name, tmp_path):
    src = open(SRC).read()
    old, new = MUTANTS[name]
    assert old in src, f"mutation site for {name} no longer in the oracle"
    c = tmp_path / "ngram_oracle.c"
    c.write_text(src.replace(old, new, 1))
    so = tmp_path / f"{name}.so"
    oracle.compile_lib(str(so), oracle.sources({"ngram_oracle.c": str(c)}), strict=False)
    assert _pins_fail(oracle.load(str(so))), f"mutant {name} passed every pin"


def test_unmutated_ngram_oracle_passes_same_pins():
    assert not _pins_fail(oracle.load())
