"""Planted mistakes in the fusion oracle must be caught by its pins.

Each mutant is a copy of ``oracle/fuse_oracle.c`` with one plausible slip in
a rule of the HyperQwen page's steps 2 and 3 (a threshold off by one, a
dropped condition, a wrong count), compiled with gcc into a temporary library
on the CPU. The hand-derived cases, the window form of the schedule and the
block invariants are then run against it; at least one must fail.
"""

from __future__ import annotations

import os

import pytest

import oracle
from test_fuse_oracle_pins import (block_invariant_errors, read_fuse_cases, run_case,
                                   window_form_errors)

HERE = os.path.dirname(oracle.__file__)
SRC = os.path.join(HERE, "fuse_oracle.c")

MUTANTS = {
    "replace_needs_more": ("int replace_head = m >= p->replace_min ||",
                           "int replace_head = m > p->replace_min ||"),
    "agree_min_exclusive": ("(m >= p->agree_min && agree)", "(m > p->agree_min && agree)"),
    "agreement_ignored": ("(m >= p->agree_min && agree)", "(m >= p->agree_min)"),
    "agree_one_token": ("t < p->agree_tokens; t++", "t < p->agree_tokens - 1; t++"),
    "agree_without_lookup_tokens": ("int agree = d >= p->agree_tokens;", "int agree = 1;"),
    "tail_min_exclusive": ("if (is_long && m >= p->tail_min) {",
                           "if (is_long && m > p->tail_min) {"),
    "tail_outside_long_block": ("if (is_long && m >= p->tail_min) {",
                                "if (m >= p->tail_min) {"),
    "tail_past_lookup_draft": ("while (n < p->positions_long && n < d) {",
                               "while (n < p->positions_long) {"),
    "fill_tail_test_drops_length": ("int fills_tail = m >= p->tail_min && d >= p->positions_long;",
                                    "int fills_tail = m >= p->tail_min;"),
    "entry_without_run": ("int entry = fills_tail && streak >= p->entry_steps;",
                          "int entry = fills_tail;"),
    "entry_run_one_short": ("int entry = fills_tail && streak >= p->entry_steps;",
                            "int entry = fills_tail && streak >= p->entry_steps - 1;"),
    "run_not_reset": ("streak = near_full ? streak + 1 : 0;", "streak = near_full ? streak + 1 : streak;"),
    "near_full_strict": ("int near_full = accepted >= prev_positions - p->near_full_slack;",
                         "int near_full = accepted > prev_positions - p->near_full_slack;"),
    "hold_not_rearmed": ("        is_long = 1;\n        hold = p->sticky;",
                         "        is_long = 1;\n        hold = hold > 0 ? hold : p->sticky;"),
    "hold_one_long": ("    } else if (state[ST_LONG] && hold > 0) {",
                      "    } else if (state[ST_LONG] && hold >= 0) {"),
    "hold_one_short": ("        hold = p->sticky;", "        hold = p->sticky - 1;"),
    "head_keeps_drafter_past_draft": ("if (replace_head && t < d) {", "if (replace_head) {"),
    "next_test_uses_long_size": ("state[ST_PREV_POSITIONS] = n;",
                                 "state[ST_PREV_POSITIONS] = is_long ? p->positions_long : p->head;"),
    "padding_zero": ("        block[t] = -1;", "        block[t] = 0;"),
}


def _pins_fail(lib) -> bool:
    for case in read_fuse_cases():
        try:
            if run_case(case, lib=lib):
                return True
        except oracle.OracleError:
            return True
    for seed in range(12):
        try:
            if window_form_errors(seed, lib) is not None:
                return True
            if block_invariant_errors(seed, lib) is not None:
                return True
        except oracle.OracleError:
            return True
    return False


@pytest.mark.parametrize("name", sorted(MUTANTS))
def test_fuse_mutant_is_caught(name, tmp_path):
    src = open(SRC).read()
    old, new = MUTANTS[name]
    assert old in src, f"mutation site for {name} no longer in the oracle"
    c = tmp_path / "fuse_oracle.c"
    c.write_text(src.replace(old, new, 1))
    so = tmp_path / f"{name}.so"
    oracle.compile_lib(str(so), oracle.sources({"fuse_oracle.c": str(c)}), strict=False)
    assert _pins_fail(oracle.load(str(so))), f"mutant {name} passed every pin"


def test_unmutated_fuse_oracle_passes_same_pins():
    assert not _pins_fail(oracle.load())
