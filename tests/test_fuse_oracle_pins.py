"""Pins for the draft-fusion and long-block-scheduling oracle.

The oracle (``oracle/fuse_oracle.c``) follows the HyperQwen lookup-drafting
page, steps 2 and 3 of its three-step principle. It is pinned here by:

- hand-derived cases of every head and tail rule and a hand-derived
  multi-step schedule (``tests/golden/fuse_cases.txt``);
- a second formulation of the schedule over whole random traces: a step is
  long exactly when the entry condition held on it or on one of the `sticky`
  steps before it, and the entry condition is the tail test plus a window of
  `entry_steps` near-full steps (the oracle uses counters instead);
- structural invariants of every fused block over random traces;
- special cases that reduce to drafter-only and to lookup-only drafting.
"""

from __future__ import annotations

import os

import numpy as np
import pytest

import oracle
from prompt_lookup_gram_amd import workloads as wl

GOLDEN = os.path.join(os.path.dirname(__file__), "golden", "fuse_cases.txt")
K_LOOKUP = 16


def read_fuse_cases(path=GOLDEN):
    cases, cur, drafter, lookup = [], None, None, None
    with open(path) as f:
        for raw in f:
            line = raw.strip()
            if not line or line.startswith("#"):
                continue
            key, _, rest = line.partition(" ")
            if key == "case":
                cur = {"name": rest, "steps": []}
                continue
            if key == "end":
                cases.append(cur)
                cur = None
                continue
            vals = [int(x) for x in rest.split()]
            if key == "params":
                cur["params"] = vals
            elif key == "drafter":
                drafter = vals
            elif key == "lookup":
                lookup = vals
            elif key == "step":
                d, m, acc, e_long, e_pos, e_src = vals
                cur["steps"].append({"drafter": drafter, "lookup": lookup, "d": d, "m": m,
                                     "accepted": acc, "long": e_long, "positions": e_pos,
                                     "src": e_src})
            elif key == "block":
                cur["steps"][-1]["block"] = vals
            else:
                raise ValueError(f"unknown line {line!r}")
    return cases


def run_case(case, lib=None):
    """Apply a golden case's steps to one request; returns the mismatches."""
    params = oracle.FuseParams(*case["params"])
    state = np.zeros((1, oracle.FUSE_STATE_WORDS), np.int32)
    bad = []
    for i, s in enumerate(case["steps"]):
        block, pos, src, state = oracle.fuse(
            params, np.array([s["lookup"]], np.int32), [s["d"]], [s["m"]],
            np.array([s["drafter"]], np.int32), [s["accepted"]], state, lib=lib)
        got = (int(state[0, 0]), int(pos[0]), int(src[0]), block[0].tolist())
        want = (s["long"], s["positions"], s["src"], s["block"])
        if got != want:
            bad.append((i, got, want))
    return bad


@pytest.mark.parametrize("case", read_fuse_cases(), ids=lambda c: c["name"])
def test_fuse_golden(case):
    assert run_case(case) == []


def test_golden_cover_every_rule():
    """The hand-derived set exercises each rule of steps 2 and 3."""
    steps = [s for c in read_fuse_cases() for s in c["steps"]]
    assert any(s["m"] >= 8 and s["src"] & 1 for s in steps)                 # replace at 8
    assert any(6 <= s["m"] < 8 and s["src"] & 1 for s in steps)             # agree at 6..7
    assert any(6 <= s["m"] < 8 and not s["src"] & 1 for s in steps)         # disagree
    assert any(4 <= s["m"] < 6 and s["positions"] > 7 for s in steps)       # tail at 4..5
    assert any(s["long"] and s["positions"] == 7 for s in steps)            # held, empty tail
    assert any(0 < s["d"] < 15 and s["long"] and 7 < s["positions"] < 15 for s in steps)


# ---------------------------------------------------------------------------
# random traces
# ---------------------------------------------------------------------------


def random_params(rng):
    return oracle.FuseParams(**wl.fuse_params_draw(rng))


def random_trace(rng, params, batch, steps):
    """Random lookup results and drafter proposals (the shared seeded
    generator); accepted counts are drawn by run_trace from the previous
    block's positions."""
    for _ in range(steps):
        yield wl.fuse_step_draws(rng, batch, params.head, K_LOOKUP)


def run_trace(params, trace, rng, batch, lib=None):
    state = np.zeros((batch, oracle.FUSE_STATE_WORDS), np.int32)
    prev_pos = np.zeros(batch, np.int32)
    rows = []
    for lookup, d, m, drafter in trace:
        acc = np.array([rng.integers(0, p + 1) for p in prev_pos], np.int32)
        block, pos, src, state = oracle.fuse(params, lookup, d, m, drafter, acc, state, lib=lib)
        rows.append(dict(lookup=lookup, d=d, m=m, drafter=drafter, acc=acc, block=block,
                         pos=pos, src=src, long=state[:, 0].copy()))
        prev_pos = pos
    return rows


def window_form_errors(seed, lib=None):
    """Long exactly when the entry condition held within the last `sticky`
    steps; entry = tail fillable and the last `entry_steps` steps near-full.
    Returns the first disagreement, or None."""
    rng = np.random.default_rng([7001, seed])
    params = random_params(rng)
    batch, steps = 6, 60
    rows = run_trace(params, random_trace(rng, params, batch, steps), rng, batch, lib)
    for b in range(batch):
        near = []   # near-full flag of each finished step
        entry = []
        for t, r in enumerate(rows):
            if t > 0:
                near.append(bool(r["acc"][b] >= rows[t - 1]["pos"][b] - params.near_full_slack))
            fills = r["m"][b] >= params.tail_min and r["d"][b] >= params.positions_long
            window = near[t - params.entry_steps:t] if params.entry_steps else []
            enough = t >= params.entry_steps and all(window)
            entry.append(bool(fills and enough))
            is_long = any(entry[max(0, t - params.sticky):t + 1])
            tail = 0
            if is_long and r["m"][b] >= params.tail_min:
                tail = max(0, min(int(r["d"][b]), params.positions_long) - params.head)
            if bool(r["long"][b]) != is_long or r["pos"][b] != params.head + tail:
                return (b, t)
    return None


@pytest.mark.parametrize("seed", range(12))
def test_schedule_window_form(seed):
    assert window_form_errors(seed) is None


def block_invariant_errors(seed, lib=None):
    """Structural checks of every fused block of a random trace; returns the
    first failure, or None."""
    rng = np.random.default_rng([7002, seed])
    params = random_params(rng)
    batch = 8
    rows = run_trace(params, random_trace(rng, params, batch, 40), rng, batch, lib)
    try:
        _check_blocks(params, rows, batch)
    except AssertionError as e:
        return str(e) or "invariant"
    return None


def _check_blocks(params, rows, batch):
    for r in rows:
        for b in range(batch):
            n, bits = int(r["pos"][b]), int(r["src"][b])
            assert params.head <= n <= params.positions_long
            for t in range(params.positions_long):
                from_lookup = bool(bits >> t & 1)
                if t >= n:
                    assert r["block"][b, t] == -1 and not from_lookup
                elif from_lookup:
                    assert t < r["d"][b] and r["block"][b, t] == r["lookup"][b, t]
                else:
                    assert t < params.head and r["block"][b, t] == r["drafter"][b, t]
            # lookup positions in the head form a prefix of the lookup draft;
            # every tail position comes from the lookup
            head_bits = bits & ((1 << params.head) - 1)
            assert head_bits & (head_bits + 1) == 0
            assert head_bits in (0, (1 << min(int(r["d"][b]), params.head)) - 1)
            tail_mask = ((1 << n) - 1) & ~((1 << params.head) - 1)
            assert bits & tail_mask == tail_mask


@pytest.mark.parametrize("seed", range(12))
def test_block_invariants(seed):
    assert block_invariant_errors(seed) is None


def test_drafter_only_when_thresholds_unreachable():
    rng = np.random.default_rng(7003)
    params = oracle.FuseParams(replace_min=99, agree_min=99, tail_min=99)
    rows = run_trace(params, random_trace(rng, params, 5, 30), rng, 5)
    for r in rows:
        assert (r["pos"] == params.head).all() and (r["src"] == 0).all()
        assert (r["block"][:, :params.head] == r["drafter"]).all()
        assert (r["block"][:, params.head:] == -1).all()


def test_lookup_only_without_run_or_hold():
    """Thresholds of 1, no near-full run, no hold: every step takes the lookup
    draft as far as it goes, long exactly when it covers the long block."""
    rng = np.random.default_rng(7004)
    params = oracle.FuseParams(replace_min=1, agree_min=1, tail_min=1, entry_steps=0,
                               sticky=0)
    rows = run_trace(params, random_trace(rng, params, 5, 30), rng, 5)
    for r in rows:
        for b in range(5):
            d = int(r["d"][b])
            full = d >= params.positions_long
            assert bool(r["long"][b]) == full
            n = params.positions_long if full else params.head
            assert r["pos"][b] == n
            k = min(d, n)
            assert (r["block"][b, :k] == r["lookup"][b, :k]).all()
            assert (r["block"][b, k:params.head] == r["drafter"][b, k:params.head]).all()


def test_rejects_bad_arguments():
    p = oracle.FuseParams()
    z = np.zeros((1, oracle.FUSE_STATE_WORDS), np.int32)
    look = np.full((1, K_LOOKUP), -1, np.int32)
    dr = np.zeros((1, 7), np.int32)
    with pytest.raises(oracle.OracleError):   # accepted above the previous block
        oracle.fuse(p, look, [0], [0], dr, [8], np.array([[0, 0, 0, 7]], np.int32))
    with pytest.raises(oracle.OracleError):   # draft length past the row
        oracle.fuse(p, look, [17], [4], dr, [0], z)
    with pytest.raises(oracle.OracleError):   # head longer than the long block
        oracle.fuse(oracle.FuseParams(head=7, positions_long=6, agree_tokens=2), look,
                    [0], [0], dr, [0], z)
