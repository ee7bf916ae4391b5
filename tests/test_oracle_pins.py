"""Pins for the CPU oracle: each test checks it against something other than
itself (see ``checkers.py`` and ``golden/worked_examples.txt``).

Rule pinned: HyperQwen lookup-drafting page, step 1 of the three-step
principle (longest n_min..n_max suffix, most recent earlier occurrence,
overlap allowed, following tokens as the draft), draft capped at k_max.
"""

from __future__ import annotations

import os

import numpy as np
import pytest

import oracle
from checkers import (all_histories, brute_force_set, by_z_function,
                      certificate_errors, z_function)
from prompt_lookup_gram_amd import workloads as wl

GOLDEN = os.path.join(os.path.dirname(__file__), "golden", "worked_examples.txt")


def read_golden(path=GOLDEN):
    cases, cur = [], None
    with open(path) as f:
        for raw in f:
            line = raw.strip()
            if not line or line.startswith("#"):
                continue
            key, _, rest = line.partition(" ")
            vals = [int(x) for x in rest.split()] if key != "case" else rest
            if key == "case":
                cur = {"name": vals}
            elif key == "end":
                cases.append(cur)
                cur = None
            else:
                cur[key] = vals
    return cases


# ---------------------------------------------------------------------------
# hand-derived worked examples
# ---------------------------------------------------------------------------


@pytest.mark.parametrize("case", read_golden(), ids=lambda c: c["name"])
def test_worked_examples(case):
    h = np.array(case.get("history", []), dtype=np.int32)
    n_min, n_max, k_max = case["params"]
    m, j, d = case["expect"]
    draft, dl, ml, pos = oracle.draft([h], n_min, n_max, k_max)
    assert (int(ml[0]), int(pos[0]), int(dl[0])) == (m, j, d)
    assert draft[0].tolist() == case["draft"]


def test_golden_file_has_cases():
    names = [c["name"] for c in read_golden()]
    assert len(names) >= 10 and len(set(names)) == len(names)


# ---------------------------------------------------------------------------
# exhaustive brute force over the set definition
# ---------------------------------------------------------------------------

PARAMS_TINY = [(1, 1, 1), (1, 3, 2), (2, 4, 3), (1, 9, 9), (3, 3, 5), (2, 2, 1),
               (4, 12, 16)]


def _compare_exhaustive(alphabet, length, params):
    H = all_histories(alphabet, length)
    n_min, n_max, k_max = params
    bd, bl, bm, bj = brute_force_set(H, n_min, n_max, k_max)
    od, ol, om, oj = oracle.draft(list(H), n_min, n_max, k_max)
    bad = np.nonzero((bm != om) | (bj != oj) | (bl != ol)
                     | np.any(bd != od, axis=1))[0]
    assert bad.size == 0, (
        f"alphabet={alphabet} L={length} params={params} "
        f"first mismatch history={H[bad[0]].tolist()} "
        f"oracle=({om[bad[0]]},{oj[bad[0]]},{ol[bad[0]]},{od[bad[0]].tolist()}) "
        f"brute=({bm[bad[0]]},{bj[bad[0]]},{bl[bad[0]]},{bd[bad[0]].tolist()})")
    return H.shape[0]


@pytest.mark.parametrize("params", PARAMS_TINY)
def test_exhaustive_alphabet3(params):
    n = sum(_compare_exhaustive(3, L, params) for L in range(0, 10))
    assert n == sum(3 ** L for L in range(10))


@pytest.mark.parametrize("params", [(1, 3, 2), (2, 4, 3), (1, 9, 9)])
def test_exhaustive_alphabet4(params):
    for L in range(0, 8):
        _compare_exhaustive(4, L, params)


def test_exhaustive_binary_long():
    # alphabet 2 up to L = 13: long runs and many overlapping matches
    for L in range(10, 14):
        _compare_exhaustive(2, L, (2, 6, 4))


# ---------------------------------------------------------------------------
# Z-function (textbook) cross-check at full workload sizes
# ---------------------------------------------------------------------------


def test_z_function_textbook_values():
    # hand-checkable Z-arrays
    assert z_function("aaaaa").tolist() == [5, 4, 3, 2, 1]
    assert z_function("aabxaab").tolist() == [7, 1, 0, 0, 3, 1, 0]
    assert z_function("abacaba").tolist() == [7, 0, 1, 0, 3, 0, 1]


def _check_by_z(histories, n_min, n_max, k_max):
    od, ol, om, oj = oracle.draft(histories, n_min, n_max, k_max)
    for b, h in enumerate(histories):
        zd, zl, zm, zj = by_z_function(h, n_min, n_max, k_max)
        assert (int(om[b]), int(oj[b]), int(ol[b])) == (zm, zj, zl), f"request {b}"
        assert np.array_equal(od[b], zd), f"request {b}"


def test_z_crosscheck_config1():
    w = wl.config1()
    _check_by_z(w.histories, w.n_min, w.n_max, w.k_max)


def test_z_crosscheck_config2():
    w = wl.config2()
    _check_by_z(w.histories, w.n_min, w.n_max, w.k_max)


def test_z_crosscheck_config3_every_request():
    w = wl.config3()
    assert w.batch == 64
    _check_by_z(w.histories, w.n_min, w.n_max, w.k_max)


def test_z_crosscheck_config4_every_request():
    w = wl.config4()
    assert w.batch == 16
    _check_by_z(w.histories, w.n_min, w.n_max, w.k_max)


def test_z_crosscheck_config5_start_every_request():
    w = wl.config5_start()
    _check_by_z(w.histories, w.n_min, w.n_max, w.k_max)


@pytest.mark.parametrize("seed", range(6))
def test_z_crosscheck_fuzz(seed):
    w = wl.fuzz_batch(seed, max_batch=8, max_len=3000)
    _check_by_z(w.histories, w.n_min, w.n_max, w.k_max)


# ---------------------------------------------------------------------------
# certificate + continuation invariant over every request of every workload
# ---------------------------------------------------------------------------


def _check_certificates(w):
    od, ol, om, oj = oracle.draft(w.histories, w.n_min, w.n_max, w.k_max)
    for b, h in enumerate(w.histories):
        errs = certificate_errors(h, w.n_min, w.n_max, w.k_max, od[b], ol[b],
                                  om[b], oj[b])
        assert not errs, f"{w.name} request {b}: {errs}"
        # continuation invariant: draft token t is the history right after
        # the occurrence, and the length is min(k_max, tokens left)
        if om[b]:
            p = int(oj[b]) + int(om[b])
            assert int(ol[b]) == min(w.k_max, h.size - p)
            for t in range(int(ol[b])):
                assert od[b, t] == h[p + t]
    return od, ol, om, oj


@pytest.mark.parametrize("cfg", [1, 2, 3, 4])
def test_certificates_configs(cfg):
    w = wl.ALL_CONFIGS[cfg]()
    od, ol, om, oj = _check_certificates(w)
    if cfg == 1:
        # planted 512-token copy of uniform tokens: full-length match
        assert om[0] == 12 and ol[0] == 16


def test_certificates_stream_start():
    _check_certificates(wl.config5_start())


@pytest.mark.parametrize("seed", range(10))
def test_certificates_fuzz(seed):
    _check_certificates(wl.fuzz_batch(seed))


# ---------------------------------------------------------------------------
# closed forms: periodic tails and planted copies
# ---------------------------------------------------------------------------


@pytest.mark.parametrize("p", list(range(1, 25)))
@pytest.mark.parametrize("n_max,k_max", [(12, 16), (4, 2), (12, 1), (30, 40)])
def test_periodic_tail(p, n_max, k_max):
    """A tail with period p whose block has p distinct tokens, at least
    n_max + p long: the n_max-suffix recurs one period back (overlapping the
    suffix when p < n_max) and at no smaller shift, so m = n_max,
    j = L - n_max - p, and exactly p tokens follow the occurrence."""
    rng = np.random.default_rng([7, p, n_max, k_max])
    block = rng.permutation(1000)[:p].astype(np.int32)
    # an earlier copy of the same periodic run must lose to the later one
    prefix = np.concatenate([rng.integers(2000, 9000, 50).astype(np.int32),
                             np.tile(block, 40)[:3 * n_max],
                             rng.integers(2000, 9000, 37).astype(np.int32)])
    tail_len = n_max + p + int(rng.integers(0, 3 * p + 1))
    tail = np.tile(block, tail_len // p + 2)[:tail_len]
    h = np.concatenate([prefix, tail]).astype(np.int32)
    L = h.size
    od, ol, om, oj = oracle.draft([h], 2, n_max, k_max)
    d = min(k_max, p)
    assert int(om[0]) == n_max
    assert int(oj[0]) == L - n_max - p
    assert int(ol[0]) == d
    assert od[0, :d].tolist() == h[L - p:L - p + d].tolist()
    assert np.all(od[0, d:] == -1)


@pytest.mark.parametrize("trial", range(12))
def test_planted_copy(trial):
    """Distinct tokens (a permutation, so no accidental repeats) whose last
    T >= n_max tokens are replaced by a copy of h[s:s+T] with s+T <= D-T:
    the n_max-suffix occurs exactly once earlier, at j = s+T-n_max, and the
    draft is what followed the copied span in the source."""
    rng = np.random.default_rng([11, trial])
    D = int(rng.integers(40, 4000))
    n_max = int(rng.integers(1, 20))
    T = int(rng.integers(n_max, max(n_max + 1, D // 2)))
    s = int(rng.integers(0, D - 2 * T + 1))
    k_max = int(rng.integers(1, 40))
    h = rng.permutation(10 * D).astype(np.int32)[:D]
    h[D - T:] = h[s:s + T]
    od, ol, om, oj = oracle.draft([h], 1, n_max, k_max)
    assert int(om[0]) == n_max
    assert int(oj[0]) == s + T - n_max
    d = min(k_max, D - (s + T))
    assert int(ol[0]) == d
    assert od[0, :d].tolist() == h[s + T:s + T + d].tolist()


# ---------------------------------------------------------------------------
# argument handling and degenerate cases
# ---------------------------------------------------------------------------


@pytest.mark.parametrize("bad", [(0, 4, 3), (5, 4, 3), (1, 4, 0), (-1, 2, 2)])
def test_oracle_rejects_bad_parameters(bad):
    with pytest.raises(oracle.OracleError):
        oracle.draft([np.arange(10, dtype=np.int32)], *bad)


def test_degenerate_lengths():
    hs = [np.zeros(0, np.int32), np.zeros(1, np.int32), np.zeros(4, np.int32),
          np.zeros(5, np.int32)]
    od, ol, om, oj = oracle.draft(hs, 4, 12, 3)
    # L = 0, 1, 4: the longest admissible suffix (L - 1 tokens) is below 4
    assert om[:3].tolist() == [0, 0, 0] and oj[:3].tolist() == [-1, -1, -1]
    # L = 5 of equal tokens: the 4-suffix occurs at 0, one token follows
    assert (int(om[3]), int(oj[3]), int(ol[3])) == (4, 0, 1)
    assert od[3].tolist() == [0, -1, -1]


def test_n_min_equals_n_max_and_large_k():
    h = np.array([3, 1, 4, 1, 5, 9, 2, 6, 1, 4, 1, 5], dtype=np.int32)
    od, ol, om, oj = oracle.draft([h], 3, 3, 100)
    # 3-suffix 4 1 5 occurs at 2; continuation is positions 5..11 (7 tokens)
    assert (int(om[0]), int(oj[0]), int(ol[0])) == (3, 2, 7)
    assert od[0, :7].tolist() == [9, 2, 6, 1, 4, 1, 5]
    assert np.all(od[0, 7:] == -1)


def test_batch_invariance():
    w = wl.fuzz_batch(3)
    full = oracle.draft(w.histories, w.n_min, w.n_max, w.k_max)
    for b in range(w.batch):
        one = oracle.draft([w.histories[b]], w.n_min, w.n_max, w.k_max)
        for a, c in zip(full, one):
            assert np.array_equal(a[b], c[0])


def test_stream_oracle_append():
    hs = [np.arange(5, dtype=np.int32), np.arange(3, dtype=np.int32)]
    tok = np.array([[7, 8, -1], [9, -1, -1]], dtype=np.int32)
    out = oracle.append(hs, tok, np.array([2, 1]))
    assert out[0].tolist() == [0, 1, 2, 3, 4, 7, 8]
    assert out[1].tolist() == [0, 1, 2, 9]
