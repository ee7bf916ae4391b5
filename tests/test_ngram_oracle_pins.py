"""Pins for the successor-count n-gram drafting oracle (llama.cpp page, its
context cache), ``oracle/ngram_oracle.c``.

The oracle recounts every context's successors from the history by brute
force. It is pinned against things other than itself:
- hand-derived golden cases (``tests/golden/ngram_cases.txt``), one per
  rule and reading: fallback order, tie order, drafted tokens in the
  context, both thresholds at their boundaries, short and empty histories;
- an independent drafter written here the way the page describes the
  cache: a dictionary from each n-gram to a counter of its successors,
  updated token by token as the stream grows, compared on every history
  over a 3-symbol alphabet up to 7 tokens and on random histories;
- closed forms: a periodic stream of distinct tokens drafts its own
  continuation, from the longest length, for every k_max;
- a special case that reduces to a library routine (the mode of the
  successors of the last token, numpy's unique counts);
- the first token's existence when no threshold can fail.
"""

from __future__ import annotations

import itertools
import os
from collections import Counter, defaultdict

import numpy as np
import pytest

import oracle

P = oracle.NgramParams
GOLDEN = os.path.join(os.path.dirname(__file__), "golden", "ngram_cases.txt")


def read_cases(path=GOLDEN):
    cases, cur = [], None
    for raw in open(path):
        line = raw.split("#", 1)[0].strip()
        if not line:
            continue
        word, _, rest = line.partition(" ")
        vals = [int(v) for v in rest.split()] if word != "case" else None
        if word == "case":
            cur = {"name": rest.strip()}
        elif word == "params":
            cur["params"] = P(vals[0], vals[1], tuple(vals[2:6]), tuple(vals[6:10]))
        elif word == "history":
            cur["history"] = np.array(vals, np.int32)
        elif word == "k":
            cur["k"] = vals[0]
        elif word in ("draft", "levels"):
            cur[word] = vals
        elif word == "end":
            cases.append(cur)
            cur = None
        else:
            raise ValueError(f"unknown line {raw!r}")
    return cases


CASES = read_cases()


@pytest.mark.parametrize("case", CASES, ids=[c["name"] for c in CASES])
def test_ngram_golden(case):
    d, n, lv = oracle.ngram_draft(case["params"], [case["history"]], case["k"])
    want_len = sum(1 for t in case["levels"] if t > 0)
    assert d[0].tolist() == case["draft"]
    assert lv[0].tolist() == case["levels"]
    assert int(n[0]) == want_len


def test_golden_cover_every_rule():
    """The hand cases exercise every reading at least once."""
    levels = {lv for c in CASES for lv in c["levels"]}
    assert {0, 1, 2, 3, 4} <= levels                        # every length, and "none"
    names = {c["name"] for c in CASES}
    for needed in ("tie_fallback_and_drafted_context", "share_threshold_boundary",
                   "share_threshold_just_above", "min_count_two_blocks_everything",
                   "signed_tie_order", "only_length_four", "empty_history",
                   "stop_at_first_miss"):
        assert needed in names


# ---------------------------------------------------------------------------
# an independent drafter: the cache as a dictionary, grown token by token
# ---------------------------------------------------------------------------


def dict_draft(h, p, k):
    """Drafts from a context cache kept the way the page describes it: for
    each size n an n-gram -> successor-counter map, updated as each token
    of the stream arrives."""
    cache = defaultdict(lambda: defaultdict(Counter))
    seen = []
    for tok in (int(t) for t in h):
        for n in range(1, oracle.NGRAM_MAX_N + 1):
            if len(seen) >= n:
                cache[n][tuple(seen[-n:])][tok] += 1
        seen.append(tok)
    stream = list(seen)
    draft, levels = [], []
    for _ in range(k):
        pick = None
        for n in range(p.n_max, p.n_min - 1, -1):
            if len(stream) < n:
                continue
            succ = cache[n].get(tuple(stream[-n:]))
            if not succ:
                continue
            count = sum(succ.values())
            top = max(succ.values())
            if count >= max(1, p.min_count[n - 1]) and 100 * top >= p.min_percent[n - 1] * count:
                pick = (min(t for t, c in succ.items() if c == top), n)
                break
        if pick is None:
            break
        draft.append(pick[0])
        levels.append(pick[1])
        stream.append(pick[0])
    pad = k - len(draft)
    return draft + [-1] * pad, len(draft), levels + [0] * pad


def compare(p, hs, k):
    d, n, lv = oracle.ngram_draft(p, hs, k)
    for b, h in enumerate(hs):
        wd, wn, wl = dict_draft(h, p, k)
        if d[b].tolist() != wd or int(n[b]) != wn or lv[b].tolist() != wl:
            return (b, h.tolist(), d[b].tolist(), wd, lv[b].tolist(), wl)
    return None


EXHAUSTIVE_PARAMS = [P(), P(min_count=(0, 0, 0, 0), min_percent=(0, 0, 0, 0)), P(1, 2),
                     P(2, 4, (1, 2, 1, 1)),
                     P(min_percent=(67, 51, 100, 34), min_count=(2, 1, 1, 2))]


@pytest.mark.parametrize("pi", range(len(EXHAUSTIVE_PARAMS)))
def test_exhaustive_tiny_against_dict_drafter(pi):
    hs = [np.array(t, np.int32) for L in range(8) for t in itertools.product(range(3), repeat=L)]
    assert compare(EXHAUSTIVE_PARAMS[pi], hs, 5) is None


def random_params(rng):
    n_min = int(rng.integers(1, 5))
    n_max = int(rng.integers(n_min, 5))
    mc = tuple(int(v) for v in rng.integers(0, 4, 4))
    mp = tuple(int(v) for v in rng.choice([0, 33, 34, 50, 51, 66, 67, 100], 4))
    return P(n_min, n_max, mc, mp)


@pytest.mark.parametrize("seed", range(12))
def test_random_against_dict_drafter(seed):
    rng = np.random.default_rng([9103, seed])
    p = random_params(rng)
    alphabet = int(rng.choice([2, 3, 5, 9]))
    hs = []
    for _ in range(40):
        L = int(rng.integers(0, 160))
        h = rng.integers(-alphabet // 2, alphabet - alphabet // 2, L).astype(np.int32)
        if L > 20 and rng.random() < 0.5:             # a copied span
            s = int(rng.integers(0, L // 2))
            t = int(rng.integers(4, L // 2))
            h = np.concatenate([h, h[s:s + t]])
        hs.append(h)
    assert compare(p, hs, int(rng.integers(1, 17))) is None


# ---------------------------------------------------------------------------
# closed forms and special cases
# ---------------------------------------------------------------------------


@pytest.mark.parametrize("period", [1, 2, 3, 5, 8, 13])
@pytest.mark.parametrize("n_max", [1, 2, 4])
def test_periodic_stream_drafts_its_continuation(period, n_max):
    """A stream repeating `period` distinct tokens: every context of any
    length fixes the position modulo the period, so each context has one
    successor (a 100% share) and the draft continues the cycle for all
    k_max tokens, from the longest allowed length, once the history holds
    a followed occurrence of it (L >= period + n_max)."""
    block = np.array([7 * i - 20 for i in range(period)], np.int32)
    hs, want = [], []
    for L in range(period + n_max, period + n_max + 2 * period + 1):
        hs.append(np.resize(block, L))
        want.append([int(block[(L + s) % period]) for s in range(16)])
    d, n, lv = oracle.ngram_draft(P(1, n_max), hs, 16)
    assert d.tolist() == want
    assert (n == 16).all() and (lv == n_max).all()


@pytest.mark.parametrize("seed", range(6))
def test_length_one_is_the_successor_mode(seed):
    """n = 1 only, no share threshold, one token: the draft is the most
    frequent token right after an earlier occurrence of the last token (the
    smallest such token on a tie), computed here with numpy's unique counts;
    no draft when the last token never occurred before the end."""
    rng = np.random.default_rng([9104, seed])
    hs = [rng.integers(0, int(rng.integers(2, 30)), int(rng.integers(1, 400))).astype(np.int32)
          for _ in range(50)]
    d, n, lv = oracle.ngram_draft(P(1, 1, min_percent=(0, 0, 0, 0)), hs, 1)
    for b, h in enumerate(hs):
        idx = np.nonzero(h[:-1] == h[-1])[0]
        if idx.size == 0:
            assert n[b] == 0 and d[b, 0] == -1 and lv[b, 0] == 0
            continue
        vals, counts = np.unique(h[idx + 1], return_counts=True)   # sorted values
        assert n[b] == 1 and lv[b, 0] == 1
        assert d[b, 0] == vals[np.argmax(counts)]                   # first maximum


@pytest.mark.parametrize("seed", range(4))
def test_first_token_exists_without_thresholds(seed):
    """With no share threshold and a count of 1, a first token is drafted
    exactly when the last token occurred before the end of the history (its
    1-gram is then followed), whatever the longer lengths say."""
    rng = np.random.default_rng([9105, seed])
    hs = [rng.integers(0, 40, int(rng.integers(0, 300))).astype(np.int32) for _ in range(60)]
    _, n, _ = oracle.ngram_draft(P(min_percent=(0, 0, 0, 0)), hs, 3)
    for b, h in enumerate(hs):
        followed = h.size >= 2 and bool((h[:-1] == h[-1]).any())
        assert (n[b] > 0) == followed


@pytest.mark.parametrize("bad", [P(0, 4), P(2, 1), P(1, 5), P(min_percent=(50, 101, 50, 50)),
                                 P(min_count=(1, -1, 1, 1))])
def test_rejects_bad_params(bad):
    with pytest.raises(oracle.OracleError):
        oracle.ngram_draft(bad, [np.arange(10, dtype=np.int32)], 4)


def test_rejects_bad_k():
    with pytest.raises(oracle.OracleError):
        oracle.ngram_draft(P(), [np.arange(10, dtype=np.int32)], 0)
