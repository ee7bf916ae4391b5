"""GPU parity of successor-count n-gram drafting (pld_create_ngram,
pld_append, pld_draft_ngram) against the CPU oracle: draft rows with their
-1 padding, draft lengths and the context length behind every token must
be identical.

Inputs are seeded and synthetic (prompt_lookup_gram_amd.workloads): the
lookup workloads' histories appended whole, the streaming workload's decode
(its appends composed from the lookup oracle's drafts, so no GPU output
feeds an input), and fuzzed streams over tiny alphabets."""

from __future__ import annotations

import numpy as np
import pytest

import oracle
from prompt_lookup_gram_amd import binding as B
from prompt_lookup_gram_amd import workloads as wl

import test_ngram_oracle_pins as pins

pytestmark = pytest.mark.gpu

P = oracle.NgramParams


@pytest.fixture(scope="module", autouse=True)
def gpu():
    import torch
    assert torch.cuda.is_available(), "GPU tests need a GPU"
    B.load()
    torch.cuda.init()
    yield
    torch.cuda.synchronize()


def to_lib(p: P) -> B.PldNgramParams:
    q = B.PldNgramParams()
    q.n_min, q.n_max = p.n_min, p.n_max
    for i in range(4):
        q.min_count[i] = p.min_count[i]
        q.min_percent[i] = p.min_percent[i]
    return q


class NgramStore:
    """A context with a successor-count cache plus a host mirror of its
    histories."""

    def __init__(self, batch, max_len, n_max=4):
        self.batch, self.max_len = batch, max_len
        self.ctx = B.pld_create_ngram(batch, max_len, n_max)
        self.host = [np.zeros(0, np.int32) for _ in range(batch)]

    def append(self, rows, width=None):
        """rows: per-request int32 arrays (may be empty); width: the source
        rows' stride (at least the longest row)."""
        import torch
        width = width or max(1, max(len(r) for r in rows))
        tok = np.full((self.batch, width), -3, np.int32)
        cnt = np.zeros(self.batch, np.int32)
        for b, r in enumerate(rows):
            tok[b, :len(r)] = r
            cnt[b] = len(r)
            if len(self.host[b]) + len(r) <= self.max_len:
                self.host[b] = np.concatenate([self.host[b], np.asarray(r, np.int32)])
        B.pld_append(self.ctx, torch.from_numpy(tok).cuda(), width,
                     torch.from_numpy(cnt).cuda(), self.batch)

    def draft(self, p: P, k_max, batch=None, levels=True):
        import torch
        batch = self.batch if batch is None else batch
        d = torch.full((batch, k_max), -7, dtype=torch.int32, device="cuda")
        n = torch.full((batch,), -7, dtype=torch.int32, device="cuda")
        lv = torch.full((batch, k_max), -7, dtype=torch.int32, device="cuda") if levels else None
        B.pld_draft_ngram(self.ctx, to_lib(p), batch, k_max, d, n, lv)
        return d, n, lv

    def check(self, p: P, k_max, label="", batch=None):
        d, n, lv = self.draft(p, k_max, batch)
        assert B.pld_sync(self.ctx) == B.PLD_OK
        d, n, lv = d.cpu().numpy(), n.cpu().numpy(), lv.cpu().numpy()
        batch = self.batch if batch is None else batch
        od, on, olv = oracle.ngram_draft(p, self.host[:batch], k_max)
        bad = np.nonzero((n != on) | np.any(d != od, axis=1) | np.any(lv != olv, axis=1))[0]
        if bad.size:
            b = int(bad[0])
            raise AssertionError(
                f"{label}: {bad.size}/{batch} requests differ; b={b} L={len(self.host[b])} "
                f"gpu d={n[b]} {d[b].tolist()} levels {lv[b].tolist()}; oracle d={on[b]} "
                f"{od[b].tolist()} levels {olv[b].tolist()}")
        return od, on

    def reset(self):
        B.pld_store_reset(self.ctx)
        self.host = [np.zeros(0, np.int32) for _ in range(self.batch)]

    def close(self):
        B.pld_destroy(self.ctx)


WORKLOADS = {"c1": wl.config1, "c2": wl.config2, "c3": wl.config3, "c4": wl.config4}
PARAM_SETS = [P(), P(2, 3, (1, 2, 2, 1), (50, 66, 75, 50)), P(min_percent=(0, 0, 0, 0)),
              P(4, 4, (3, 3, 3, 3), (100, 100, 100, 100))]


@pytest.mark.parametrize("name", sorted(WORKLOADS))
def test_ngram_workloads(name):
    """Each lookup workload's histories appended whole (one append per
    request, through the multi-workgroup insert path), then drafted with the
    page's thresholds and three other parameter sets."""
    w = WORKLOADS[name]()
    max_len = max(len(h) for h in w.histories)
    s = NgramStore(len(w.histories), max_len)
    try:
        s.append(w.histories)
        for p in PARAM_SETS:
            s.check(p, w.k_max, f"{w.name} {p.n_min}..{p.n_max}")
        s.check(P(), 40, f"{w.name} k_max 40")
    finally:
        s.close()


def test_ngram_streaming_workload():
    """The streaming workload (64 requests from 32,768 tokens, 1,024 steps of
    1..16 appended tokens through the one-workgroup append): drafts checked
    against the oracle every 4th step and at the end. The appended tokens
    follow the workload's rule with the lookup oracle's drafts."""
    start = wl.config5_start()
    s = NgramStore(start.batch, wl.STREAM_MAX_LEN)
    try:
        s.append(start.histories)
        for step in range(wl.STREAM_STEPS):
            if step % 4 == 0:
                s.check(P(), start.k_max, f"step {step}")
            ld, ll, _, _ = oracle.draft(s.host, start.n_min, start.n_max, start.k_max)
            counts, fresh = wl.stream_step_draws(step)
            tok = wl.compose_append(ld, ll, counts, fresh)
            s.append([tok[b, :counts[b]] for b in range(start.batch)], width=tok.shape[1])
        s.check(P(), start.k_max, "final")
    finally:
        s.close()


@pytest.mark.parametrize("seed", range(8))
def test_ngram_fuzz_streams(seed):
    """Tiny alphabets (many equal n-grams and tied successors, so concurrent
    inserts of one n-gram are the rule), appends of 0..300 tokens, a large
    first append, random thresholds and lengths, k_max up to 70."""
    rng = np.random.default_rng([9201, seed])
    batch = int(rng.integers(1, 9))
    alpha = int(rng.integers(2, 5))
    cache_n = int(rng.integers(1, 5))
    s = NgramStore(batch, 6000, cache_n)
    try:
        s.append([rng.integers(-alpha // 2, alpha - alpha // 2,
                               int(rng.integers(0, 2000))).astype(np.int32)
                  for _ in range(batch)], width=2048)
        for step in range(25):
            p = pins.random_params(rng)
            n_min = min(p.n_min, cache_n)
            p = P(n_min, min(max(p.n_max, n_min), cache_n), tuple(p.min_count),
                  tuple(p.min_percent))
            s.check(p, int(rng.integers(1, 71)), f"seed {seed} step {step}")
            rows = []
            for b in range(batch):
                room = 6000 - len(s.host[b])
                c = min(room, int(rng.integers(0, 300)))
                if rng.random() < 0.3 and len(s.host[b]) > 8:
                    r = np.resize(s.host[b][-int(rng.integers(1, 8)):], c)
                else:
                    r = rng.integers(-alpha // 2, alpha - alpha // 2, c)
                rows.append(np.asarray(r, np.int32))
            s.append(rows)
        s.check(P(1, cache_n), 16, f"seed {seed} final")
    finally:
        s.close()


def test_ngram_golden_cases():
    """The hand-derived cases, each one request of its own context."""
    for case in pins.CASES:
        s = NgramStore(1, 64)
        try:
            if len(case["history"]):
                s.append([case["history"]])
            d, n, lv = s.draft(case["params"], case["k"])
            assert B.pld_sync(s.ctx) == B.PLD_OK
            assert d.cpu().numpy()[0].tolist() == case["draft"], case["name"]
            assert lv.cpu().numpy()[0].tolist() == case["levels"], case["name"]
        finally:
            s.close()


def test_ngram_extreme_tokens_and_ties():
    """Successor ties between the extreme int32 values, 0 and -1: the
    smaller token as a signed integer wins, in every length."""
    lo, hi = np.iinfo(np.int32).min, np.iinfo(np.int32).max
    rng = np.random.default_rng(9202)
    vals = np.array([lo, hi, 0, -1, 1, lo + 1, hi - 1], np.int32)
    rows = [vals[rng.integers(0, len(vals), int(rng.integers(1, 400)))] for _ in range(32)]
    s = NgramStore(32, 512)
    try:
        s.append(rows)
        for p in (P(), P(min_percent=(0, 0, 0, 0)), P(1, 1), P(3, 4)):
            s.check(p, 24, f"extremes {p.n_min}..{p.n_max}")
    finally:
        s.close()


def test_ngram_subset_batch_no_levels_and_reset():
    """Drafting the first rows only, without the levels output; then a
    reset empties the cache and the same histories give the same drafts."""
    import torch
    rng = np.random.default_rng(9203)
    rows = [rng.integers(0, 6, int(rng.integers(50, 900))).astype(np.int32) for _ in range(12)]
    s = NgramStore(12, 2000)
    try:
        s.append(rows)
        s.check(P(), 16, "all rows")
        s.check(P(), 16, "first five", batch=5)
        d, n, _ = s.draft(P(), 16, batch=5, levels=False)
        od, on, _ = oracle.ngram_draft(P(), s.host[:5], 16)
        assert (d.cpu().numpy() == od).all() and (n.cpu().numpy() == on).all()
        s.reset()
        d, n, lv = s.draft(P(), 16)
        assert B.pld_sync(s.ctx) == B.PLD_OK
        assert (n.cpu().numpy() == 0).all() and (d.cpu().numpy() == -1).all()
        assert (lv.cpu().numpy() == 0).all()
        s.append(rows)
        s.check(P(), 16, "after reset")
        torch.cuda.synchronize()
    finally:
        s.close()


def test_ngram_rejected_append_leaves_cache():
    """An append past max_len is rejected: the row and its counts stay as
    they were (the flag reports PLD_ECAPACITY), and drafts still match."""
    rng = np.random.default_rng(9204)
    rows = [rng.integers(0, 5, 90).astype(np.int32) for _ in range(4)]
    s = NgramStore(4, 100)
    try:
        s.append(rows)
        s.append([np.arange(20, dtype=np.int32)] + [np.zeros(0, np.int32)] * 3)
        assert B.pld_sync(s.ctx) == B.PLD_ECAPACITY
        assert len(s.host[0]) == 90
        s.check(P(), 16, "after rejected append")
    finally:
        s.close()


def test_ngram_rejects_lengths_beyond_cache():
    s = NgramStore(2, 100, n_max=2)
    try:
        with pytest.raises(B.PldError):
            s.draft(P(1, 3), 8)
        with pytest.raises(B.PldError):
            s.draft(P(min_percent=(50, 101, 50, 50)), 8)
    finally:
        s.close()


def test_ngram_append_longer_than_stride():
    """Source rows 8 tokens apart with counts up to 1,500 (rows overlap): the
    one-workgroup append reads such long appends from memory instead of its
    LDS window, and still counts exactly."""
    import torch
    rng = np.random.default_rng(9205)
    batch, stride = 6, 8
    counts = np.array([1500, 0, 1029, 1024, 7, 1100], np.int32)
    src = rng.integers(0, 4, (batch - 1) * stride + int(counts.max())).astype(np.int32)
    s = NgramStore(batch, 4000)
    try:
        s.append([rng.integers(0, 4, 30).astype(np.int32) for _ in range(batch)])
        for b in range(batch):
            s.host[b] = np.concatenate([s.host[b], src[b * stride:b * stride + counts[b]]])
        B.pld_append(s.ctx, torch.from_numpy(src).cuda(), stride, torch.from_numpy(counts).cuda(),
                     batch)
        s.check(P(), 32, "overlapping rows")
    finally:
        s.close()


def test_ngram_append_draft_streaming_workload():
    """The streaming workload through pld_append_draft_ngram (append and
    draft in one launch per step), checked every 4th step and at the end;
    the appended tokens follow the lookup oracle's drafts as above."""
    import torch
    start = wl.config5_start()
    s = NgramStore(start.batch, wl.STREAM_MAX_LEN)
    lib_p = to_lib(P())
    d = torch.empty((start.batch, start.k_max), dtype=torch.int32, device="cuda")
    n = torch.empty(start.batch, dtype=torch.int32, device="cuda")
    lv = torch.empty_like(d)
    try:
        s.append(start.histories)
        for step in range(wl.STREAM_STEPS):
            ld, ll, _, _ = oracle.draft(s.host, start.n_min, start.n_max, start.k_max)
            counts, fresh = wl.stream_step_draws(step)
            tok = wl.compose_append(ld, ll, counts, fresh)
            for b in range(start.batch):
                s.host[b] = np.concatenate([s.host[b], tok[b, :counts[b]]])
            B.pld_append_draft_ngram(s.ctx, torch.from_numpy(tok).cuda(), tok.shape[1],
                                     torch.from_numpy(counts).cuda(), start.batch, lib_p,
                                     start.k_max, d, n, lv)
            if step % 4 == 3 or step == wl.STREAM_STEPS - 1:
                assert B.pld_sync(s.ctx) == B.PLD_OK
                od, on, olv = oracle.ngram_draft(P(), s.host, start.k_max)
                assert (d.cpu().numpy() == od).all(), f"step {step}"
                assert (n.cpu().numpy() == on).all() and (lv.cpu().numpy() == olv).all()
    finally:
        s.close()


@pytest.mark.parametrize("seed", range(6))
def test_ngram_append_draft_fuzz(seed):
    """Random streams through pld_append_draft_ngram: tiny alphabets, counts
    of 0..40 (some rows past capacity, so rejected), source strides of 0
    (every row reads the same tokens), 40 (one launch) and 1,100 (append and
    draft as two calls), random thresholds; every step checked."""
    import torch
    rng = np.random.default_rng([9206, seed])
    batch = int(rng.integers(1, 9))
    alpha = int(rng.integers(2, 5))
    max_len = 600
    s = NgramStore(batch, max_len)
    try:
        s.append([rng.integers(0, alpha, int(rng.integers(0, 500))).astype(np.int32)
                  for _ in range(batch)])
        for step in range(30):
            stride = int(rng.choice([0, 40, 1100]))
            width = max(stride, 40)
            src = rng.integers(0, alpha, (batch, width)).astype(np.int32)
            if stride == 0:
                src[:] = src[0]
            counts = rng.integers(0, 41, batch).astype(np.int32)
            flat = src.reshape(-1) if stride else src[0]
            status_expect = B.PLD_OK
            for b in range(batch):
                row = flat[b * stride:b * stride + counts[b]] if stride else flat[:counts[b]]
                if len(s.host[b]) + counts[b] <= max_len:
                    s.host[b] = np.concatenate([s.host[b], row])
                else:
                    status_expect = B.PLD_ECAPACITY
            p = pins.random_params(rng)
            k = int(rng.integers(1, 40))
            d = torch.empty((batch, k), dtype=torch.int32, device="cuda")
            n = torch.empty(batch, dtype=torch.int32, device="cuda")
            lv = torch.empty_like(d)
            B.pld_append_draft_ngram(s.ctx, torch.from_numpy(np.ascontiguousarray(flat)).cuda(),
                                     stride, torch.from_numpy(counts).cuda(), batch, to_lib(p),
                                     k, d, n, lv)
            assert B.pld_sync(s.ctx) == status_expect, f"seed {seed} step {step}"
            od, on, olv = oracle.ngram_draft(p, s.host, k)
            assert (d.cpu().numpy() == od).all(), f"seed {seed} step {step} stride {stride}"
            assert (n.cpu().numpy() == on).all() and (lv.cpu().numpy() == olv).all()
    finally:
        s.close()


def test_ngram_append_draft_long_rows():
    """Counts above the one-launch window (rows 8 tokens apart, up to 1,500
    tokens): the fused kernel reads such appends from memory."""
    import torch
    rng = np.random.default_rng(9207)
    batch, stride = 5, 8
    counts = np.array([1500, 3, 1030, 0, 1200], np.int32)
    src = rng.integers(0, 3, (batch - 1) * stride + int(counts.max())).astype(np.int32)
    s = NgramStore(batch, 4000)
    try:
        s.append([rng.integers(0, 3, 50).astype(np.int32) for _ in range(batch)])
        for b in range(batch):
            s.host[b] = np.concatenate([s.host[b], src[b * stride:b * stride + counts[b]]])
        d = torch.empty((batch, 24), dtype=torch.int32, device="cuda")
        n = torch.empty(batch, dtype=torch.int32, device="cuda")
        lv = torch.empty_like(d)
        B.pld_append_draft_ngram(s.ctx, torch.from_numpy(src).cuda(), stride,
                                 torch.from_numpy(counts).cuda(), batch, to_lib(P()), 24, d, n,
                                 lv)
        assert B.pld_sync(s.ctx) == B.PLD_OK
        od, on, olv = oracle.ngram_draft(P(), s.host, 24)
        assert (d.cpu().numpy() == od).all() and (lv.cpu().numpy() == olv).all()
    finally:
        s.close()
