"""GPU parity of the incremental n-gram index (pld_create_indexed,
pld_append, pld_draft_store) against the CPU oracle: the index must give
exactly the scan's results (draft rows with padding, draft lengths, match
lengths, occurrence starts) after every append.

Inputs are seeded and synthetic (prompt_lookup_gram_amd.workloads)."""

from __future__ import annotations

import numpy as np
import pytest

import oracle
from prompt_lookup_gram_amd import binding as B
from prompt_lookup_gram_amd import workloads as wl

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def gpu():
    import torch
    assert torch.cuda.is_available(), "GPU tests need a GPU"
    B.load()
    torch.cuda.init()
    yield
    torch.cuda.synchronize()


class IndexedStore:
    """An indexed context plus a host mirror of its histories."""

    def __init__(self, batch, max_len, n_lo, n_hi):
        self.batch, self.max_len = batch, max_len
        self.ctx = B.pld_create_indexed(batch, max_len, n_lo, n_hi)
        self.host = [np.zeros(0, np.int32) for _ in range(batch)]

    def append(self, rows):
        """rows: list of per-request int32 arrays (may be empty)."""
        import torch
        width = max(1, max(len(r) for r in rows))
        tok = np.zeros((self.batch, width), np.int32)
        cnt = np.zeros(self.batch, np.int32)
        for b, r in enumerate(rows):
            tok[b, :len(r)] = r
            cnt[b] = len(r)
            self.host[b] = np.concatenate([self.host[b], np.asarray(r, np.int32)])
        B.pld_append(self.ctx, torch.from_numpy(tok).cuda(), width,
                     torch.from_numpy(cnt).cuda(), self.batch)

    def check(self, n_min, n_max, k_max, label=""):
        out = B.alloc_outputs(self.batch, k_max)
        for t in out:
            t.fill_(-7)
        B.pld_draft_store(self.ctx, self.batch, n_min, n_max, k_max, *out)
        assert B.pld_sync(self.ctx) == B.PLD_OK
        d, l, m, p = [t.cpu().numpy() for t in out]
        od, ol, om, oj = oracle.draft(self.host, n_min, n_max, k_max)
        bad = np.nonzero((m != om) | (p != oj) | (l != ol) | np.any(d != od, axis=1))[0]
        if bad.size:
            b = int(bad[0])
            raise AssertionError(
                f"{label}: {bad.size}/{self.batch} requests differ; b={b} L={len(self.host[b])} "
                f"index=(m={m[b]}, j={p[b]}, d={l[b]}) oracle=(m={om[b]}, j={oj[b]}, d={ol[b]})")
        return d, l, m, p

    def reset(self):
        B.pld_store_reset(self.ctx)
        self.host = [np.zeros(0, np.int32) for _ in range(self.batch)]

    def close(self):
        B.pld_destroy(self.ctx)


def test_index_streaming_all_steps():
    """The streaming workload (64 requests from 32,768 tokens, 1,024 steps of
    1..16 appended tokens) drafted from the index, in lockstep with the
    oracle at every step."""
    start = wl.config5_start()
    s = IndexedStore(start.batch, wl.STREAM_MAX_LEN, start.n_min, start.n_max)
    try:
        s.append(start.histories)
        for step in range(wl.STREAM_STEPS):
            d, l, m, p = s.check(start.n_min, start.n_max, start.k_max, f"step {step}")
            counts, fresh = wl.stream_step_draws(step)
            tok = wl.compose_append(d, l, counts, fresh)
            s.append([tok[b, :counts[b]] for b in range(start.batch)])
        s.check(start.n_min, start.n_max, start.k_max, "final")
    finally:
        s.close()


@pytest.mark.parametrize("seed", range(6))
def test_index_fuzz_streams(seed):
    """Tiny alphabets (many repeated and overlapping n-grams, so concurrent
    inserts of one n-gram are common), appends of 0..300 tokens, a large first
    append, query ranges inside the indexed one."""
    rng = np.random.default_rng([9001, seed])
    batch = int(rng.integers(1, 9))
    alpha = int(rng.integers(2, 5))
    n_lo = int(rng.integers(1, 6))
    n_hi = int(rng.integers(n_lo, 17))
    s = IndexedStore(batch, 6000, n_lo, n_hi)
    try:
        s.append([rng.integers(0, alpha, int(rng.integers(0, 2000))).astype(np.int32)
                  for _ in range(batch)])
        for step in range(25):
            n_min = int(rng.integers(n_lo, n_hi + 1))
            n_max = int(rng.integers(n_min, n_hi + 1))
            k_max = int(rng.integers(1, 40))
            s.check(n_min, n_max, k_max, f"seed {seed} step {step}")
            rows = []
            for b in range(batch):
                room = 6000 - len(s.host[b])
                c = min(room, int(rng.integers(0, 300)))
                if rng.random() < 0.3 and len(s.host[b]) > 8:
                    # repeat a recent span: long matches, periodic overlaps
                    src = s.host[b][-int(rng.integers(1, 8)):]
                    r = np.resize(src, c)
                else:
                    r = rng.integers(0, alpha, c)
                rows.append(r.astype(np.int32))
            s.append(rows)
        s.check(n_lo, n_hi, 16, f"seed {seed} final")
    finally:
        s.close()


def test_index_every_length():
    """Lengths 1..64 all indexed; periodic runs of many periods."""
    rng = np.random.default_rng(9002)
    s = IndexedStore(6, 3000, 1, 64)
    try:
        rows = []
        for b in range(6):
            blk = rng.permutation(40)[:b + 1].astype(np.int32)
            rows.append(np.concatenate([rng.integers(50, 90, 500), np.resize(blk, 400)]).astype(
                np.int32))
        s.append(rows)
        for n_min, n_max in [(1, 64), (1, 1), (64, 64), (3, 40), (17, 33)]:
            s.check(n_min, n_max, 70, f"n {n_min}..{n_max}")
        for _ in range(5):
            s.append([rng.integers(0, 3, 37).astype(np.int32) for _ in range(6)])
            s.check(1, 64, 20, "after appends")
    finally:
        s.close()


def test_index_one_periodic_append():
    """A whole periodic history in one append: every thread inserts the same
    few n-grams at once; the largest end must win."""
    s = IndexedStore(3, 20000, 4, 12)
    try:
        s.append([np.resize(np.array([7, 8, 9], np.int32), 20000 - 5),
                  np.resize(np.array([1], np.int32), 12000),
                  np.resize(np.arange(11, dtype=np.int32), 15001)])
        s.check(4, 12, 16, "periodic")
        s.check(5, 5, 3, "periodic, one length")
    finally:
        s.close()


def test_index_reset_and_reuse():
    """After pld_store_reset nothing of the old histories is left in the
    index: new histories that reuse the old n-grams draft exactly."""
    rng = np.random.default_rng(9003)
    s = IndexedStore(4, 4000, 2, 10)
    try:
        old = [rng.integers(0, 4, 3000).astype(np.int32) for _ in range(4)]
        s.append(old)
        s.check(2, 10, 8, "before reset")
        s.reset()
        s.check(2, 10, 8, "empty after reset")
        s.append([o[:50] for o in old])    # a prefix: old later positions must not appear
        s.check(2, 10, 8, "after reset")
        s.append([rng.integers(0, 4, 400).astype(np.int32) for _ in range(4)])
        s.check(2, 10, 8, "after reset, more")
    finally:
        s.close()


def test_index_overflow_and_errors():
    import torch
    s = IndexedStore(2, 100, 3, 8)
    try:
        s.append([np.arange(60, dtype=np.int32) % 7, np.arange(90, dtype=np.int32) % 5])
        s.check(3, 8, 8, "filled")
        # request 1 would pass max_len: rejected whole, nothing indexed
        tok = torch.zeros((2, 20), dtype=torch.int32, device="cuda")
        B.pld_append(s.ctx, tok, 20, torch.tensor([5, 20], dtype=torch.int32, device="cuda"), 2)
        assert B.pld_sync(s.ctx) == B.PLD_ECAPACITY
        s.host[0] = np.concatenate([s.host[0], np.zeros(5, np.int32)])
        s.check(3, 8, 8, "after a rejected append")
        out = B.alloc_outputs(2, 8)
        for lo, hi in [(2, 8), (3, 9), (5, 4)]:
            with pytest.raises(B.PldError) as e:
                B.pld_draft_store(s.ctx, 2, lo, hi, 8, *out)
            assert e.value.status == B.PLD_EINVAL
        with pytest.raises(B.PldError):
            B.pld_draft_store(s.ctx, 3, 3, 8, 8, *out)     # batch above max_batch
        B.pld_draft_store(s.ctx, 0, 3, 8, 8, *out)          # batch 0: no-op
        assert B.pld_sync(s.ctx) == B.PLD_OK
    finally:
        s.close()
    plain = B.pld_create(2, 100, own_store=True)
    try:
        with pytest.raises(B.PldError) as e:
            B.pld_draft_store(plain, 2, 3, 8, 8, *B.alloc_outputs(2, 8))
        assert "index" in str(e.value)
    finally:
        B.pld_destroy(plain)


def test_index_agrees_with_scan_on_store():
    """pld_draft_store and pld_draft_batch_pos over pld_histories give the
    same bits on one indexed store (both are checked against the oracle
    elsewhere; this pins the two GPU paths to each other directly)."""
    w = wl.config3()
    s = IndexedStore(w.batch, int(w.lengths.max()), 4, 12)
    try:
        s.append(w.histories)
        a = s.check(4, 12, 16, "config 3")
        rows, lens = B.pld_histories(s.ctx)
        out = B.alloc_outputs(w.batch, 16)
        B.pld_draft_batch_pos(s.ctx, rows, lens, w.batch, 4, 12, 16, *out)
        assert B.pld_sync(s.ctx) == B.PLD_OK
        for x, y in zip(a, [t.cpu().numpy() for t in out]):
            assert np.array_equal(x, y)
    finally:
        s.close()


@pytest.mark.parametrize("bits", [0, 3, 12])
def test_index_fingerprint_collisions(bits):
    """With few fingerprint bits, n-grams share slots all the time and most
    queries land on a slot that does not confirm: those requests are answered
    by the exact scan, and every result still equals the oracle's."""
    rng = np.random.default_rng([9004, bits])
    s = IndexedStore(5, 3000, 3, 9)
    try:
        B.pld_index_fingerprint_bits(s.ctx, bits)
        s.append([rng.integers(0, 6, int(rng.integers(50, 1500))).astype(np.int32)
                  for _ in range(5)])
        for step in range(12):
            s.check(3, 9, 12, f"bits {bits} step {step}")
            rows = []
            for b in range(5):
                c = min(3000 - len(s.host[b]), int(rng.integers(0, 60)))
                if rng.random() < 0.4 and len(s.host[b]) > 20:
                    start = int(rng.integers(0, len(s.host[b]) - 20))
                    r = s.host[b][start:start + c]
                else:
                    r = rng.integers(0, 6, c)
                rows.append(np.asarray(r, np.int32))
            s.append(rows)
        s.check(4, 6, 5, f"bits {bits} final")
    finally:
        s.close()
    with pytest.raises(B.PldError):
        plain = B.pld_create(1, 10, own_store=True)
        try:
            B.pld_index_fingerprint_bits(plain, 8)
        finally:
            B.pld_destroy(plain)


# ---------------------------------------------------------------------------
# pld_append_draft_store: one decode step (append, then draft) per call
# ---------------------------------------------------------------------------


def _stream_with_append_draft(ctx, steps, fp_bits=None):
    """The streaming workload driven by pld_append_draft_store: each call
    appends a step's tokens and drafts the new histories; every draft is
    compared with the oracle on the mirrored histories."""
    import torch
    start = wl.config5_start()
    nb = start.batch
    if fp_bits is not None:
        B.pld_index_fingerprint_bits(ctx, fp_bits)
    host = [h.copy() for h in start.histories]
    out = B.alloc_outputs(nb, start.k_max)
    init = torch.from_numpy(np.stack(start.histories)).cuda()
    counts0 = torch.full((nb,), wl.STREAM_START_LEN, dtype=torch.int32, device="cuda")
    B.pld_append_draft_store(ctx, init, wl.STREAM_START_LEN, counts0, nb, start.n_min,
                             start.n_max, start.k_max, *out)
    for step in range(steps):
        d, l, m, p = [t.cpu().numpy() for t in out]
        od, ol, om, oj = oracle.draft(host, start.n_min, start.n_max, start.k_max)
        bad = np.nonzero((m != om) | (p != oj) | (l != ol) | np.any(d != od, axis=1))[0]
        assert bad.size == 0, f"step {step}: request {bad[:1]} differs"
        counts, fresh = wl.stream_step_draws(step)
        tok = wl.compose_append(d, l, counts, fresh)
        host = [np.concatenate([h, tok[b, :counts[b]]]) for b, h in enumerate(host)]
        for t in out:
            t.fill_(-7)
        B.pld_append_draft_store(ctx, torch.from_numpy(tok).cuda(), tok.shape[1],
                                 torch.from_numpy(counts).cuda(), nb, start.n_min, start.n_max,
                                 start.k_max, *out)
    assert B.pld_sync(ctx) == B.PLD_OK


@pytest.mark.parametrize("mode", ["indexed", "indexed_collisions", "scan"])
def test_append_draft_streaming(mode):
    start = wl.config5_start()
    if mode == "scan":
        ctx = B.pld_create(start.batch, wl.STREAM_MAX_LEN, own_store=True)
    else:
        ctx = B.pld_create_indexed(start.batch, wl.STREAM_MAX_LEN, start.n_min, start.n_max)
    try:
        steps = 300 if mode == "indexed_collisions" else wl.STREAM_STEPS
        _stream_with_append_draft(ctx, steps, fp_bits=6 if mode == "indexed_collisions" else None)
    finally:
        B.pld_destroy(ctx)


def test_append_draft_rejected_and_errors():
    """A rejected append drafts its row as it stands; argument errors are
    caught before anything is enqueued (the store is unchanged)."""
    import torch
    s = IndexedStore(2, 50, 3, 8)
    try:
        s.append([np.arange(40, dtype=np.int32) % 6, np.arange(45, dtype=np.int32) % 4])
        out = B.alloc_outputs(2, 8)
        tok = torch.tensor([[1, 2, 3, 4, 5, 0, 0, 0], [1, 2, 3, 0, 1, 2, 3, 0]],
                           dtype=torch.int32, device="cuda")
        B.pld_append_draft_store(s.ctx, tok, 8, torch.tensor([5, 8], dtype=torch.int32,
                                                             device="cuda"), 2, 3, 8, 8, *out)
        assert B.pld_sync(s.ctx) == B.PLD_ECAPACITY   # request 1 would pass max_len
        s.host[0] = np.concatenate([s.host[0], np.arange(1, 6, dtype=np.int32)])
        d, l, m, p = [t.cpu().numpy() for t in out]
        od, ol, om, oj = oracle.draft(s.host, 3, 8, 8)
        assert np.array_equal(d, od) and np.array_equal(l, ol) and np.array_equal(m, om)
        assert np.array_equal(p, oj)
        cnt = torch.tensor([1, 1], dtype=torch.int32, device="cuda")
        for args in [(2, 9, 8), (3, 2, 8), (3, 8, 0)]:
            with pytest.raises(B.PldError):
                B.pld_append_draft_store(s.ctx, tok, 8, cnt, 2, *args, *out)
        s.check(3, 8, 8, "store unchanged by rejected calls")
    finally:
        s.close()
