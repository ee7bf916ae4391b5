"""GPU parity of one decode step in one launch on a context with a plain
store: pld_append_draft_store appends each request's new tokens and drafts
the new histories by scanning them, in the scan kernel's own launch (the
appended positions are read from the caller's source row; the request's
last tile copies them into the store; the workgroup that emits the draft
stores the new length).

Every draft is compared, element by element, with the CPU oracle run on a
host mirror of the histories, and the store's rows, lengths and the sticky
error status are compared with what pld_append followed by pld_draft_batch
would leave. Inputs are seeded and synthetic."""

from __future__ import annotations

import ctypes

import numpy as np
import pytest

import oracle
from prompt_lookup_gram_amd import binding as B
from prompt_lookup_gram_amd import workloads as wl

pytestmark = pytest.mark.gpu

TILES = (256, 1024, 2048, 4096, 8192, 16384)


@pytest.fixture(scope="module", autouse=True)
def gpu():
    import torch
    assert torch.cuda.is_available(), "GPU tests need a GPU"
    B.load()
    torch.cuda.init()
    yield
    torch.cuda.synchronize()


def _hip():
    hip = ctypes.CDLL("libamdhip64.so")
    hip.hipMemcpy.argtypes = [ctypes.c_void_p, ctypes.c_void_p, ctypes.c_size_t, ctypes.c_int]
    return hip


def to_host(dst: np.ndarray, src_ptr: int) -> np.ndarray:
    assert _hip().hipMemcpy(dst.ctypes.data, src_ptr, dst.nbytes, 2) == 0  # device->host
    return dst


def to_device(dst_ptr: int, src: np.ndarray) -> None:
    src = np.ascontiguousarray(src)
    assert _hip().hipMemcpy(dst_ptr, src.ctypes.data, src.nbytes, 1) == 0  # host->device


class Mirror:
    """The histories as the store should hold them, kept on the host with
    pld_append's rules: an append is taken whole or (negative count, or past
    max_len) rejected and flagged."""

    def __init__(self, max_batch: int, max_len: int):
        self.max_len = max_len
        self.rows = [np.zeros(0, np.int32) for _ in range(max_batch)]

    def append(self, tok: np.ndarray, counts: np.ndarray, batch: int) -> int:
        """Applies one call's appends; returns the status pld_sync reports."""
        cap = neg = False
        for b in range(batch):
            c = int(counts[b])
            if c < 0:
                neg = True
            elif len(self.rows[b]) + c > self.max_len:
                cap = True
            else:
                self.rows[b] = np.concatenate([self.rows[b], tok[b, :c]]).astype(np.int32)
        return B.PLD_ECAPACITY if cap else (B.PLD_EINVAL if neg else B.PLD_OK)


def store_state(ctx, max_batch: int):
    rows, lens = B.pld_histories(ctx)
    table = to_host(np.zeros(max_batch, np.int64), rows)
    got_len = to_host(np.zeros(max_batch, np.int32), lens)
    got = [to_host(np.zeros(max(int(n), 0), np.int32), int(table[b])) if n > 0
           else np.zeros(0, np.int32) for b, n in enumerate(got_len)]
    return got_len, got


def check_outputs(mirror: Mirror, batch, n_min, n_max, k_max, out, label):
    d, l, m, p = [t.cpu().numpy() for t in out]
    od, ol, om, oj = oracle.draft(mirror.rows[:batch], n_min, n_max, k_max)
    bad = np.nonzero((m[:batch] != om) | (p[:batch] != oj) | (l[:batch] != ol)
                     | np.any(d[:batch] != od, axis=1))[0]
    if bad.size:
        b = int(bad[0])
        raise AssertionError(
            f"{label}: {bad.size}/{batch} requests differ; first b={b} "
            f"L={len(mirror.rows[b])} gpu=(m={m[b]}, j={p[b]}, d={l[b]}, row={d[b].tolist()}) "
            f"oracle=(m={om[b]}, j={oj[b]}, d={ol[b]}, row={od[b].tolist()})")


def check_store(ctx, mirror: Mirror, max_batch: int, label: str):
    got_len, got = store_state(ctx, max_batch)
    for b in range(max_batch):
        assert got_len[b] == len(mirror.rows[b]), f"{label}: length of row {b}"
        assert np.array_equal(got[b], mirror.rows[b]), f"{label}: tokens of row {b}"


# ---------------------------------------------------------------------------
# the streaming workload at every tile size
# ---------------------------------------------------------------------------


@pytest.mark.parametrize("tile", TILES)
def test_streaming_one_launch_every_tile(tile):
    """64 requests from 32,768 tokens; each call appends 1..16 tokens (the
    previous draft's tokens while they last, then fresh Zipf tokens) and
    drafts. Tiles of 256 tokens give 192 workgroups per request, most of
    them past the histories' last tile early on."""
    import torch
    start = wl.config5_start()
    nb, steps = start.batch, 160
    ctx = B.pld_create(nb, wl.STREAM_MAX_LEN, own_store=True)
    try:
        B.pld_configure(ctx, tile, 1)
        mirror = Mirror(nb, wl.STREAM_MAX_LEN)
        init = np.stack(start.histories).astype(np.int32)
        mirror.append(init, np.full(nb, wl.STREAM_START_LEN), nb)
        B.pld_append(ctx, torch.from_numpy(init).cuda(), wl.STREAM_START_LEN,
                     torch.full((nb,), wl.STREAM_START_LEN, dtype=torch.int32,
                                device="cuda"), nb)
        out = B.alloc_outputs(nb, start.k_max)
        B.pld_draft_batch_pos(ctx, *B.pld_histories(ctx), nb, start.n_min, start.n_max,
                              start.k_max, *out)
        for step in range(steps):
            d, l = out[0].cpu().numpy(), out[1].cpu().numpy()
            counts, fresh = wl.stream_step_draws(step)
            tok = wl.compose_append(d, l, counts, fresh)
            mirror.append(tok, counts, nb)
            for t in out:
                t.fill_(-7)   # poison: every slot must be written
            B.pld_append_draft_store(ctx, torch.from_numpy(tok).cuda(), tok.shape[1],
                                     torch.from_numpy(counts).cuda(), nb, start.n_min,
                                     start.n_max, start.k_max, *out)
            check_outputs(mirror, nb, start.n_min, start.n_max, start.k_max, out,
                          f"tile {tile} step {step}")
        assert B.pld_sync(ctx) == B.PLD_OK
        check_store(ctx, mirror, nb, f"tile {tile}")
    finally:
        B.pld_destroy(ctx)


# ---------------------------------------------------------------------------
# fuzz: ragged rows, idle tiles, rejected appends, subset batches
# ---------------------------------------------------------------------------


def fuzz_tokens(rng, rows, width):
    """Appends that often repeat what the row already holds (copied spans,
    periodic runs) over a small alphabet, so long and overlapping matches
    are common."""
    alphabet = int(rng.choice([2, 3, 7, 50]))
    tok = rng.integers(-alphabet // 2, alphabet - alphabet // 2, (rows, width)).astype(np.int32)
    return tok


@pytest.mark.parametrize("seed", range(24))
def test_fuzz_against_oracle(seed):
    import torch
    rng = np.random.default_rng([7301, seed])
    max_batch = int(rng.integers(1, 10))
    max_len = int(rng.choice([1, 5, 70, 300, 1500, 5000]))
    tile = int(rng.choice(TILES))
    n_min = int(rng.integers(1, 6))
    n_max = int(rng.integers(n_min, min(64, n_min + 14) + 1))
    k_max = int(rng.integers(1, 41))
    width = int(rng.choice([1, 4, 16, 100, 1024]))
    ctx = B.pld_create(max_batch, max_len, own_store=True)
    try:
        B.pld_configure(ctx, tile, 1)
        mirror = Mirror(max_batch, max_len)
        for step in range(30):
            batch = int(rng.integers(0, max_batch + 1))
            tok = fuzz_tokens(rng, max(batch, 1), width)
            for b in range(batch):   # repeat an earlier span of the row now and then
                h = mirror.rows[b]
                if h.size > 8 and rng.random() < 0.5:
                    s = int(rng.integers(0, h.size - 4))
                    span = h[s:s + width]
                    tok[b, :span.size] = span
            counts = rng.integers(0, width + 1, max(batch, 1)).astype(np.int32)
            if rng.random() < 0.15 and batch:
                counts[int(rng.integers(0, batch))] = -int(rng.integers(1, 5))
            if rng.random() < 0.15 and batch:   # one row asks for more than is left
                b = int(rng.integers(0, batch))
                counts[b] = min(width, max_len - len(mirror.rows[b]) + 1)
            want = mirror.append(tok, counts, batch)
            out = B.alloc_outputs(max(batch, 1), k_max)
            for t in out:
                t.fill_(-7)
            pos = out[3] if rng.random() < 0.7 else None
            B.pld_append_draft_store(ctx, torch.from_numpy(tok).cuda(), width,
                                     torch.from_numpy(counts).cuda(), batch, n_min, n_max,
                                     k_max, out[0], out[1], out[2], pos)
            st = B.pld_sync(ctx)
            label = (f"seed {seed} step {step} (batch {batch}/{max_batch}, max_len {max_len}, "
                     f"tile {tile}, n {n_min}..{n_max}, k {k_max}, width {width})")
            assert st == want, f"{label}: status {st}, want {want}"
            if batch and pos is None:
                d, l, m = [t.cpu().numpy() for t in out[:3]]
                od, ol, om, _ = oracle.draft(mirror.rows[:batch], n_min, n_max, k_max)
                assert np.array_equal(d, od) and np.array_equal(l, ol) \
                    and np.array_equal(m, om), label
            elif batch:
                check_outputs(mirror, batch, n_min, n_max, k_max, out, label)
        check_store(ctx, mirror, max_batch, f"seed {seed} final")
    finally:
        B.pld_destroy(ctx)


@pytest.mark.parametrize("seed", range(6))
def test_same_as_append_then_draft(seed):
    """The one-launch step and the two-call step (pld_append, then the scan
    over pld_histories) leave the same outputs, store and status; the
    second context drafts with the separate gather kernel, which never
    takes the one-launch path."""
    import torch
    rng = np.random.default_rng([7302, seed])
    nb, max_len, width = 12, 3000, 16
    ctxs = [B.pld_create(nb, max_len, own_store=True) for _ in range(2)]
    try:
        B.pld_configure(ctxs[0], int(rng.choice(TILES)), 1)
        B.pld_configure(ctxs[1], int(rng.choice(TILES)), 0)
        for step in range(40):
            tok = torch.from_numpy(fuzz_tokens(rng, nb, width)).cuda()
            counts = rng.integers(0, width + 1, nb).astype(np.int32)
            if step % 7 == 3:
                counts[step % nb] = -1
            cnt = torch.from_numpy(counts).cuda()
            res = []
            for ctx in ctxs:
                out = B.alloc_outputs(nb, 16)
                for t in out:
                    t.fill_(-7)
                B.pld_append_draft_store(ctx, tok, width, cnt, nb, 4, 12, 16, *out)
                res.append((B.pld_sync(ctx), [t.cpu().numpy() for t in out],
                            store_state(ctx, nb)))
            (s0, o0, (l0, r0)), (s1, o1, (l1, r1)) = res
            assert s0 == s1, f"step {step}"
            assert all(np.array_equal(a, b) for a, b in zip(o0, o1)), f"step {step}"
            assert np.array_equal(l0, l1) and all(np.array_equal(a, b) for a, b in zip(r0, r1))
    finally:
        for ctx in ctxs:
            B.pld_destroy(ctx)


# ---------------------------------------------------------------------------
# errors
# ---------------------------------------------------------------------------


@pytest.mark.parametrize("one_launch", [True, False])
def test_corrupt_lengths_are_rejected(one_launch):
    """Lengths outside [0, max_len] written into the store's length array
    (the caller can reach it through pld_histories) reject that row's
    append, flag the context and give a no-match row; nothing outside the
    rows' tokens is written and the other rows go on as usual."""
    import torch
    nb, max_len = 4, 40
    ctx = B.pld_create(nb, max_len, own_store=True)
    try:
        B.pld_configure(ctx, 256, 1 if one_launch else 0)
        mirror = Mirror(nb, max_len)
        base = (np.arange(nb * 16, dtype=np.int32).reshape(nb, 16) % 5)
        mirror.append(base, np.full(nb, 16), nb)
        B.pld_append(ctx, torch.from_numpy(base).cuda(), 16,
                     torch.full((nb,), 16, dtype=torch.int32, device="cuda"), nb)
        assert B.pld_sync(ctx) == B.PLD_OK
        rows, lens = B.pld_histories(ctx)
        table = to_host(np.zeros(nb, np.int64), rows)
        pitch = int(table[1] - table[0]) // 4
        before = to_host(np.zeros(nb * pitch, np.int32), int(table[0]))
        bad = np.array([16, -5, max_len + 3, 16], np.int32)
        to_device(lens, bad)
        tok = torch.from_numpy(np.full((nb, 4), 3, np.int32)).cuda()
        out = B.alloc_outputs(nb, 8)
        B.pld_append_draft_store(ctx, tok, 4, torch.full((nb,), 2, dtype=torch.int32,
                                                          device="cuda"), nb, 3, 8, 8, *out)
        assert B.pld_sync(ctx) == B.PLD_ECAPACITY
        d, l, m, p = [t.cpu().numpy() for t in out]
        for b in (1, 2):
            assert l[b] == 0 and m[b] == 0 and p[b] == -1 and np.all(d[b] == -1)
        after = to_host(np.zeros(nb * pitch, np.int32), int(table[0]))
        for b in (0, 3):
            mirror.rows[b] = np.concatenate([mirror.rows[b], np.full(2, 3, np.int32)])
            before[b * pitch + 16:b * pitch + 18] = 3
        assert np.array_equal(after, before)   # rows 1 and 2 untouched, nothing else written
        got_len = to_host(np.zeros(nb, np.int32), lens)
        assert got_len.tolist() == [18, -5, max_len + 3, 18]
        od, ol, om, oj = oracle.draft([mirror.rows[0], mirror.rows[3]], 3, 8, 8)
        assert np.array_equal(d[[0, 3]], od) and np.array_equal(l[[0, 3]], ol)
        assert np.array_equal(m[[0, 3]], om) and np.array_equal(p[[0, 3]], oj)
        B.pld_store_reset(ctx)
        assert B.pld_sync(ctx) == B.PLD_OK
    finally:
        B.pld_destroy(ctx)


def test_host_validation_enqueues_nothing():
    import torch
    ctx = B.pld_create(2, 50, own_store=True)
    try:
        tok = torch.zeros((2, 8), dtype=torch.int32, device="cuda")
        cnt = torch.full((2,), 8, dtype=torch.int32, device="cuda")
        out = B.alloc_outputs(2, 8)
        for args in [(0, 8, 8), (3, 2, 8), (3, 65, 8), (3, 8, 0)]:
            with pytest.raises(B.PldError):
                B.pld_append_draft_store(ctx, tok, 8, cnt, 2, *args, *out)
        with pytest.raises(B.PldError):
            B.pld_append_draft_store(ctx, tok, 8, cnt, 3, 3, 8, 8, *out)
        assert B.pld_sync(ctx) == B.PLD_OK
        got_len, _ = store_state(ctx, 2)
        assert got_len.tolist() == [0, 0]
    finally:
        B.pld_destroy(ctx)


def test_more_tiles_than_grid_rows():
    """A capacity of 17,000,000 tokens at 256-token tiles needs 66,407 tiles
    per request, more than one grid dimension holds: the tiles continue in a
    third dimension. Short histories at the start of such rows, drafted by
    the one-launch step and by the plain scan, match the oracle."""
    import torch
    nb, max_len = 2, 17_000_000
    ctx = B.pld_create(nb, max_len, own_store=True)
    try:
        B.pld_configure(ctx, 256, 1)
        mirror = Mirror(nb, max_len)
        rng = np.random.default_rng(7303)
        out = B.alloc_outputs(nb, 16)
        for step in range(4):
            tok = rng.integers(0, 5, (nb, 600)).astype(np.int32)
            counts = np.array([600, 317], np.int32)
            mirror.append(tok, counts, nb)
            for t in out:
                t.fill_(-7)
            B.pld_append_draft_store(ctx, torch.from_numpy(tok).cuda(), 600,
                                     torch.from_numpy(counts).cuda(), nb, 4, 12, 16, *out)
            check_outputs(mirror, nb, 4, 12, 16, out, f"step {step}")
        for t in out:
            t.fill_(-7)
        B.pld_draft_batch_pos(ctx, *B.pld_histories(ctx), nb, 4, 12, 16, *out)
        check_outputs(mirror, nb, 4, 12, 16, out, "plain scan")
        assert B.pld_sync(ctx) == B.PLD_OK
        check_store(ctx, mirror, nb, "store")
    finally:
        B.pld_destroy(ctx)
