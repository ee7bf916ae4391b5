"""GPU parity: pld_draft_batch (HIP, gfx950) against the CPU oracle, element
by element (draft rows including the -1 padding, draft lengths, match
lengths, occurrence starts). Everything is integer, so the bar is bit-exact.

All inputs are seeded and synthetic (prompt_lookup_gram_amd.workloads)."""

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


def run_gpu(w, tile=0, fused=-1, offsets=None, max_len=None, max_batch=None):
    db = B.DeviceBatch(w.histories, offsets=offsets)
    ctx = B.pld_create(max_batch or max(1, w.batch), max_len or db.max_len)
    try:
        B.pld_configure(ctx, tile, fused)
        out = B.alloc_outputs(w.batch, w.k_max)
        for t in out:
            t.fill_(-7)  # poison: every slot must be written
        B.pld_draft_batch_pos(ctx, db.rows, db.lengths, w.batch, w.n_min, w.n_max,
                              w.k_max, *out)
        st = B.pld_sync(ctx)
    finally:
        B.pld_destroy(ctx)
    return st, [t.cpu().numpy() for t in out]


def assert_parity(w, got, label=""):
    od, ol, om, oj = oracle.draft(w.histories, w.n_min, w.n_max, w.k_max)
    d, l, m, p = got
    bad = np.nonzero((m != om) | (p != oj) | (l != ol) | np.any(d != od, axis=1))[0]
    if bad.size:
        b = int(bad[0])
        raise AssertionError(
            f"{w.name} {label}: {bad.size}/{w.batch} requests differ; first b={b} "
            f"L={len(w.histories[b])} gpu=(m={m[b]}, j={p[b]}, d={l[b]}, "
            f"row={d[b].tolist()}) oracle=(m={om[b]}, j={oj[b]}, d={ol[b]}, "
            f"row={od[b].tolist()})")


# ---------------------------------------------------------------------------
# the four batch workloads at full size, default launch configuration
# ---------------------------------------------------------------------------


@pytest.mark.parametrize("cfg", [1, 2, 3, 4])
def test_config_parity(cfg):
    w = wl.ALL_CONFIGS[cfg]()
    st, got = run_gpu(w)
    assert st == B.PLD_OK
    assert_parity(w, got, "default")


@pytest.mark.parametrize("cfg", [2, 3, 4])
@pytest.mark.parametrize("tile", TILES)
@pytest.mark.parametrize("fused", [1, 0])
def test_config_parity_every_tiling(cfg, tile, fused):
    """Split invariance: any tile size, fused or separate gather."""
    w = wl.ALL_CONFIGS[cfg]()
    st, got = run_gpu(w, tile=tile, fused=fused)
    assert st == B.PLD_OK
    assert_parity(w, got, f"tile={tile} fused={fused}")


# ---------------------------------------------------------------------------
# fuzz: tiny alphabets, ragged lengths, random parameters, every alignment
# ---------------------------------------------------------------------------


@pytest.mark.parametrize("seed", range(40))
def test_fuzz(seed):
    w = wl.fuzz_batch(seed)
    rng = np.random.default_rng([123, seed])
    offsets = rng.integers(0, 4, size=w.batch)
    tile = int(rng.choice(TILES))
    fused = int(rng.integers(0, 2))
    st, got = run_gpu(w, tile=tile, fused=fused, offsets=offsets)
    assert st == B.PLD_OK
    assert_parity(w, got, f"tile={tile} fused={fused} offsets={offsets.tolist()}")


@pytest.mark.parametrize("tile", TILES)
def test_tile_boundary_lengths(tile):
    """Lengths just around multiples of the tile, over a 2-letter alphabet
    so that matches run across tile edges and through the halo."""
    rng = np.random.default_rng([5, tile])
    lens = sorted({max(0, k * tile + d) for k in (1, 2, 3) for d in (-2, -1, 0, 1, 2, 3, 5)})
    hs = [rng.integers(0, 2, n).astype(np.int32) for n in lens]
    # a long planted copy straddling the first tile edge
    for h in hs:
        if h.size > 200:
            h[-40:] = h[tile - 60:tile - 20] if h.size > tile else h[-40:]
    for n_min, n_max in [(4, 12), (1, 64), (16, 64)]:
        w = wl.Workload(f"edges{tile}", hs, n_min, n_max, 16)
        st, got = run_gpu(w, tile=tile, offsets=rng.integers(0, 4, len(hs)))
        assert st == B.PLD_OK
        assert_parity(w, got, f"tile={tile} n={n_min}..{n_max}")


# ---------------------------------------------------------------------------
# invariances
# ---------------------------------------------------------------------------


def test_repeat_calls_identical():
    """100 calls on one context give identical outputs (the per-request
    reduction slots are cleared correctly between calls)."""
    import torch
    w = wl.config3()
    db = B.DeviceBatch(w.histories)
    ctx = B.pld_create(w.batch, db.max_len)
    try:
        out = B.alloc_outputs(w.batch, w.k_max)
        ref = None
        for i in range(100):
            for t in out:
                t.fill_(-7)
            B.pld_draft_batch_pos(ctx, db.rows, db.lengths, w.batch, w.n_min,
                                  w.n_max, w.k_max, *out)
            cur = [t.clone() for t in out]
            if ref is None:
                ref = cur
            else:
                for a, b in zip(ref, cur):
                    assert torch.equal(a, b), f"call {i} differs"
        assert B.pld_sync(ctx) == B.PLD_OK
    finally:
        B.pld_destroy(ctx)
    assert_parity(w, [t.cpu().numpy() for t in ref], "repeat")


def test_batch_invariance():
    w = wl.fuzz_batch(7)
    _, full = run_gpu(w)
    for b in range(w.batch):
        one = wl.Workload("one", [w.histories[b]], w.n_min, w.n_max, w.k_max)
        _, got = run_gpu(one, max_len=max(1, w.max_len))
        for a, c in zip(full, got):
            assert np.array_equal(a[b], c[0]), f"request {b}"


def test_unused_rows_of_context_untouched():
    """A context sized for more requests than the call uses."""
    w = wl.fuzz_batch(11)
    st, got = run_gpu(w, max_batch=w.batch + 9, max_len=w.max_len + 5000)
    assert st == B.PLD_OK
    assert_parity(w, got, "oversized context")


# ---------------------------------------------------------------------------
# edge cases
# ---------------------------------------------------------------------------


def test_degenerate_requests():
    hs = [np.zeros(0, np.int32), np.array([5], np.int32), np.full(4, 7, np.int32),
          np.full(5, 7, np.int32), np.full(65, 3, np.int32),
          np.arange(100, dtype=np.int32)]
    for n_min, n_max, k_max in [(4, 12, 16), (1, 1, 1), (4, 4, 3), (1, 64, 1000),
                                (64, 64, 2), (3, 64, 5)]:
        w = wl.Workload("degenerate", hs, n_min, n_max, k_max)
        st, got = run_gpu(w)
        assert st == B.PLD_OK
        assert_parity(w, got, f"n={n_min}..{n_max} k={k_max}")


@pytest.mark.parametrize("short", [1, 2, 3])
@pytest.mark.parametrize("n_min", [1, 2, 3])
def test_short_best_match_inside_interior_tiles(short, n_min):
    """The best match is only 1, 2 or 3 tokens long and sits deep inside a
    long history (an interior tile for every tile size): distinct tokens,
    with the last `short` tokens planted once more at a middle position
    behind a different token. Rejection filters must never drop a position
    whose exact match length can still reach n_min."""
    rng = np.random.default_rng([31, short, n_min])
    hs = []
    for L in (20_000, 50_001, 70_003):
        h = rng.permutation(10 * L)[:L].astype(np.int32)
        at = int(rng.integers(L // 3, 2 * L // 3))
        h[at:at + short] = h[L - short:]
        hs.append(h)
    w = wl.Workload("short", hs, n_min, 12, 8)
    od, ol, om, oj = oracle.draft(hs, n_min, 12, 8)
    assert om.tolist() == ([short] * 3 if short >= n_min else [0] * 3)
    for tile in TILES:
        st, got = run_gpu(w, tile=tile, offsets=rng.integers(0, 4, len(hs)))
        assert st == B.PLD_OK
        assert_parity(w, got, f"tile={tile}")


def _lane_boundary_ends(tile: int, L: int, delta: int):
    """End positions at every lane-0 chunk start (offsets 0..3) of every
    wavefront, in the first, an interior and the last tile, plus the last
    positions of each tile (the chunk after the last wavefront's span) and
    the first of the next. A wavefront of a `tile`-token tile covers
    min(tile, 1,024) positions, lane 0's chunks start every 256 positions
    of it, and a row misaligned by `delta` tokens shifts every chunk start
    back by delta."""
    ends = set()
    span = min(tile, 1024)
    for t0 in (0, tile, 3 * tile):
        for w in range(tile // span):
            for k in range(span // 256):
                for i in range(4):
                    ends.add(t0 - delta + w * span + 256 * k + i)
        for i in range(-4, 4):
            ends.add(t0 + tile + i)
    return sorted(e for e in ends if 2 <= e <= L - 5)


@pytest.mark.parametrize("tile", [1024, 2048, 4096])
@pytest.mark.parametrize("delta", [0, 1, 2, 3])
def test_three_token_match_at_every_lane_boundary(tile, delta):
    """The 3-token register test takes the two tokens before lane 0's chunk
    from lane 63 of the previous chunk (or from the halo), across the DPP
    shift. Each request has distinct tokens and one copy of its last three
    tokens, whose last token sits on one of those boundary positions; the
    oracle's answer is that copy (match length 3, start e - 2)."""
    L = 3 * tile + 101
    rng = np.random.default_rng([47, tile, delta])
    ends = _lane_boundary_ends(tile, L, delta)
    hs = []
    for e in ends:
        h = rng.permutation(20 * L)[:L].astype(np.int32)
        h[e - 2:e + 1] = h[L - 3:]
        hs.append(h)
    w = wl.Workload("lane_boundary", hs, 3, 12, 8)
    od, ol, om, oj = oracle.draft(hs, 3, 12, 8)
    assert om.tolist() == [3] * len(ends) and oj.tolist() == [e - 2 for e in ends]
    st, got = run_gpu(w, tile=tile, offsets=[delta] * len(hs))
    assert st == B.PLD_OK
    assert_parity(w, got, f"tile={tile} delta={delta}")


@pytest.mark.parametrize("tile", [1024, 4096])
@pytest.mark.parametrize("n_min", [1, 3, 4])
def test_last_tile_past_the_row_end(tile, n_min):
    """A request's last tile (when it is not also its first) reads its chunks
    through the row's end: the chunk holding the last token whole, the ones
    after it from the zero block. Every history here ends in twelve zeros
    (one earlier run of five zeros sits among nonzero tokens), so the zero
    chunks, the suffix's own position and any zero bytes past the row pass
    the register tests; the answer is the 11-token match that ends one token
    before the row's end, and a position at or past the end would give a
    longer one. The last tile holds 1..tile+6 candidates (the tile before it
    is then interior or a last-tile case too), over all four row alignments."""
    rng = np.random.default_rng([53, tile, n_min])
    counts = sorted({1, 2, 3, 4, 5, 6, 7, 8, 61, 62, 63, 64, 65, 66, 67, 68, 255, 256, 257}
                    | {tile + d for d in range(-6, 7)})
    hs = []
    for c in counts:
        L = tile + 1 + c  # tile 1 holds c candidates (positions tile .. L - 2)
        h = rng.integers(1, 50, L).astype(np.int32)
        h[-12:] = 0
        s = int(rng.integers(5, tile - 10))
        h[s:s + 5] = 0
        hs.append(h)
    for n_max in (12, 64):
        w = wl.Workload("last_tile", hs, n_min, n_max, 16)
        od, ol, om, oj = oracle.draft(hs, n_min, n_max, 16)
        assert om.tolist() == [11] * len(hs) and oj.tolist() == [len(h) - 12 for h in hs]
        for delta in range(4):
            st, got = run_gpu(w, tile=tile, offsets=[delta] * len(hs))
            assert st == B.PLD_OK
            assert_parity(w, got, f"tile={tile} n={n_min}..{n_max} delta={delta}")


def test_periodic_tails_all_periods():
    hs = []
    rng = np.random.default_rng(17)
    for p in range(1, 40):
        blk = rng.permutation(1000)[:p].astype(np.int32)
        pre = rng.integers(2000, 9000, int(rng.integers(0, 5000))).astype(np.int32)
        tail = np.tile(blk, 200)[: 64 + p + int(rng.integers(0, 300))]
        hs.append(np.concatenate([pre, tail]))
    for n_max in (12, 64):
        w = wl.Workload("periodic", hs, 4, n_max, 16)
        st, got = run_gpu(w, offsets=rng.integers(0, 4, len(hs)))
        assert st == B.PLD_OK
        assert_parity(w, got, f"n_max={n_max}")


def test_batch_zero_is_noop():
    ctx = B.pld_create(4, 100)
    try:
        B.pld_draft_batch(ctx, 0, 0, 0, 4, 12, 16, 0, 0, 0)
        assert B.pld_sync(ctx) == B.PLD_OK
    finally:
        B.pld_destroy(ctx)


def test_host_validation_rejects_and_enqueues_nothing():
    import torch
    w = wl.fuzz_batch(2)
    db = B.DeviceBatch(w.histories)
    ctx = B.pld_create(w.batch, db.max_len)
    out = B.alloc_outputs(w.batch, 8)
    for t in out:
        t.fill_(-7)
    try:
        for n_min, n_max, k_max, batch in [(0, 4, 8, w.batch), (5, 4, 8, w.batch),
                                           (1, 65, 8, w.batch), (1, 4, 0, w.batch),
                                           (1, 4, 8, w.batch + 1), (1, 4, 8, -1)]:
            with pytest.raises(B.PldError) as e:
                B.pld_draft_batch_pos(ctx, db.rows, db.lengths, batch, n_min, n_max,
                                      k_max, *out)
            assert e.value.status == B.PLD_EINVAL
        with pytest.raises(B.PldError):
            B.pld_configure(ctx, 512, -1)
        assert B.pld_sync(ctx) == B.PLD_OK
        for t in out:
            assert torch.all(t == -7)
    finally:
        B.pld_destroy(ctx)


def test_device_side_errors_reported_and_cleared():
    """Bad per-request inputs: that request reads as no match, the others are
    unaffected, and pld_sync reports then clears the sticky flag."""
    import torch
    rng = np.random.default_rng(3)
    hs = [rng.integers(0, 3, 500).astype(np.int32) for _ in range(4)]
    w = wl.Workload("errs", hs, 2, 8, 6)
    od, ol, om, oj = oracle.draft(hs, 2, 8, 6)
    db = B.DeviceBatch(hs)
    ctx = B.pld_create(4, 500)
    out = B.alloc_outputs(4, 6)

    def call(rows, lengths):
        for t in out:
            t.fill_(-7)
        B.pld_draft_batch_pos(ctx, rows, lengths, 4, 2, 8, 6, *out)
        return B.pld_sync(ctx), [t.cpu().numpy() for t in out]

    try:
        cases = []
        L = db.lengths.clone(); L[1] = 501                       # > max_len
        cases.append((db.rows, L, B.PLD_ECAPACITY))
        L = db.lengths.clone(); L[1] = -5                        # negative
        cases.append((db.rows, L, B.PLD_EINVAL))
        R = db.rows.clone(); R[1] = R[1] + 2                     # misaligned
        cases.append((R, db.lengths, B.PLD_EINVAL))
        R = db.rows.clone(); R[1] = 0                            # null row
        cases.append((R, db.lengths, B.PLD_EINVAL))
        for rows, lengths, want in cases:
            st, (d, l, m, p) = call(rows, lengths)
            assert st == want
            assert m[1] == 0 and l[1] == 0 and p[1] == -1 and np.all(d[1] == -1)
            for b in (0, 2, 3):
                assert (m[b], p[b], l[b]) == (om[b], oj[b], ol[b])
                assert np.array_equal(d[b], od[b])
            # cleared
            assert B.pld_sync(ctx) == B.PLD_OK
        # a null row with length 0 is fine
        R = db.rows.clone(); R[2] = 0
        L = db.lengths.clone(); L[2] = 0
        st, (d, l, m, p) = call(R, L)
        assert st == B.PLD_OK and m[2] == 0 and np.all(d[2] == -1)
    finally:
        B.pld_destroy(ctx)
    del torch, w


# ---------------------------------------------------------------------------
# streaming: pld_append into the context's store, then re-draft
# ---------------------------------------------------------------------------


def _hip_copy_to_host(dst: np.ndarray, src_ptr: int):
    hip = ctypes.CDLL("libamdhip64.so")
    hip.hipMemcpy.argtypes = [ctypes.c_void_p, ctypes.c_void_p, ctypes.c_size_t, ctypes.c_int]
    assert hip.hipMemcpy(dst.ctypes.data, src_ptr, dst.nbytes, 2) == 0  # device->host


def _stream_run(steps: int, check_every: int = 1):
    """Closed-loop streaming decode: each step drafts all 64 requests, then
    appends 1..16 tokens per request (the draft's tokens while they last,
    then fresh Zipf tokens). The oracle runs the same loop on the CPU; every
    step's drafts are compared."""
    import torch
    start = wl.config5_start()
    B_ = start.batch
    ctx = B.pld_create(B_, wl.STREAM_MAX_LEN, own_store=True)
    try:
        rows, lens = B.pld_histories(ctx)
        init = torch.from_numpy(np.stack(start.histories)).cuda()
        counts0 = torch.full((B_,), wl.STREAM_START_LEN, dtype=torch.int32, device="cuda")
        B.pld_append(ctx, init, wl.STREAM_START_LEN, counts0, B_)
        # oracle-side mirror in one preallocated array
        host = np.zeros((B_, wl.STREAM_MAX_LEN), np.int32)
        hl = np.full(B_, wl.STREAM_START_LEN, np.int64)
        host[:, :wl.STREAM_START_LEN] = np.stack(start.histories)
        out = B.alloc_outputs(B_, start.k_max)
        for step in range(steps):
            B.pld_draft_batch_pos(ctx, rows, lens, B_, start.n_min, start.n_max,
                                  start.k_max, *out)
            d, l, m, p = [t.cpu().numpy() for t in out]
            if step % check_every == 0 or step == steps - 1:
                views = [host[b, :hl[b]] for b in range(B_)]
                od, ol, om, oj = oracle.draft(views, start.n_min, start.n_max, start.k_max)
                bad = np.nonzero((m != om) | (p != oj) | (l != ol)
                                 | np.any(d != od, axis=1))[0]
                assert bad.size == 0, f"step {step}: first diverging request {bad[0]}"
            counts, fresh = wl.stream_step_draws(step)
            tok = wl.compose_append(d, l, counts, fresh)
            for b in range(B_):
                c = int(counts[b])
                host[b, hl[b]:hl[b] + c] = tok[b, :c]
                hl[b] += c
            B.pld_append(ctx, torch.from_numpy(tok).cuda(), tok.shape[1],
                         torch.from_numpy(counts).cuda(), B_)
        assert B.pld_sync(ctx) == B.PLD_OK
        # the store now holds exactly the oracle-side histories
        table = np.zeros(B_, np.int64)
        _hip_copy_to_host(table, rows)
        got_len = np.zeros(B_, np.int32)
        _hip_copy_to_host(got_len, lens)
        assert np.array_equal(got_len, hl)
        for b in (0, 17, 63):
            row = np.zeros(int(hl[b]), np.int32)
            _hip_copy_to_host(row, int(table[b]))
            assert np.array_equal(row, host[b, :hl[b]])
        return hl
    finally:
        B.pld_destroy(ctx)


def test_streaming_all_steps():
    hl = _stream_run(wl.STREAM_STEPS, check_every=1)
    assert hl.max() <= wl.STREAM_MAX_LEN


def test_append_overflow_sets_capacity_flag():
    import torch
    ctx = B.pld_create(2, 10, own_store=True)
    try:
        tok = torch.arange(32, dtype=torch.int32, device="cuda").reshape(2, 16)
        B.pld_append(ctx, tok, 16, torch.tensor([6, 10], dtype=torch.int32, device="cuda"), 2)
        assert B.pld_sync(ctx) == B.PLD_OK
        B.pld_append(ctx, tok, 16, torch.tensor([5, 0], dtype=torch.int32, device="cuda"), 2)
        assert B.pld_sync(ctx) == B.PLD_ECAPACITY
        B.pld_append(ctx, tok, 16, torch.tensor([-1, 0], dtype=torch.int32, device="cuda"), 2)
        assert B.pld_sync(ctx) == B.PLD_EINVAL
        rows, lens = B.pld_histories(ctx)
        got = np.zeros(2, np.int32)
        _hip_copy_to_host(got, lens)
        assert got.tolist() == [6, 10]
        B.pld_store_reset(ctx)
        assert B.pld_sync(ctx) == B.PLD_OK
        _hip_copy_to_host(got, lens)
        assert got.tolist() == [0, 0]
    finally:
        B.pld_destroy(ctx)


# ---------------------------------------------------------------------------
# strided batches (rows at a fixed stride, tiles read ahead of the lengths)
# ---------------------------------------------------------------------------


def run_strided(w, min_len, tile=0, fused=-1, stride=None, max_len=None):
    sb = B.StridedBatch(w.histories, stride=stride)
    ctx = B.pld_create(max(1, w.batch), max_len or max(sb.max_len, min_len, 1))
    try:
        B.pld_configure(ctx, tile, fused)
        out = B.alloc_outputs(w.batch, w.k_max)
        for t in out:
            t.fill_(-7)
        B.pld_draft_batch_strided(ctx, sb.buf, sb.stride, sb.lengths, min_len, w.batch,
                                  w.n_min, w.n_max, w.k_max, *out)
        st = B.pld_sync(ctx)
    finally:
        B.pld_destroy(ctx)
    return st, [t.cpu().numpy() for t in out]


@pytest.mark.parametrize("cfg", [1, 2, 3, 4])
@pytest.mark.parametrize("bound", ["exact", "zero", "half"])
def test_strided_config_parity(cfg, bound):
    w = wl.ALL_CONFIGS[cfg]()
    lmin = int(w.lengths.min())
    min_len = {"exact": lmin, "zero": 0, "half": lmin // 2}[bound]
    st, got = run_strided(w, min_len)
    assert st == B.PLD_OK
    assert_parity(w, got, f"strided min_len={min_len}")


@pytest.mark.parametrize("cfg", [3, 4])
@pytest.mark.parametrize("tile", TILES)
@pytest.mark.parametrize("fused", [1, 0])
def test_strided_every_tiling(cfg, tile, fused):
    w = wl.ALL_CONFIGS[cfg]()
    st, got = run_strided(w, int(w.lengths.min()), tile=tile, fused=fused)
    assert st == B.PLD_OK
    assert_parity(w, got, f"strided tile={tile} fused={fused}")


@pytest.mark.parametrize("seed", range(20))
def test_strided_fuzz(seed):
    w = wl.fuzz_batch(seed)
    rng = np.random.default_rng([321, seed])
    lmin = int(w.lengths.min())
    min_len = int(rng.integers(0, lmin + 1))
    extra = int(rng.integers(0, 3)) * 4
    stride = max(4, -(-max(1, w.max_len) // 4) * 4 + extra)
    st, got = run_strided(w, min_len, tile=int(rng.choice(TILES)),
                          fused=int(rng.integers(0, 2)), stride=stride)
    assert st == B.PLD_OK
    assert_parity(w, got, f"strided min_len={min_len} stride={stride}")


def pinned_batch(seed, L, batch=6, n_min=4, n_max=12, k_max=16):
    """Rows of one length L over small alphabets (long, overlapping matches
    anywhere, also across tile edges) and one large-alphabet row (usually no
    match)."""
    rng = np.random.default_rng([555, seed, L])
    hs = []
    for b in range(batch):
        alpha = 151936 if b == batch - 1 else int(rng.integers(2, 6))
        hs.append(rng.integers(0, alpha, L).astype(np.int32))
    return wl.Workload(f"pinned{seed}_L{L}", hs, n_min, n_max, k_max)


# a batch whose bounds pin every length (min_len equals the stride or
# max_len): the strided scan's interior tiles load before the length is read,
# and every stored length is still checked against the bounds
@pytest.mark.parametrize("L", [2, 3, 5, 13, 64, 67, 68, 69, 255, 256, 257, 1031, 4096, 4097,
                               4100, 8195])
@pytest.mark.parametrize("pin", ["stride", "max_len"])
def test_strided_pinned_lengths(L, pin):
    for n_min, tile, fused in ((4, 0, -1), (1, 256, 1), (2, 1024, 0), (3, 4096, 1)):
        w = pinned_batch(n_min, L, n_min=n_min, n_max=max(n_min, 12))
        if pin == "stride":
            stride = -(-L // 4) * 4
            if stride != L:
                continue  # the stride is a multiple of 4: pinned through max_len only
            st, got = run_strided(w, L, tile=tile, fused=fused, stride=stride, max_len=L + 100)
        else:
            st, got = run_strided(w, L, tile=tile, fused=fused, stride=-(-L // 4) * 4 + 8,
                                  max_len=L)
        assert st == B.PLD_OK
        assert_parity(w, got, f"pinned by {pin} L={L} n_min={n_min} tile={tile} fused={fused}")


@pytest.mark.parametrize("tile", TILES)
@pytest.mark.parametrize("fused", [1, 0])
def test_strided_pinned_every_tiling(tile, fused):
    w = wl.ALL_CONFIGS[4]()
    st, got = run_strided(w, int(w.lengths.min()), tile=tile, fused=fused)
    assert st == B.PLD_OK
    assert_parity(w, got, f"pinned tile={tile} fused={fused}")


@pytest.mark.parametrize("fused", [1, 0])
def test_strided_pinned_bad_stored_lengths(fused):
    """With min_len equal to the stride, a stored length other than min_len
    is an error: that row gets the no-match row and the error is reported;
    the other rows are drafted as usual."""
    L = 9000
    w = pinned_batch(7, L, batch=5)
    sb = B.StridedBatch(w.histories, stride=L)
    od, ol, om, oj = oracle.draft(w.histories, w.n_min, w.n_max, w.k_max)
    for bad, expect in ((L - 1, B.PLD_EINVAL), (-3, B.PLD_EINVAL), (L + 4, B.PLD_ECAPACITY)):
        ctx = B.pld_create(w.batch, L + 64)
        try:
            B.pld_configure(ctx, 0, fused)
            out = B.alloc_outputs(w.batch, w.k_max)
            for t in out:
                t.fill_(-7)
            lens = sb.lengths.clone()
            lens[2] = bad
            B.pld_draft_batch_strided(ctx, sb.buf, sb.stride, lens, L, w.batch, w.n_min,
                                      w.n_max, w.k_max, *out)
            assert B.pld_sync(ctx) == expect
            d, l, m, p = [t.cpu().numpy() for t in out]
            assert (m[2], l[2], p[2]) == (0, 0, -1) and np.all(d[2] == -1)
            for b in (0, 1, 3, 4):
                assert (m[b], p[b], l[b]) == (om[b], oj[b], ol[b]), (bad, b)
                assert np.array_equal(d[b], od[b])
            # the slots were left clean: a second call with good lengths is exact
            B.pld_draft_batch_strided(ctx, sb.buf, sb.stride, sb.lengths, L, w.batch,
                                      w.n_min, w.n_max, w.k_max, *out)
            assert B.pld_sync(ctx) == B.PLD_OK
            assert_parity(w, [t.cpu().numpy() for t in out], f"after bad length {bad}")
        finally:
            B.pld_destroy(ctx)


def test_strided_store_views_match_row_table():
    """The context's own store drafted through its row table and through a
    strided call over the same memory give the same outputs."""
    import torch
    start = wl.config5_start()
    nb = 8
    ctx = B.pld_create(nb, wl.STREAM_MAX_LEN, own_store=True)
    try:
        rows, lens = B.pld_histories(ctx)
        init = torch.from_numpy(np.stack(start.histories[:nb])).cuda()
        B.pld_append(ctx, init, wl.STREAM_START_LEN,
                     torch.full((nb,), wl.STREAM_START_LEN, dtype=torch.int32,
                                device="cuda"), nb)
        table = np.zeros(nb, np.int64)
        _hip_copy_to_host(table, rows)
        pitch = int((table[1] - table[0]) // 4)
        a = B.alloc_outputs(nb, 16)
        b_ = B.alloc_outputs(nb, 16)
        B.pld_draft_batch_pos(ctx, rows, lens, nb, 4, 12, 16, *a)
        B.pld_draft_batch_strided(ctx, int(table[0]), pitch, lens, wl.STREAM_START_LEN,
                                  nb, 4, 12, 16, *b_)
        assert B.pld_sync(ctx) == B.PLD_OK
        for x, y in zip(a, b_):
            assert torch.equal(x, y)
    finally:
        B.pld_destroy(ctx)


def test_strided_errors():
    import torch
    rng = np.random.default_rng(9)
    hs = [rng.integers(0, 3, 600).astype(np.int32) for _ in range(3)]
    sb = B.StridedBatch(hs)
    ctx = B.pld_create(3, 1000)
    out = B.alloc_outputs(3, 5)
    try:
        # host-side: misaligned base, bad stride, min_len out of range
        with pytest.raises(B.PldError):
            B.pld_draft_batch_strided(ctx, sb.buf.data_ptr() + 4, sb.stride, sb.lengths,
                                      0, 3, 2, 8, 5, *out)
        with pytest.raises(B.PldError):
            B.pld_draft_batch_strided(ctx, sb.buf, 6, sb.lengths, 0, 3, 2, 8, 5, *out)
        with pytest.raises(B.PldError):
            B.pld_draft_batch_strided(ctx, sb.buf, sb.stride, sb.lengths, sb.stride + 4,
                                      3, 2, 8, 5, *out)
        # device-side: a length below min_len, and one above the stride
        od, ol, om, oj = oracle.draft(hs, 2, 8, 5)
        L = sb.lengths.clone(); L[1] = 100
        B.pld_draft_batch_strided(ctx, sb.buf, sb.stride, L, 500, 3, 2, 8, 5, *out)
        assert B.pld_sync(ctx) == B.PLD_EINVAL
        d, l, m, p = [t.cpu().numpy() for t in out]
        assert m[1] == 0 and np.all(d[1] == -1)
        for b in (0, 2):
            assert (m[b], p[b], l[b]) == (om[b], oj[b], ol[b]) and np.array_equal(d[b], od[b])
        L = sb.lengths.clone(); L[2] = sb.stride + 1
        B.pld_draft_batch_strided(ctx, sb.buf, sb.stride, L, 0, 3, 2, 8, 5, *out)
        assert B.pld_sync(ctx) == B.PLD_ECAPACITY
        assert B.pld_sync(ctx) == B.PLD_OK
    finally:
        B.pld_destroy(ctx)
    del torch
