"""Call-to-call coverage of the cross-workgroup merge, where it is busiest.

The fused gather's last workgroup reads and clears the request's reduction
slot; a slot left dirty, or a merge that loses a maximum, would show as a
call that differs from the one before it. Each test makes 100 calls back to
back on one context (no host synchronisation between them, every call's
outputs kept) and checks every call against the oracle, stopping at the
first mismatch. Also here: the automatic tile choice across calls whose
batch changes it, and the sticky error word read across streams."""

from __future__ import annotations

import numpy as np
import pytest

import oracle
from prompt_lookup_gram_amd import binding as B
from prompt_lookup_gram_amd import workloads as wl

pytestmark = pytest.mark.gpu

CALLS = 100


@pytest.fixture(scope="module", autouse=True)
def gpu():
    import torch
    assert torch.cuda.is_available(), "GPU tests need a GPU"
    B.load()
    torch.cuda.init()
    yield
    torch.cuda.synchronize()


def _outs(calls: int, batch: int, k_max: int):
    import torch
    return (torch.full((calls, batch, k_max), -7, dtype=torch.int32, device="cuda"),
            torch.full((calls, batch), -7, dtype=torch.int32, device="cuda"),
            torch.full((calls, batch), -7, dtype=torch.int32, device="cuda"),
            torch.full((calls, batch), -7, dtype=torch.int32, device="cuda"))


def _first_mismatch(w, outs, label):
    od, ol, om, oj = oracle.draft(w.histories, w.n_min, w.n_max, w.k_max)
    d, l, m, p = [t.cpu().numpy() for t in outs]
    for i in range(d.shape[0]):
        bad = np.nonzero((m[i] != om) | (p[i] != oj) | (l[i] != ol)
                         | np.any(d[i] != od, axis=1))[0]
        if bad.size:
            b = int(bad[0])
            raise AssertionError(
                f"{label}: call {i} differs for {bad.size}/{w.batch} requests; first b={b} "
                f"gpu=(m={m[i][b]}, j={p[i][b]}, d={l[i][b]}) oracle=(m={om[b]}, j={oj[b]}, "
                f"d={ol[b]})")


@pytest.mark.parametrize("cfg", [4, 2])
def test_repeat_default_tile(cfg):
    """Workload 4 (16 x 262,144: 64 workgroups per request count in on one
    slot) and workload 2 (8 x 25,000 at its automatic 1,024-token tile:
    25 per request), 100 calls back to back."""
    w = wl.ALL_CONFIGS[cfg]()
    db = B.DeviceBatch(w.histories)
    ctx = B.pld_create(w.batch, db.max_len)
    try:
        tile = B.pld_scan_tile(ctx, w.batch)
        tiles = -(-(db.max_len - 1) // tile)
        assert tiles > 1, "the test needs requests split over several workgroups"
        if cfg == 2:
            assert tile == 1024
        outs = _outs(CALLS, w.batch, w.k_max)
        for i in range(CALLS):
            B.pld_draft_batch_pos(ctx, db.rows, db.lengths, w.batch, w.n_min, w.n_max,
                                  w.k_max, outs[0][i], outs[1][i], outs[2][i], outs[3][i])
        assert B.pld_sync(ctx) == B.PLD_OK
    finally:
        B.pld_destroy(ctx)
    _first_mismatch(w, outs, f"workload {cfg}, tile {tile} ({tiles} per request)")


def test_repeat_pinned_strided():
    """Workload 4 as one [16, 262,144] buffer whose stride pins every length:
    the strided scan, whose interior tiles issue their loads before reading
    the stored lengths, 100 calls back to back."""
    w = wl.config4()
    sb = B.StridedBatch(w.histories)
    assert sb.min_len == sb.stride == sb.max_len  # the pinned case
    ctx = B.pld_create(w.batch, sb.max_len)
    try:
        outs = _outs(CALLS, w.batch, w.k_max)
        for i in range(CALLS):
            B.pld_draft_batch_strided(ctx, sb.buf, sb.stride, sb.lengths, sb.min_len, w.batch,
                                      w.n_min, w.n_max, w.k_max, outs[0][i], outs[1][i],
                                      outs[2][i], outs[3][i])
        assert B.pld_sync(ctx) == B.PLD_OK
    finally:
        B.pld_destroy(ctx)
    _first_mismatch(w, outs, "pinned strided workload 4")


def test_repeat_append_draft_steps():
    """100 streaming steps of workload 5 in one launch each
    (pld_append_draft_store, default tile), back to back: the appended
    tokens come from the oracle's own drafts, computed beforehand, so no
    step waits for the host; every step's draft is then checked."""
    import torch
    start = wl.config5_start()
    nb, k = start.batch, start.k_max
    hist = [h.copy() for h in start.histories]
    od, ol, _, _ = oracle.draft(hist, start.n_min, start.n_max, k)
    toks, cnts, want = [], [], []
    for step in range(CALLS):
        counts, fresh = wl.stream_step_draws(step)
        tok = wl.compose_append(od, ol, counts, fresh)
        for b in range(nb):
            hist[b] = np.concatenate([hist[b], tok[b, :counts[b]]]).astype(np.int32)
        od, ol, om, oj = oracle.draft(hist, start.n_min, start.n_max, k)
        toks.append(tok)
        cnts.append(counts)
        want.append((od, ol, om, oj))
    ctx = B.pld_create(nb, wl.STREAM_MAX_LEN, own_store=True)
    try:
        init = np.stack(start.histories).astype(np.int32)
        B.pld_append(ctx, torch.from_numpy(init).cuda(), wl.STREAM_START_LEN,
                     torch.full((nb,), wl.STREAM_START_LEN, dtype=torch.int32, device="cuda"),
                     nb)
        tok_d = torch.from_numpy(np.stack(toks)).cuda()
        cnt_d = torch.from_numpy(np.stack(cnts).astype(np.int32)).cuda()
        outs = _outs(CALLS, nb, k)
        for i in range(CALLS):
            B.pld_append_draft_store(ctx, tok_d[i], tok_d.shape[2], cnt_d[i], nb, start.n_min,
                                     start.n_max, k, outs[0][i], outs[1][i], outs[2][i],
                                     outs[3][i])
        assert B.pld_sync(ctx) == B.PLD_OK
    finally:
        B.pld_destroy(ctx)
    d, l, m, p = [t.cpu().numpy() for t in outs]
    for i, (wd, wlen, wm, wj) in enumerate(want):
        ok = (np.array_equal(d[i], wd) and np.array_equal(l[i], wlen)
              and np.array_equal(m[i], wm) and np.array_equal(p[i], wj))
        assert ok, f"append+draft step {i} differs from the oracle"


def test_tile_setting_round_trip():
    """An explicit tile, then -1 (back to the automatic rule), then 0 (keep):
    pld_scan_tile reports each, and every call matches the oracle."""
    w = wl.config2()
    db = B.DeviceBatch(w.histories)
    ctx = B.pld_create(w.batch, db.max_len)
    try:
        auto = B.pld_scan_tile(ctx, w.batch)
        for setting, want in ((4096, 4096), (-1, auto), (256, 256), (0, 256), (-1, auto)):
            B.pld_configure(ctx, setting, -1)
            assert B.pld_scan_tile(ctx, w.batch) == want, setting
            out = B.alloc_outputs(w.batch, w.k_max)
            for t in out:
                t.fill_(-7)
            B.pld_draft_batch_pos(ctx, db.rows, db.lengths, w.batch, w.n_min, w.n_max,
                                  w.k_max, *out)
            assert B.pld_sync(ctx) == B.PLD_OK
            _first_mismatch(w, [t.unsqueeze(0) for t in out], f"tile setting {setting}")
    finally:
        B.pld_destroy(ctx)


def test_automatic_tile_changes_between_calls():
    """One context (max_len 49,152) drafting batches of 1, 8 and 64
    requests in turn: the automatic tile moves between 1,024 and 2,048
    tokens, and the per-request slots (shared between calls with different
    arrival counts) must come back clean every time. A second context whose
    requests fit one 4,096-token tile takes that tile, with no merge."""
    start = wl.config5_start()
    hs = [np.concatenate([h, h[:16384]]).astype(np.int32) for h in start.histories]
    full = wl.Workload("c5_49152", hs, 4, 12, 16)
    ctx = B.pld_create(64, 49_152)
    try:
        seen = set()
        for rnd in range(3):
            for nb in (1, 8, 64):
                w = wl.Workload(f"b{nb}", full.histories[:nb], 4, 12, 16)
                db = B.DeviceBatch(w.histories)
                tile = B.pld_scan_tile(ctx, nb)
                seen.add(tile)
                out = B.alloc_outputs(nb, 16)
                for t in out:
                    t.fill_(-7)
                B.pld_draft_batch_pos(ctx, db.rows, db.lengths, nb, 4, 12, 16, *out)
                assert B.pld_sync(ctx) == B.PLD_OK
                _first_mismatch(w, [t.unsqueeze(0) for t in out], f"round {rnd} batch {nb}")
        assert seen == {1024, 2048}, seen
    finally:
        B.pld_destroy(ctx)
    small = wl.config1()
    db = B.DeviceBatch(small.histories)
    ctx = B.pld_create(1, 4000)
    try:
        assert B.pld_scan_tile(ctx, 1) == 4096
    finally:
        B.pld_destroy(ctx)


def test_sync_sees_errors_from_other_streams():
    """pld_sync waits for the whole device before it reads the error word:
    a bad length drafted on one stream and an append past capacity made on
    another (queued behind the first) are both reported by a pld_sync given
    only the first stream."""
    import torch
    ctx = B.pld_create(4, 64, own_store=True)
    try:
        s1, s2 = torch.cuda.Stream(), torch.cuda.Stream()
        h = torch.arange(32, dtype=torch.int32, device="cuda")
        rows = torch.tensor([h.data_ptr()] * 4, dtype=torch.int64, device="cuda")
        lens = torch.tensor([32, -3, 32, 32], dtype=torch.int32, device="cuda")
        out = B.alloc_outputs(4, 16)
        tok = torch.zeros((4, 80), dtype=torch.int32, device="cuda")
        counts = torch.tensor([80, 1, 1, 1], dtype=torch.int32, device="cuda")
        torch.cuda.synchronize()
        with torch.cuda.stream(s1):
            B.pld_draft_batch_pos(ctx, rows, lens, 4, 4, 12, 16, *out, stream=s1)
        ev = torch.cuda.Event()
        ev.record(s1)
        s2.wait_event(ev)
        with torch.cuda.stream(s2):
            B.pld_append(ctx, tok, 80, counts, 4, stream=s2)
        st = B.pld_sync(ctx, s1)
        msg = B.pld_last_error()
        assert st == B.PLD_ECAPACITY, (st, msg)
        assert "append past max_len" in msg and "negative length" in msg, msg
        # both bits were read and cleared by that one call
        assert B.pld_sync(ctx, s1) == B.PLD_OK
    finally:
        B.pld_destroy(ctx)


def _every_tile_matches(batch: int, L: int, tile: int, seed: int):
    """Histories of distinct tokens in which every span of `tile` positions
    (but the last two) holds one copy of the history's last l tokens, l
    drawn from 4..12 per span, ending at a random position inside the span:
    with the span a tile, every workgroup of the request has its own
    maximum; with the span a wavefront's share of a tile, every wavefront
    has. The request's key is raised many times, in whatever order the
    workgroups and wavefronts reach the merge."""
    rng = np.random.default_rng([61, seed])
    hs = []
    for _ in range(batch):
        h = rng.permutation(20 * L)[:L].astype(np.int32)
        suffix = h[L - 12:].copy()
        for t in range((L - 1) // tile - 1):
            ell = int(rng.integers(4, 13))
            e = t * tile + int(rng.integers(ell + 1, tile - 1))
            h[e - ell + 1:e + 1] = suffix[12 - ell:]
        hs.append(h)
    return wl.Workload(f"every_tile_{seed}", hs, 4, 12, 16)


@pytest.mark.parametrize("tile", [256, 1024, 4096])
def test_repeat_every_tile_raises_the_maximum(tile):
    """Every workgroup of a request has a match (up to 255 per request at
    256-token tiles), 20 calls back to back, each checked against the
    oracle: the merge's key increases must add up to the maximum in every
    order the workgroups arrive in."""
    w = _every_tile_matches(8, 65_536, tile, tile)
    od, ol, om, oj = oracle.draft(w.histories, w.n_min, w.n_max, w.k_max)
    assert (om >= 4).all()
    db = B.DeviceBatch(w.histories)
    ctx = B.pld_create(w.batch, db.max_len)
    try:
        B.pld_configure(ctx, tile, 1)
        outs = _outs(20, w.batch, w.k_max)
        for i in range(20):
            B.pld_draft_batch_pos(ctx, db.rows, db.lengths, w.batch, w.n_min, w.n_max,
                                  w.k_max, outs[0][i], outs[1][i], outs[2][i], outs[3][i])
        assert B.pld_sync(ctx) == B.PLD_OK
    finally:
        B.pld_destroy(ctx)
    _first_mismatch(w, outs, f"every tile matching, tile {tile}")


@pytest.mark.parametrize("tile", [2048, 4096])
def test_repeat_every_wavefront_raises_the_maximum(tile):
    """Every wavefront of every workgroup has a match (a copy planted in each
    1,024-position wavefront span; 2 or 4 wavefronts per workgroup), 20
    calls back to back, each checked against the oracle: each wavefront's
    atomicMax increase must reach its workgroup's arrival add, and the
    increases must add up to the maximum in every order."""
    w = _every_tile_matches(8, 65_536, 1024, 7 + tile)
    od, ol, om, oj = oracle.draft(w.histories, w.n_min, w.n_max, w.k_max)
    assert (om >= 4).all()
    db = B.DeviceBatch(w.histories)
    ctx = B.pld_create(w.batch, db.max_len)
    try:
        B.pld_configure(ctx, tile, 1)
        outs = _outs(20, w.batch, w.k_max)
        for i in range(20):
            B.pld_draft_batch_pos(ctx, db.rows, db.lengths, w.batch, w.n_min, w.n_max,
                                  w.k_max, outs[0][i], outs[1][i], outs[2][i], outs[3][i])
        assert B.pld_sync(ctx) == B.PLD_OK
    finally:
        B.pld_destroy(ctx)
    _first_mismatch(w, outs, f"every wavefront matching, tile {tile}")
