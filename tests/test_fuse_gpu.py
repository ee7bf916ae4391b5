"""GPU parity: pld_fuse (HIP, gfx950) against the fusion oracle, element by
element (fused block including the -1 padding, draft positions, source
masks, and the carried per-request state), step after step with the state
kept on the device. Everything is integer, so the bar is bit-exact.

Inputs are seeded and synthetic (prompt_lookup_gram_amd.workloads)."""

from __future__ import annotations

import numpy as np
import pytest

import oracle
from prompt_lookup_gram_amd import binding as B
from prompt_lookup_gram_amd import workloads as wl
from test_fuse_oracle_pins import read_fuse_cases

pytestmark = pytest.mark.gpu

W = B.PLD_FUSE_STATE_WORDS


@pytest.fixture(scope="module", autouse=True)
def gpu():
    import torch
    assert torch.cuda.is_available(), "GPU tests need a GPU"
    B.load()
    torch.cuda.init()
    yield
    torch.cuda.synchronize()


def to_dev(a, dtype=None):
    import torch
    return torch.as_tensor(np.ascontiguousarray(a), dtype=dtype or torch.int32).cuda()


def gpu_params(p: dict) -> B.PldFuseParams:
    return B.PldFuseParams(*[p[f] for f in wl.FUSE_PARAM_FIELDS])


class GpuFuser:
    """One context and device-resident state for a batch, stepped through
    pld_fuse."""

    def __init__(self, params: dict, batch: int):
        import torch
        self.params, self.batch = params, batch
        self.ctx = B.pld_create(max(batch, 1), 16)
        self.state = torch.zeros((batch, W), dtype=torch.int32, device="cuda")

    def step(self, lookup, d, m, drafter, accepted, poison=True):
        import torch
        n = self.params["positions_long"]
        out_block = torch.full((self.batch, n), -7 if poison else 0, dtype=torch.int32,
                               device="cuda")
        out_pos = torch.full((self.batch,), -7, dtype=torch.int32, device="cuda")
        out_src = torch.full((self.batch,), -7, dtype=torch.int64, device="cuda")
        look = to_dev(lookup)
        B.pld_fuse(self.ctx, gpu_params(self.params), look, look.shape[1], to_dev(d),
                   to_dev(m), to_dev(drafter), to_dev(accepted), self.state, self.batch,
                   out_block, out_pos, out_src)
        st = B.pld_sync(self.ctx)
        return (st, out_block.cpu().numpy(), out_pos.cpu().numpy(),
                out_src.cpu().numpy().view(np.uint64), self.state.cpu().numpy())

    def close(self):
        B.pld_destroy(self.ctx)


@pytest.mark.parametrize("case", read_fuse_cases(), ids=lambda c: c["name"])
def test_fuse_golden_cases(case):
    """The hand-derived cases, on the GPU."""
    params = dict(zip(wl.FUSE_PARAM_FIELDS, case["params"]))
    f = GpuFuser(params, 1)
    try:
        for i, s in enumerate(case["steps"]):
            st, block, pos, src, state = f.step(
                np.array([s["lookup"]]), [s["d"]], [s["m"]], np.array([s["drafter"]]),
                [s["accepted"]])
            assert st == B.PLD_OK
            got = (int(state[0, 0]), int(pos[0]), int(src[0]), block[0].tolist())
            assert got == (s["long"], s["positions"], s["src"], s["block"]), f"step {i}"
    finally:
        f.close()


def run_trace_parity(params: dict, batch: int, steps: int, seed: int, lookup_k: int = 16):
    rng = np.random.default_rng([7101, seed])
    op = oracle.FuseParams(**params)
    ostate = np.zeros((batch, W), np.int32)
    prev_pos = np.zeros(batch, np.int32)
    f = GpuFuser(params, batch)
    try:
        for t in range(steps):
            lookup, d, m, drafter = wl.fuse_step_draws(rng, batch, params["head"], lookup_k)
            acc = np.array([rng.integers(0, p + 1) for p in prev_pos], np.int32)
            ob, opos, osrc, ostate = oracle.fuse(op, lookup, d, m, drafter, acc, ostate)
            st, gb, gpos, gsrc, gstate = f.step(lookup, d, m, drafter, acc)
            assert st == B.PLD_OK
            bad = np.nonzero((gpos != opos) | (gsrc != osrc) | np.any(gb != ob, axis=1) |
                             np.any(gstate != ostate, axis=1))[0]
            if bad.size:
                b = int(bad[0])
                raise AssertionError(
                    f"seed {seed} step {t}: {bad.size}/{batch} requests differ; b={b} "
                    f"d={d[b]} m={m[b]} acc={acc[b]} gpu=({gpos[b]}, {gsrc[b]:#x}, "
                    f"{gb[b].tolist()}, {gstate[b].tolist()}) oracle=({opos[b]}, "
                    f"{osrc[b]:#x}, {ob[b].tolist()}, {ostate[b].tolist()})")
            prev_pos = opos
    finally:
        f.close()


def test_fuse_page_parameters_trace():
    run_trace_parity(dict(zip(wl.FUSE_PARAM_FIELDS, [7, 15, 8, 6, 2, 4, 2, 3, 1])),
                     batch=64, steps=150, seed=0)


@pytest.mark.parametrize("seed", range(1, 9))
def test_fuse_random_parameter_traces(seed):
    params = wl.fuse_params_draw(np.random.default_rng([7102, seed]))
    run_trace_parity(params, batch=33, steps=60, seed=seed)


def test_fuse_largest_block():
    """64 draft positions: every lane of the wavefront holds one."""
    params = dict(zip(wl.FUSE_PARAM_FIELDS, [64, 64, 8, 6, 64, 4, 0, 2, 1]))
    run_trace_parity(params, batch=5, steps=20, seed=11, lookup_k=80)
    params = dict(zip(wl.FUSE_PARAM_FIELDS, [8, 64, 8, 6, 2, 4, 1, 2, 1]))
    run_trace_parity(params, batch=5, steps=40, seed=12, lookup_k=70)


@pytest.mark.parametrize("cfg", [2, 3])
def test_fuse_after_lookup_draft(cfg):
    """The pipeline a decode step runs: pld_draft_batch on a workload, then
    pld_fuse on its outputs, against the two oracles chained the same way."""
    import torch
    w = wl.ALL_CONFIGS[cfg]()
    k = 16
    rng = np.random.default_rng([7103, cfg])
    params = dict(zip(wl.FUSE_PARAM_FIELDS, [7, 15, 8, 6, 2, 4, 2, 3, 1]))
    db = B.DeviceBatch(w.histories)
    ctx = B.pld_create(w.batch, db.max_len)
    state = torch.zeros((w.batch, W), dtype=torch.int32, device="cuda")
    ostate = np.zeros((w.batch, W), np.int32)
    od, ol, om, _ = oracle.draft(w.histories, w.n_min, w.n_max, k)
    prev_pos = np.zeros(w.batch, np.int32)
    try:
        out = B.alloc_outputs(w.batch, k)
        for step in range(6):
            # the drafter agrees with the lookup on some requests
            drafter = rng.integers(0, 50, size=(w.batch, 7)).astype(np.int32)
            agree = rng.random(w.batch) < 0.5
            drafter[agree, :2] = od[agree, :2]
            acc = np.array([rng.integers(max(0, p - 1), p + 1) for p in prev_pos], np.int32)
            B.pld_draft_batch(ctx, db.rows, db.lengths, w.batch, w.n_min, w.n_max, k, *out[:3])
            blk = torch.empty((w.batch, 15), dtype=torch.int32, device="cuda")
            pos = torch.empty(w.batch, dtype=torch.int32, device="cuda")
            src = torch.empty(w.batch, dtype=torch.int64, device="cuda")
            B.pld_fuse(ctx, gpu_params(params), out[0], k, out[1], out[2], to_dev(drafter),
                       to_dev(acc), state, w.batch, blk, pos, src)
            assert B.pld_sync(ctx) == B.PLD_OK
            ob, opos, osrc, ostate = oracle.fuse(oracle.FuseParams(**params), od, ol, om,
                                                 drafter, acc, ostate)
            assert np.array_equal(blk.cpu().numpy(), ob), f"step {step}"
            assert np.array_equal(pos.cpu().numpy(), opos)
            assert np.array_equal(src.cpu().numpy().view(np.uint64), osrc)
            assert np.array_equal(state.cpu().numpy(), ostate)
            prev_pos = opos
        assert (ostate[:, 0] == 1).any(), "the copy-heavy requests reach long blocks"
    finally:
        B.pld_destroy(ctx)


def test_fuse_device_side_errors():
    """Inconsistent per-request inputs: the drafter's head, state reset, the
    sticky flag set; other requests unaffected."""
    params = dict(zip(wl.FUSE_PARAM_FIELDS, [7, 15, 8, 6, 2, 4, 2, 3, 1]))
    f = GpuFuser(params, 4)
    try:
        look = np.tile(np.arange(100, 116, dtype=np.int32), (4, 1))
        dr = np.tile(np.arange(200, 207, dtype=np.int32), (4, 1))
        st, *_ = f.step(look, [16] * 4, [12] * 4, dr, [0] * 4)
        assert st == B.PLD_OK
        # request 1: draft length past the row; 2: accepted above the previous
        # block's 7 positions; 3: negative match; 0 is fine
        st, block, pos, src, state = f.step(look, [16, 17, 16, 16], [12, 12, 12, -1], dr,
                                            [7, 7, 8, 7])
        assert st == B.PLD_EINVAL
        assert "fusion" in B.pld_last_error()
        for b in (1, 2, 3):
            assert pos[b] == 7 and src[b] == 0
            assert block[b].tolist() == list(range(200, 207)) + [-1] * 8
            assert state[b].tolist() == [0, 0, 0, 0]
        # request 0: accepted 7 of 7, a run of 1 (< 2): short, head replaced
        assert pos[0] == 7 and src[0] == 127 and state[0].tolist() == [0, 0, 1, 7]
        assert B.pld_sync(f.ctx) == B.PLD_OK   # the flag was cleared
    finally:
        f.close()


def test_fuse_host_validation():
    import torch
    ctx = B.pld_create(4, 16)
    z = torch.zeros(64, dtype=torch.int32, device="cuda")
    try:
        good = [7, 15, 8, 6, 2, 4, 2, 3, 1]
        bad_sets = {
            "head": [0, 15, 8, 6, 2, 4, 2, 3, 1],
            "positions_long": [7, 6, 8, 6, 1, 4, 2, 3, 1],
            "positions_long_max": [7, 65, 8, 6, 2, 4, 2, 3, 1],
            "agree_tokens": [7, 15, 8, 6, 8, 4, 2, 3, 1],
            "thresholds": [7, 15, 0, 6, 2, 4, 2, 3, 1],
            "sticky": [7, 15, 8, 6, 2, 4, 2, -1, 1],
        }
        for what, vals in bad_sets.items():
            with pytest.raises(B.PldError) as e:
                B.pld_fuse(ctx, B.PldFuseParams(*vals), z, 16, z, z, z, z, z, 1, z, z)
            assert e.value.status == B.PLD_EINVAL, what
        p = B.PldFuseParams(*good)
        with pytest.raises(B.PldError):            # lookup_k
            B.pld_fuse(ctx, p, z, 0, z, z, z, z, z, 1, z, z)
        with pytest.raises(B.PldError):            # batch above max_batch
            B.pld_fuse(ctx, p, z, 16, z, z, z, z, z, 5, z, z)
        raw = B.load().pld_fuse(ctx, B.ctypes.byref(p), z.data_ptr(), 16, z.data_ptr(),
                                z.data_ptr(), z.data_ptr(), z.data_ptr(), z.data_ptr(), 1,
                                z.data_ptr(), z.data_ptr(), z.data_ptr() + 4, None)
        assert raw == B.PLD_EINVAL and "8-byte" in B.pld_last_error()   # misaligned out_src
        B.pld_fuse(ctx, p, z, 16, z, z, z, z, z, 0, z, z)   # batch 0: no-op
        assert B.pld_sync(ctx) == B.PLD_OK
    finally:
        B.pld_destroy(ctx)


# ---------------------------------------------------------------------------
# pld_draft_fuse_batch: lookup drafting and fusion in one launch
# ---------------------------------------------------------------------------

PAGE = dict(zip(wl.FUSE_PARAM_FIELDS, [7, 15, 8, 6, 2, 4, 2, 3, 1]))


def run_one_launch(w, steps, seed, tile=0, fused=-1, params=PAGE, k=None):
    """`steps` decode steps of pld_draft_fuse_batch on one batch (the same
    histories each step, new drafter proposals and accepted counts), against
    oracle.draft followed by oracle.fuse."""
    import torch
    k = k or w.k_max
    rng = np.random.default_rng([7104, seed])
    db = B.DeviceBatch(w.histories)
    ctx = B.pld_create(max(1, w.batch), db.max_len)
    op = oracle.FuseParams(**params)
    n = params["positions_long"]
    od, ol, om, _ = oracle.draft(w.histories, w.n_min, w.n_max, k)
    state = torch.zeros((w.batch, W), dtype=torch.int32, device="cuda")
    ostate = np.zeros((w.batch, W), np.int32)
    prev_pos = np.zeros(w.batch, np.int32)
    try:
        B.pld_configure(ctx, tile, fused)
        for step in range(steps):
            drafter = rng.integers(0, 40, size=(w.batch, params["head"])).astype(np.int32)
            agree = rng.random(w.batch) < 0.5
            a = min(params["agree_tokens"], k)
            drafter[agree, :a] = od[agree, :a]
            acc = np.array([rng.integers(max(0, p - 2), p + 1) for p in prev_pos], np.int32)
            out = B.alloc_outputs(w.batch, k)
            for t in out:
                t.fill_(-7)
            blk = torch.full((w.batch, n), -7, dtype=torch.int32, device="cuda")
            pos = torch.full((w.batch,), -7, dtype=torch.int32, device="cuda")
            src = torch.full((w.batch,), -7, dtype=torch.int64, device="cuda")
            B.pld_draft_fuse_batch(ctx, db.rows, db.lengths, w.batch, w.n_min, w.n_max, k,
                                   out[0], out[1], out[2], gpu_params(params), to_dev(drafter),
                                   to_dev(acc), state, blk, pos, src)
            assert B.pld_sync(ctx) == B.PLD_OK
            ob, opos, osrc, ostate = oracle.fuse(op, od, ol, om, drafter, acc, ostate)
            label = f"{w.name} tile={tile} fused={fused} step={step}"
            assert np.array_equal(out[0].cpu().numpy(), od), label
            assert np.array_equal(out[1].cpu().numpy(), ol), label
            assert np.array_equal(out[2].cpu().numpy(), om), label
            gb = blk.cpu().numpy()
            bad = np.nonzero(np.any(gb != ob, axis=1))[0]
            assert bad.size == 0, f"{label}: block of b={bad[:1]} {gb[bad[:1]]} vs {ob[bad[:1]]}"
            assert np.array_equal(pos.cpu().numpy(), opos), label
            assert np.array_equal(src.cpu().numpy().view(np.uint64), osrc), label
            assert np.array_equal(state.cpu().numpy(), ostate), label
            prev_pos = opos
        return ostate
    finally:
        B.pld_destroy(ctx)


@pytest.mark.parametrize("cfg", [1, 2, 3])
@pytest.mark.parametrize("tile,fused", [(0, -1), (256, 1), (256, 0), (16384, 1), (1024, 0)])
def test_draft_fuse_one_launch(cfg, tile, fused):
    """Every emit site fuses: single-tile requests, the last workgroup of a
    split request, and the separate gather kernel."""
    w = wl.ALL_CONFIGS[cfg]()
    st = run_one_launch(w, steps=5, seed=cfg, tile=tile, fused=fused)
    if cfg in (1, 2):
        assert (st[:, 0] == 1).any(), "copy tails reach long blocks"


def test_draft_fuse_one_launch_long_rows():
    """64 workgroups per request at the 262,144-token rows."""
    run_one_launch(wl.config4(), steps=3, seed=4)


@pytest.mark.parametrize("seed", range(4))
def test_draft_fuse_one_launch_fuzz(seed):
    """Random batches (tiny and empty histories included), random
    parameters, k_max below and above the long block."""
    w = wl.fuzz_batch(100 + seed)
    params = wl.fuse_params_draw(np.random.default_rng([7105, seed]))
    for k in (max(1, params["positions_long"] - 3), params["positions_long"] + 5, 70):
        run_one_launch(w, steps=4, seed=seed, params=params, k=k,
                       tile=(256, 1024)[seed % 2], fused=seed % 2)
