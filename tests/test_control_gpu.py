"""GPU parity: pld_control (HIP, gfx950) against the controller oracle, step
after step with the state on the device. Decisions are integers taken from
double-precision estimates that both sides compute in the same order with
each operation rounded on its own, so states, rates and choices must agree
bit for bit.

Inputs are seeded and synthetic."""

from __future__ import annotations

import numpy as np
import pytest

import oracle
from prompt_lookup_gram_amd import binding as B

pytestmark = pytest.mark.gpu
W = B.PLD_CONTROL_STATE_WORDS


@pytest.fixture(scope="module", autouse=True)
def gpu():
    import torch
    assert torch.cuda.is_available(), "GPU tests need a GPU"
    B.load()
    torch.cuda.init()
    yield
    torch.cuda.synchronize()


def dev(a, dtype):
    import torch
    return torch.as_tensor(np.ascontiguousarray(a), dtype=dtype).cuda()


def both_params(**kw):
    op = oracle.ControlParams(**kw)
    gp = B.pld_control_params_default()
    for f in ("alpha", "beta", "margin", "prior_accept", "prior_time", "mtp_tokens"):
        setattr(gp, f, getattr(op, f))
    for i in range(3):
        gp.bucket_edge[i] = op.edge[i]
    return op, gp


def run_parity(op, gp, batch, steps, seed):
    import torch
    rng = np.random.default_rng([7301, seed])
    ctx = B.pld_create(batch, 16)
    state = torch.zeros((batch, W), dtype=torch.float64, device="cuda")
    ostate = np.zeros((batch, W))
    drafted = np.zeros(batch, np.int64)
    last = np.full(batch, -1)
    # per request: how repetitive its text is (lookup acceptance) and how
    # well the model's draft layer does
    rep = rng.uniform(0, 1, batch)
    mtp_ok = rng.uniform(0, 0.6, batch)
    sources = []
    try:
        for t in range(steps):
            # the previous round's outcome, by the source that ran
            p_acc = np.where(last == 2, rep, np.where(last == 1, mtp_ok, 0.0))
            acc = rng.binomial(drafted, p_acc).astype(np.int32)
            tm = np.where(last == 0, 0.5, np.where(last == 1, 1.0, 1.0 + 0.05 * drafted))
            tm = tm * np.exp(0.1 * rng.standard_normal(batch))
            d = np.where(rng.random(batch) < 0.75, rng.integers(1, 17, batch), 0).astype(np.int32)
            m = np.where(d > 0, rng.integers(1, 20, batch), 0).astype(np.int32)
            osrc, orates, ostate = oracle.control(op, acc, tm, d, m, ostate)
            src = torch.full((batch,), -7, dtype=torch.int32, device="cuda")
            rates = torch.full((batch, 3), -7.0, dtype=torch.float64, device="cuda")
            B.pld_control(ctx, gp, dev(acc, torch.int32), dev(tm, torch.float64),
                          dev(d, torch.int32), dev(m, torch.int32), state, batch, src, rates)
            assert B.pld_sync(ctx) == B.PLD_OK
            g_src, g_rates, g_state = src.cpu().numpy(), rates.cpu().numpy(), state.cpu().numpy()
            bad = np.nonzero((g_src != osrc) | np.any(g_rates != orates, axis=1) |
                             np.any(g_state != ostate, axis=1))[0]
            if bad.size:
                b = int(bad[0])
                raise AssertionError(
                    f"seed {seed} step {t}: {bad.size}/{batch} differ; b={b} gpu=({g_src[b]}, "
                    f"{g_rates[b].tolist()}, {g_state[b].tolist()}) oracle=({osrc[b]}, "
                    f"{orates[b].tolist()}, {ostate[b].tolist()})")
            drafted = ostate[:, 10].astype(np.int64)
            last = ostate[:, 8].astype(np.int64) - 1
            sources.append(osrc)
    finally:
        B.pld_destroy(ctx)
    return np.array(sources)


def test_control_default_parameters():
    op, gp = both_params()
    src = run_parity(op, gp, batch=300, steps=120, seed=0)
    # every source is chosen somewhere
    assert set(np.unique(src)) == {0, 1, 2}


@pytest.mark.parametrize("seed", range(1, 7))
def test_control_random_parameters(seed):
    rng = np.random.default_rng([7302, seed])
    op, gp = both_params(alpha=float(rng.uniform(0, 1)), beta=float(rng.uniform(0, 1)),
                         margin=float(rng.uniform(0.5, 2.0)),
                         prior_accept=float(rng.uniform(0, 1)),
                         prior_time=float(rng.uniform(0.5, 2)),
                         mtp_tokens=int(rng.integers(0, 6)),
                         edge=tuple(sorted(rng.integers(1, 16, 3).tolist())))
    run_parity(op, gp, batch=97, steps=60, seed=seed)


def test_control_hand_decisions():
    """The hand-derived decisions of the oracle's pins, on the GPU."""
    import torch
    from test_control_oracle_pins import HAND_DECISIONS
    ctx = B.pld_create(len(HAND_DECISIONS), 16)
    try:
        n = len(HAND_DECISIONS)
        d = np.array([h[0] for h in HAND_DECISIONS], np.int32)
        m = np.array([h[1] for h in HAND_DECISIONS], np.int32)
        state = torch.zeros((n, W), dtype=torch.float64, device="cuda")
        src = torch.empty(n, dtype=torch.int32, device="cuda")
        rates = torch.empty((n, 3), dtype=torch.float64, device="cuda")
        B.pld_control(ctx, B.pld_control_params_default(), dev(np.zeros(n), torch.int32),
                      dev(np.ones(n), torch.float64), dev(d, torch.int32), dev(m, torch.int32),
                      state, n, src, rates)
        assert B.pld_sync(ctx) == B.PLD_OK
        assert src.cpu().tolist() == [h[2] for h in HAND_DECISIONS]
        assert rates.cpu().numpy().tolist() == [list(h[3]) for h in HAND_DECISIONS]
    finally:
        B.pld_destroy(ctx)


def test_control_bad_outcomes_flagged():
    """An outcome out of range is not folded in and sets the flag; the
    choice is still made; other requests are unaffected."""
    import torch
    ctx = B.pld_create(3, 16)
    try:
        p = B.pld_control_params_default()
        state = torch.zeros((3, W), dtype=torch.float64, device="cuda")
        src = torch.empty(3, dtype=torch.int32, device="cuda")
        d = dev([4, 4, 4], torch.int32)
        m = dev([12, 12, 12], torch.int32)
        B.pld_control(ctx, p, dev([0, 0, 0], torch.int32), dev([1.0] * 3, torch.float64), d, m,
                      state, 3, src)
        assert B.pld_sync(ctx) == B.PLD_OK and src.cpu().tolist() == [2, 2, 2]
        before = state.cpu().numpy().copy()
        # request 0: fine; 1: accepted 5 of 4; 2: time 0
        B.pld_control(ctx, p, dev([4, 5, 2], torch.int32), dev([1.0, 1.0, 0.0], torch.float64),
                      d, m, state, 3, src)
        assert B.pld_sync(ctx) == B.PLD_EINVAL
        after = state.cpu().numpy()
        assert (after[1, :8] == before[1, :8]).all() and (after[2, :8] == before[2, :8]).all()
        assert after[0, 3] == 0.1 * 1.0 + 0.9 * 0.5
        with pytest.raises(B.PldError):
            bad = B.pld_control_params_default()
            bad.alpha = 1.5
            B.pld_control(ctx, bad, dev([0] * 3, torch.int32), dev([1.0] * 3, torch.float64),
                          d, m, state, 3, src)
    finally:
        B.pld_destroy(ctx)


@pytest.mark.parametrize("fused_gather", [1, 0])
def test_draft_control_batch_matches_oracles(fused_gather):
    """pld_draft_control_batch (the lookup draft and the controller step in
    one launch; with fused_gather 0 the gather kernel runs the step): every
    step drafts prefixes of random length of the ragged workload's 64
    histories, so drafts and match lengths change from step to step; the
    draft must equal the lookup oracle's and the controller's state, rates
    and choices the controller oracle's fed with those drafts."""
    import torch
    from prompt_lookup_gram_amd import workloads as wl
    w = wl.config3()
    batch = w.batch
    db = B.DeviceBatch(w.histories)
    ctx = B.pld_create(batch, db.max_len)
    B.pld_configure(ctx, 0, fused_gather)
    op, gp = both_params(margin=1.02)
    rng = np.random.default_rng([7302, fused_gather])
    state = torch.zeros((batch, W), dtype=torch.float64, device="cuda")
    ostate = np.zeros((batch, W))
    drafted = np.zeros(batch, np.int64)
    seen = set()
    try:
        for t in range(40):
            lens = np.array([int(rng.integers(1, len(h) + 1)) for h in w.histories], np.int32)
            acc = np.array([rng.integers(0, k + 1) for k in drafted], np.int32)
            tm = rng.uniform(0.3, 2.0, batch)
            out = B.alloc_outputs(batch, w.k_max)
            src = torch.full((batch,), -7, dtype=torch.int32, device="cuda")
            rates = torch.full((batch, 3), -7.0, dtype=torch.float64, device="cuda")
            B.pld_draft_control_batch(ctx, db.rows, dev(lens, torch.int32), batch, w.n_min,
                                      w.n_max, w.k_max, out[0], out[1], out[2], gp,
                                      dev(acc, torch.int32), dev(tm, torch.float64), state, src,
                                      rates)
            assert B.pld_sync(ctx) == B.PLD_OK
            prefixes = [h[:n] for h, n in zip(w.histories, lens)]
            od, ol, om, _ = oracle.draft(prefixes, w.n_min, w.n_max, w.k_max)
            assert np.array_equal(out[0].cpu().numpy(), od), f"step {t}: draft"
            assert np.array_equal(out[1].cpu().numpy(), ol) and np.array_equal(
                out[2].cpu().numpy(), om)
            osrc, orates, ostate = oracle.control(op, acc, tm, ol, om, ostate)
            assert np.array_equal(src.cpu().numpy(), osrc), f"step {t}: source"
            assert np.array_equal(rates.cpu().numpy(), orates), f"step {t}: rates"
            assert np.array_equal(state.cpu().numpy(), ostate), f"step {t}: state"
            drafted = ostate[:, 10].astype(np.int64)
            seen |= set(osrc.tolist())
    finally:
        B.pld_destroy(ctx)
    assert len(seen) >= 2  # the trace reaches more than one source


def test_draft_control_batch_rejects_bad_arguments():
    import torch
    ctx = B.pld_create(4, 64)
    try:
        gp = B.pld_control_params_default()
        gp.alpha = 2.0
        out = B.alloc_outputs(4, 8)
        z = torch.zeros(4, dtype=torch.int32, device="cuda")
        with pytest.raises(B.PldError):
            B.pld_draft_control_batch(ctx, torch.zeros(4, dtype=torch.int64, device="cuda"), z,
                                      4, 4, 12, 8, out[0], out[1], out[2], gp, z,
                                      torch.ones(4, dtype=torch.float64, device="cuda"),
                                      torch.zeros((4, W), dtype=torch.float64, device="cuda"), z)
    finally:
        B.pld_destroy(ctx)
