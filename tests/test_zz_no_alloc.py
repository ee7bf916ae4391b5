"""pld_draft_batch_noalloc, the entry point for callers that cannot
allocate, against pld_draft_batch_pos on a context: bit-exact outputs on two
calls in a row (the second smaller, so the static reduction state is reused
with a different batch and tile), against the oracle too, and the error
report of a bad row followed by a clean call. Calls go through the C ABI."""

from __future__ import annotations

import numpy as np
import pytest

import oracle
from prompt_lookup_gram_amd import binding as B
from prompt_lookup_gram_amd import workloads as wl

pytestmark = pytest.mark.gpu


def _poisoned(batch: int, k_max: int):
    out = B.alloc_outputs(batch, k_max)
    for t in out:
        t.fill_(-7)
    return out


def _context_outputs(w, db):
    ctx = B.pld_create(w.batch, db.max_len)
    try:
        ref = _poisoned(w.batch, w.k_max)
        B.pld_draft_batch_pos(ctx, db.rows, db.lengths, w.batch, w.n_min, w.n_max, w.k_max,
                              *ref)
        assert B.pld_sync(ctx) == B.PLD_OK
    finally:
        B.pld_destroy(ctx)
    return ref


def test_noalloc_equals_context_call_on_two_calls_in_a_row():
    import torch
    torch.cuda.set_device(0)
    # 8 x 25,000: split over 25 tiles each, so the static slots carry the
    # cross-workgroup merge; then a smaller ragged batch with other sizes
    for w in (wl.config2(), wl.fuzz_batch(3)):
        db = B.DeviceBatch(w.histories)
        print(f"noalloc: {w.name} batch {w.batch} max_len {db.max_len}", flush=True)
        ref = _context_outputs(w, db)
        got = _poisoned(w.batch, w.k_max)
        err = torch.zeros(1, dtype=torch.int32, device="cuda")
        B.pld_draft_batch_noalloc(db.rows, db.lengths, w.batch, db.max_len, w.n_min, w.n_max,
                                  w.k_max, *got, out_err=err)
        torch.cuda.synchronize()
        for name, a, b in zip(("draft", "len", "match", "pos"), ref, got):
            assert torch.equal(a, b), f"{w.name}: {name} differs from pld_draft_batch_pos"
        assert int(err.item()) == 0
        od, ol, om, oj = oracle.draft(w.histories, w.n_min, w.n_max, w.k_max)
        d, l, m, j = [t.cpu().numpy() for t in got]
        assert np.array_equal(d, od) and np.array_equal(l, ol)
        assert np.array_equal(m, om) and np.array_equal(j, oj)


def test_noalloc_reports_a_bad_row_then_runs_clean():
    import torch
    torch.cuda.set_device(0)
    w = wl.config2()
    db = B.DeviceBatch(w.histories)
    lens = db.lengths.clone()
    lens[3] = db.max_len + 1  # past max_len: no-match row, error bit
    got = _poisoned(w.batch, w.k_max)
    err = torch.zeros(1, dtype=torch.int32, device="cuda")
    B.pld_draft_batch_noalloc(db.rows, lens, w.batch, db.max_len, w.n_min, w.n_max, w.k_max,
                              *got, out_err=err)
    torch.cuda.synchronize()
    assert int(err.item()) != 0
    d, l, m, j = [t.cpu().numpy() for t in got]
    assert (d[3] == -1).all() and l[3] == 0 and m[3] == 0 and j[3] == -1
    od, ol, om, oj = oracle.draft(w.histories, w.n_min, w.n_max, w.k_max)
    keep = np.arange(w.batch) != 3
    assert np.array_equal(d[keep], od[keep]) and np.array_equal(l[keep], ol[keep])
    assert np.array_equal(m[keep], om[keep]) and np.array_equal(j[keep], oj[keep])
    # the same static state serves a clean call right after
    got2 = _poisoned(w.batch, w.k_max)
    err.zero_()
    B.pld_draft_batch_noalloc(db.rows, db.lengths, w.batch, db.max_len, w.n_min, w.n_max,
                              w.k_max, *got2, out_err=err)
    torch.cuda.synchronize()
    assert int(err.item()) == 0
    d2, l2, m2, j2 = [t.cpu().numpy() for t in got2]
    assert np.array_equal(d2, od) and np.array_equal(l2, ol)
    assert np.array_equal(m2, om) and np.array_equal(j2, oj)
