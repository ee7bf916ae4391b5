"""The seeded generators produce the shapes and structure the workloads call
for, reproducibly, and independently per request."""

from __future__ import annotations

import numpy as np

from prompt_lookup_gram_amd import workloads as wl


def test_zipf_law_mass():
    rng = np.random.default_rng(0)
    x = wl.zipf_tokens(rng, 400_000)
    assert x.dtype == np.int32 and x.min() >= 0 and x.max() < wl.ZIPF_VOCAB
    # P(id 0) = 1 / H_{V,1.1} ~ 0.1324 for V = 151,936
    assert abs(np.mean(x == 0) - 0.1324) < 0.003
    # collision probability sum p^2 ~ 0.0261
    p = np.bincount(x, minlength=wl.ZIPF_VOCAB) / x.size
    assert abs(float(np.sum(p * p)) - 0.0261) < 0.002


def test_substitute_changes_exactly_hit_positions():
    rng = np.random.default_rng(1)
    seg = rng.integers(0, 50, 20_000).astype(np.int32)
    out = wl.substitute(np.random.default_rng(2), seg, 0.01, 50)
    frac = float(np.mean(out != seg))
    assert 0.007 < frac < 0.013
    assert out.min() >= 0 and out.max() < 50


def test_config_shapes_and_determinism():
    c1 = wl.config1()
    assert c1.batch == 1 and c1.lengths.tolist() == [4096]
    assert np.array_equal(c1.histories[0], wl.config1().histories[0])
    c2 = wl.config2()
    assert c2.batch == 8 and set(c2.lengths.tolist()) == {25_000}
    assert c2.k_max == 15
    c3 = wl.config3()
    assert c3.batch == 64
    assert c3.lengths.min() >= 8192 and c3.lengths.max() <= 65536
    c4 = wl.config4()
    assert c4.batch == 16 and set(c4.lengths.tolist()) == {262_144}
    assert c4.total_tokens * 4 == 16_777_216
    c5 = wl.config5_start()
    assert c5.batch == 64 and set(c5.lengths.tolist()) == {32_768}
    for w in (c1, c2, c3, c4, c5):
        assert all(h.dtype == np.int32 for h in w.histories)


def test_copy_tails_are_planted():
    c1 = wl.config1()
    h = c1.histories[0]
    tail = h[3584:]
    # the tail occurs verbatim somewhere in the first 3584 tokens
    w = np.lib.stride_tricks.sliding_window_view(h[:3584], 512)
    assert np.any(np.all(w == tail, axis=1))
    c4 = wl.config4()
    h = c4.histories[0]
    tail = h[-4096:]
    w = np.lib.stride_tricks.sliding_window_view(h[:-4096], 32)
    # with 0.5% substitutions most 32-token pieces of the tail are clean
    # copies of a piece of the document
    hits = [bool(np.any(np.all(w == tail[o:o + 32], axis=1)))
            for o in range(0, 4096, 512)]
    assert sum(hits) >= 5


def test_config3_periodic_ends():
    c3 = wl.config3()
    for b in range(3, 64, 4):
        h = c3.histories[b]
        tail = h[-200:]
        # some period 3..20 holds over the whole 200-token tail
        assert any(np.array_equal(tail[p:], tail[:-p]) for p in range(3, 21))


def test_requests_independent_of_batch():
    assert np.array_equal(wl.config2().histories[5],
                          wl._copy_heavy(2, 5, 25_000, 1_000, 0.01))


def test_stream_draws_and_compose():
    counts, fresh = wl.stream_step_draws(0)
    assert counts.shape == (64,) and counts.min() >= 1 and counts.max() <= 16
    assert fresh.shape == (64, 16)
    c2, f2 = wl.stream_step_draws(0)
    assert np.array_equal(counts, c2) and np.array_equal(fresh, f2)
    draft = np.arange(64 * 16, dtype=np.int32).reshape(64, 16)
    dlen = np.full(64, 3, dtype=np.int32)
    tok = wl.compose_append(draft, dlen, counts, fresh)
    for b in range(64):
        a = int(counts[b])
        for t in range(16):
            if t >= a:
                assert tok[b, t] == -1
            elif t < 3:
                assert tok[b, t] == draft[b, t]
            else:
                assert tok[b, t] == fresh[b, t]


def test_fuzz_parameters_in_range():
    for s in range(20):
        w = wl.fuzz_batch(s)
        assert 1 <= w.n_min <= w.n_max <= 64 and w.k_max >= 1
        assert 1 <= w.batch <= 24
