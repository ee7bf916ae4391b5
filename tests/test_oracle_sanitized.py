"""The C oracles under AddressSanitizer and UndefinedBehaviorSanitizer (host
only, no GPU).

The oracle sources are compiled with gcc's address and undefined-behaviour
sanitizers (any report aborts the run) and driven from a child Python
process that preloads the sanitizer runtime: lookup drafting on fuzz
batches and edge cases (empty and one-token histories, n_min = n_max,
k_max past every continuation), successor-count drafting, fusion steps with
random parameters and controller steps. Every result must also equal the
plain build's, so the sanitized run checks memory safety without changing
what is computed."""

from __future__ import annotations

import os
import subprocess
import sys
import textwrap

import pytest

import oracle

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))

DRIVER = textwrap.dedent("""
    import sys
    import numpy as np
    sys.path.insert(0, {root!r})
    import oracle
    from prompt_lookup_gram_amd import workloads as wl

    san = oracle.load({lib!r})
    plain = oracle.load()

    def same(a, b):
        return all(np.array_equal(x, y) for x, y in zip(a, b))

    batches = [wl.fuzz_batch(s, max_batch=12, max_len=1500) for s in range(24)]
    edge = [np.zeros(0, np.int32), np.array([5], np.int32), np.array([5, 5], np.int32),
            np.array([7, 7, 7, 7, 7, 7, 7, 7], np.int32), np.arange(40, dtype=np.int32) % 3]
    n = 0
    for w in batches:
        for (n_min, n_max, k_max) in ((w.n_min, w.n_max, w.k_max), (1, 1, 1), (3, 3, 64),
                                      (1, 64, 64)):
            hs = list(w.histories) + edge
            assert same(oracle.draft(hs, n_min, n_max, k_max, lib=san),
                        oracle.draft(hs, n_min, n_max, k_max, lib=plain)), (w.name, n_min)
            n += 1
        p = oracle.NgramParams()
        assert same(oracle.ngram_draft(p, list(w.histories) + edge, 16, lib=san),
                    oracle.ngram_draft(p, list(w.histories) + edge, 16, lib=plain)), w.name
    rng = np.random.default_rng(11)
    for trace in range(8):
        # a fusion trace: state carried, accepted counts within the last block
        fp = oracle.FuseParams(**wl.fuse_params_draw(rng))
        batch = int(rng.integers(1, 9))
        st = np.zeros((batch, oracle.FUSE_STATE_WORDS), np.int32)
        prev = np.zeros(batch, np.int32)
        cp = oracle.ControlParams()
        cst = np.zeros((batch, oracle.CONTROL_STATE_WORDS))
        for step in range(25):
            lookup, d, m, drafter = wl.fuse_step_draws(rng, batch, fp.head)
            acc = np.array([rng.integers(0, q + 1) for q in prev], np.int32)
            a = oracle.fuse(fp, lookup, d, m, drafter, acc, st, lib=san)
            assert same(a, oracle.fuse(fp, lookup, d, m, drafter, acc, st, lib=plain)), step
            st, prev = a[3], a[1]
            # the controller's outcome: accepted within what it drafted last
            cacc = np.array([rng.integers(0, int(k) + 1) for k in cst[:, 10]], np.int32)
            args = (cacc, rng.uniform(0.5, 2.0, size=batch), d, m)
            c = oracle.control(cp, *args, cst, lib=san)
            assert same(c, oracle.control(cp, *args, cst, lib=plain)), step
            cst = c[2]
    print("sanitized oracle runs:", n, flush=True)
""")


def _runtime(name: str) -> str | None:
    p = subprocess.run(["gcc", f"-print-file-name={name}"], capture_output=True, text=True)
    path = p.stdout.strip()
    return path if p.returncode == 0 and os.path.isabs(path) and os.path.exists(path) else None


@pytest.mark.skipif(_runtime("libasan.so") is None, reason="gcc's sanitizer runtime is not installed")
def test_oracles_clean_under_address_and_undefined_sanitizers(tmp_path):
    lib = str(tmp_path / "liboracle_san.so")
    subprocess.run(["gcc", "-O1", "-g", "-std=c11", "-ffp-contract=off", "-fPIC", "-shared",
                    "-fsanitize=address,undefined", "-fno-sanitize-recover=all",
                    "-fno-omit-frame-pointer", "-o", lib, *oracle.sources()], check=True)
    oracle.build(force=False)
    script = tmp_path / "drive.py"
    script.write_text(DRIVER.format(root=ROOT, lib=lib))
    env = dict(os.environ, LD_PRELOAD=_runtime("libasan.so"),
               ASAN_OPTIONS="detect_leaks=0:abort_on_error=1",
               UBSAN_OPTIONS="halt_on_error=1:print_stacktrace=1")
    r = subprocess.run([sys.executable, str(script)], env=env, capture_output=True, text=True,
                       timeout=600)
    assert r.returncode == 0, r.stdout[-2000:] + r.stderr[-4000:]
    assert "sanitized oracle runs:" in r.stdout
