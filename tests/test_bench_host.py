"""Host logic of bench.py: the exact step counts of its graph replays, the
profile staleness check, and the one-GPU guard (no GPU needed)."""

from __future__ import annotations

import os
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
sys.path.insert(0, ROOT)

import bench  # noqa: E402


@pytest.mark.parametrize("n,g", [(20, 20), (5, 20), (4096, 128), (4100, 128), (0, 7),
                                 (1, 1), (129, 128), (255, 128)])
def test_step_plan_runs_exactly_n_steps(n, g):
    plan = bench.step_plan(n, g)
    assert sum(plan) == n
    assert all(0 < m <= g for m in plan)
    assert len(set(plan)) <= 2
    assert plan == sorted(plan, reverse=True)  # the partial graph runs last


def test_driver_warmup_and_steps_are_exact():
    """--steps 20 --warmup 5: one 20-step and one 5-step graph."""
    g = max(1, min(128, 20))
    assert bench.step_plan(20, g) == [20]
    assert bench.step_plan(5, g) == [5]


def test_profiled_traffic_tracks_the_sources(tmp_path, monkeypatch):
    h = bench.source_hash()
    assert len(h) == 16 and int(h, 16) >= 0
    prof = tmp_path / "profiles"
    prof.mkdir()
    (prof / "good.md").write_text(f"source-sha256-16: {h}\ntraffic-bytes-per-launch: 123\n")
    (prof / "stale.md").write_text("source-sha256-16: 0000000000000000\n"
                                   "traffic-bytes-per-launch: 123\n")
    monkeypatch.setattr(bench, "ROOT", str(tmp_path))
    assert bench.profiled_traffic("good.md") == 123
    assert bench.profiled_traffic("stale.md") is None
    assert bench.profiled_traffic("missing.md") is None
    assert bench.profiled_traffic(None) is None


def test_source_hash_covers_the_launch_code():
    assert "pld_api.cpp" in bench.PROFILED_SOURCES
    assert "pld_kernels.hip" in bench.PROFILED_SOURCES


def test_committed_profiles_name_their_sources():
    """Every summary that gives a traffic figure records the source hash."""
    d = os.path.join(ROOT, "profiles")
    for name in sorted(os.listdir(d)):
        text = open(os.path.join(d, name)).read()
        if "traffic-bytes-per-launch:" in text:
            assert "source-sha256-16:" in text, name


def test_bench_refuses_more_than_one_gpu():
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"],
                       capture_output=True, text=True, timeout=120)
    assert r.returncode == 2
    assert "one GPU" in r.stderr
