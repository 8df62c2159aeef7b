"""bench.py's host-side contract (no GPU): the single-GPU refusal, the
source digest and the traffic lookup that keeps stale PMC figures out of
the roofline entry."""
from __future__ import annotations

import os
import subprocess
import sys

import bench

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def test_more_than_one_gpu_exits_with_a_message():
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"],
                       capture_output=True, text=True, timeout=120)
    assert r.returncode == 2
    assert "single GPU" in r.stderr
    assert r.stdout == ""


def test_source_digest_is_stable_and_short():
    d = bench.source_digest()
    assert d == bench.source_digest()
    assert len(d) == 16 and all(c in "0123456789abcdef" for c in d)


def test_traffic_only_for_the_current_sources(tmp_path, monkeypatch):
    prof = tmp_path / "profiles"
    prof.mkdir()
    (prof / "k_x_w_traffic.md").write_text(
        "# k_x\n\n- source_digest: `abcd`\n- hbm_bytes_per_launch: 1234.5\n")
    monkeypatch.setattr(bench, "ROOT", str(tmp_path))
    assert bench.read_traffic("k_x", "w", "abcd") == 1234.5
    assert bench.read_traffic("k_x", "w", "other") is None
    assert bench.read_traffic("k_missing", "w", "abcd") is None


def test_committed_profiles_name_their_digest():
    for name in os.listdir(os.path.join(ROOT, "profiles")):
        if name.endswith("_traffic.md"):
            text = open(os.path.join(ROOT, "profiles", name)).read()
            assert "- source_digest: `" in text, name
            assert "- hbm_bytes_per_launch:" in text, name


def test_stats_reports_median_min_max():
    s = bench._stats([3.0, 1.0, 2.0, 10.0])
    assert s == {"median": 2.5, "min": 1.0, "max": 10.0, "mean": 4.0}
    assert bench._stats([5.0])["median"] == 5.0
    assert abs(bench.NOMINAL_BF16_TFLOPS - 2516.58) < 0.01
