"""bench.py's host-side contract (no GPU): the one-GPU rule and the reading of
the committed counter summary."""
import os
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
sys.path.insert(0, ROOT)
import bench  # noqa: E402


def test_more_than_one_gpu_is_refused():
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"],
                       capture_output=True, text=True, timeout=120)
    assert r.returncode == 2
    assert "one GPU" in r.stderr
    assert r.stdout == ""


def test_traffic_follows_the_sources_hash(tmp_path, monkeypatch):
    h = bench.kernel_sources_sha256()
    assert len(h) == 64 and h == bench.kernel_sources_sha256()
    prof = tmp_path / "traffic.md"
    prof.write_text("text\n\ntraffic_bytes_per_launch: 123456\nsources_sha256: " + h + "\n")
    monkeypatch.setattr(bench, "TRAFFIC_PROFILE", str(prof))
    assert bench.measured_traffic() == 123456
    # counters taken with other sources are not reported
    prof.write_text("traffic_bytes_per_launch: 123456\nsources_sha256: " + "0" * 64 + "\n")
    assert bench.measured_traffic() is None
    # a missing or malformed summary reads as unknown, never as an error
    prof.write_text("traffic_bytes_per_launch: many\nsources_sha256: " + h + "\n")
    assert bench.measured_traffic() is None
    monkeypatch.setattr(bench, "TRAFFIC_PROFILE", str(tmp_path / "absent.md"))
    assert bench.measured_traffic() is None


def test_committed_summary_is_well_formed():
    with open(bench.TRAFFIC_PROFILE) as f:
        kv = dict(l.split(": ", 1) for l in f.read().splitlines() if l.startswith(("traffic_", "sources_")))
    assert int(kv["traffic_bytes_per_launch"]) > 0
    assert len(kv["sources_sha256"].strip()) == 64
