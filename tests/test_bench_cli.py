"""bench.py's contract pieces that need no GPU: the one-GPU refusal and the traffic bookkeeping."""
import os
import subprocess
import sys

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
sys.path.insert(0, ROOT)

import bench  # noqa: E402


def test_bench_refuses_several_gpus():
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"], capture_output=True, text=True,
                       timeout=120)
    assert r.returncode == 2
    assert "one GPU" in r.stderr


def test_traffic_reported_only_for_the_measured_sources(monkeypatch):
    for which in ("prefill", "decode"):
        rec = dict(bench.MEASURED_TRAFFIC[which])
        monkeypatch.setitem(bench.MEASURED_TRAFFIC, which, dict(rec, sources=bench.sources_digest(which)))
        assert bench.traffic(which) == rec["fetch_bytes"] + rec["write_bytes"]
        monkeypatch.setitem(bench.MEASURED_TRAFFIC, which, dict(rec, sources="0" * 16))
        assert bench.traffic(which) is None


def test_committed_traffic_records_match_the_kernel_sources():
    # The byte counters in bench.py were taken on the kernels as committed: a kernel edit without
    # new counter runs makes the bench report traffic as null, and this test says so.
    for which in ("prefill", "decode"):
        assert bench.MEASURED_TRAFFIC[which]["sources"] == bench.sources_digest(which), which
        assert bench.traffic(which) is not None
