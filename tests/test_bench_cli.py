"""Host-side checks of bench.py's command line (no GPU needed)."""
import os
import subprocess
import sys

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def test_more_than_one_gpu_is_refused_with_a_message():
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"], capture_output=True,
                       text=True, timeout=300)
    assert r.returncode == 2
    assert "one GPU" in r.stderr
    assert r.stdout == ""  # no JSON line is printed


def test_traffic_is_reported_only_for_the_measured_sources(monkeypatch):
    import bench
    for name, c in bench.COUNTERS.items():
        t = bench.traffic_bytes(name)
        assert t is None or t > 0
        if c["fetch_kib"] is not None:
            # another source than the measured one reads as unmeasured
            monkeypatch.setitem(c, "sha256", "0" * 64)
            assert bench.traffic_bytes(name) is None
    assert bench.traffic_bytes("no such workload") is None
