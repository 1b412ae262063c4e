"""Host-side parts of bench.py's output contract (no GPU needed)."""
import os
import subprocess
import sys

import bench

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def test_traffic_tied_to_the_measured_kernel_source(tmp_path, monkeypatch):
    """The stored fwd traffic is reported only for the kernel source it was measured on:
    an edited kernel reports null until its counters are taken again."""
    measured = tmp_path / "fwd_bf16.hip"
    with open(bench.FWD_SRC, "rb") as f:
        measured.write_bytes(f.read())
    monkeypatch.setattr(bench, "FWD_SRC", str(measured))
    monkeypatch.setattr(bench, "FWD_TRAFFIC_SRC_SHA256", bench.fwd_source_sha())
    assert bench.fwd_traffic_bytes() == bench.FWD_TRAFFIC_BYTES
    measured.write_bytes(measured.read_bytes() + b"\n// edited\n")
    assert bench.fwd_traffic_bytes() is None


def test_more_than_one_gpu_is_refused():
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"], capture_output=True,
                       text=True, timeout=120)
    assert r.returncode == 2
    assert "one GPU" in r.stderr
