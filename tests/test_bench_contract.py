"""Host-side parts of bench.py's output contract (no GPU needed)."""
import os
import subprocess
import sys

import bench

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def test_traffic_tied_to_the_measured_kernel_source(tmp_path, monkeypatch):
    """The stored fwd traffic is reported only for the kernel source it was measured on:
    an edited kernel reports null until its counters are taken again."""
    assert bench.fwd_traffic_bytes() == bench.FWD_TRAFFIC_BYTES
    edited = tmp_path / "fwd_bf16.hip"
    with open(bench.FWD_SRC, "rb") as f:
        edited.write_bytes(f.read() + b"\n// edited\n")
    monkeypatch.setattr(bench, "FWD_SRC", str(edited))
    assert bench.fwd_traffic_bytes() is None


def test_more_than_one_gpu_is_refused():
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"], capture_output=True,
                       text=True, timeout=120)
    assert r.returncode == 2
    assert "one GPU" in r.stderr
