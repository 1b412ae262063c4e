"""Host-side parts of bench.py's output contract (no GPU needed)."""
import os
import subprocess
import sys

import bench

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def test_traffic_tied_to_the_measured_kernel_code(tmp_path, monkeypatch):
    """The stored fwd traffic is reported only for the kernel code it was measured on: an
    edited kernel reports null until its counters are taken again; edited comments or
    whitespace do not change the code."""
    measured = tmp_path / "fwd_bf16.hip"
    with open(bench.FWD_SRC, "rb") as f:
        src = f.read().decode()
    measured.write_text(src)
    monkeypatch.setattr(bench, "FWD_SRC", str(measured))
    monkeypatch.setattr(bench, "FWD_TRAFFIC_SRC_SHA256", bench.fwd_source_sha())
    assert bench.fwd_traffic_bytes() == bench.FWD_TRAFFIC_BYTES
    measured.write_text("// a new first line\n" + src.replace("\n", "\n  \n", 3) + "\n/* trailing\n block */\n")
    assert bench.fwd_traffic_bytes() == bench.FWD_TRAFFIC_BYTES
    measured.write_text(src.replace("constexpr int kKAhead = 4;", "constexpr int kKAhead = 3;"))
    assert src != measured.read_text()
    assert bench.fwd_traffic_bytes() is None
    measured.write_text(src + "\nstatic const int extra = 1;\n")
    assert bench.fwd_traffic_bytes() is None


def test_code_hash_ignores_comments_only():
    a = bench.code_sha('int a; // note\n/* block\n comment */ const char* s = "// not a comment";')
    assert a == bench.code_sha('int a;\nconst char* s = "// not a comment";')
    assert a != bench.code_sha('int a;\nconst char* s = "// changed";')
    assert a != bench.code_sha('int b;\nconst char* s = "// not a comment";')


def test_stored_traffic_matches_the_kernel_in_the_tree():
    """The kernel in the tree is the one the stored traffic was measured on."""
    assert bench.fwd_traffic_bytes() == bench.FWD_TRAFFIC_BYTES


def test_more_than_one_gpu_is_refused():
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"], capture_output=True,
                       text=True, timeout=120)
    assert r.returncode == 2
    assert "one GPU" in r.stderr
