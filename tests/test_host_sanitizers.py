"""The C-ABI host code under AddressSanitizer and UndefinedBehaviorSanitizer.

sol_attn_api.cpp is compiled with the sanitizers on its host side only (each
-fsanitize after -Xarch_host: the device code is untouched), linked with the kernel
objects of the normal build and a driver (tests/abi_sanitize_driver.cpp) that feeds
every entry point arguments its checks must reject; the driver checks the status codes
and the sanitizers abort on any memory error or undefined behaviour."""
import os
import shutil
import subprocess

import pytest

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(HERE)
BUILD = os.path.join(ROOT, "_build")
KERNEL_OBJS = ["pool.o", "select.o", "fwd_bf16.o", "fwd_f32.o", "cube.o", "quant.o", "check.o", "probe_mfma.o"]


def _hipcc():
    for cand in (os.environ.get("HIPCC"), "/opt/rocm/bin/hipcc", shutil.which("hipcc")):
        if cand and os.path.exists(cand):
            return cand
    return None


@pytest.mark.timeout(600)
def test_abi_host_code_under_sanitizers(tmp_path):
    hipcc = _hipcc()
    if hipcc is None:
        pytest.skip("hipcc not available")
    if not all(os.path.exists(os.path.join(BUILD, o)) for o in KERNEL_OBJS):
        from block_sparse_attention_attn_amd import build
        build.build()
    san = ["-Xarch_host", "-fsanitize=address", "-Xarch_host", "-fsanitize=undefined",
           "-Xarch_host", "-fno-sanitize-recover=all"]
    common = ["-O1", "-g", "-std=c++17", "--offload-arch=gfx950", "-Xclang", "-target-feature", "-Xclang",
              "-packed-fp32-ops", "-I", os.path.join(ROOT, "include")]
    api = tmp_path / "api_san.o"
    drv = tmp_path / "drv.o"
    exe = tmp_path / "drv"
    subprocess.run([hipcc, *common, "-fPIC", *san, "-x", "hip", "-c",
                    os.path.join(ROOT, "block_sparse_attention_attn_amd", "csrc", "sol_attn_api.cpp"),
                    "-o", str(api)], check=True, capture_output=True)
    subprocess.run([hipcc, *common, *san, "-x", "hip", "-c", os.path.join(HERE, "abi_sanitize_driver.cpp"),
                    "-o", str(drv)], check=True, capture_output=True)
    subprocess.run([hipcc, "--offload-arch=gfx950", *san, str(drv), str(api),
                    *(os.path.join(BUILD, o) for o in KERNEL_OBJS), "-o", str(exe)], check=True, capture_output=True)
    env = dict(os.environ, ASAN_OPTIONS="detect_leaks=0:abort_on_error=1", UBSAN_OPTIONS="halt_on_error=1")
    res = subprocess.run([str(exe)], capture_output=True, text=True, timeout=120, env=env)
    assert res.returncode == 0, res.stdout + res.stderr
    assert "0 failures" in res.stdout
    assert "runtime error" not in res.stderr and "AddressSanitizer" not in res.stderr
