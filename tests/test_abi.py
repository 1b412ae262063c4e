"""The C-ABI library loads on the host and exports what include/sol_attn.h declares, and
its argument checks reject bad calls before anything touches a GPU (no compute calls
here: every call below returns from host-side validation)."""
import ctypes
import os

import pytest

from block_sparse_attention_attn_amd import sol_attn as S


@pytest.fixture(scope="module")
def lib():
    if not os.path.exists(S.LIB_PATH):
        from block_sparse_attention_attn_amd import build
        build.build()
    return S.load_library()


def test_header_symbols_exported(lib):
    names = S.header_symbols()
    assert set(names) == {"sol_attn_pool", "sol_attn_select", "sol_attn_fwd", "sol_attn_last_error",
                          "sol_attn_version", "sol_attn_frame_order", "sol_attn_window_blocks",
                          "sol_attn_cube_permute", "sol_attn_quantize", "sol_attn_dequantize",
                          "sol_attn_check_block_idx", "sol_attn_probe_mfma", "sol_attn_pool_cube",
                          "sol_attn_fwd_cube"}
    raw = ctypes.CDLL(S.LIB_PATH)
    for n in names:
        assert hasattr(raw, n), n


def test_version(lib):
    assert lib.sol_attn_version() == 102


FAKE = 0x10000      # 64 KiB-aligned dummy "device" address; never dereferenced
MIS = FAKE + 2      # misaligned


def _fwd(lib, q=FAKE, k=FAKE, v=FAKE, dtype=0, B=1, H=1, L=256, d=128, block=128, topk=1, idx=FAKE,
         out=FAKE, lse=None, order=None, scale=0.0):
    return lib.sol_attn_fwd(q, k, v, dtype, B, H, L, d, block, topk, idx, order, scale, out, lse, None)


def test_fwd_argument_errors(lib):
    assert _fwd(lib, dtype=7) == 4
    assert _fwd(lib, B=-1) == 2
    assert _fwd(lib, block=0) == 2
    assert _fwd(lib, d=64) == 4                        # bf16 path needs d = block = 128
    assert _fwd(lib, block=64, L=256) == 4
    assert _fwd(lib, dtype=1, d=96, block=64) == 4     # fp32 needs d in {64,128}
    assert _fwd(lib, dtype=1, d=64, block=512, L=1024) == 4
    assert _fwd(lib, topk=0) == 3
    assert _fwd(lib, topk=3) == 3                      # only 2 blocks
    assert _fwd(lib, L=200, topk=3) == 3               # 200 tokens: 2 blocks (the second short)
    assert _fwd(lib, q=None) == 1
    assert _fwd(lib, idx=None) == 1
    assert _fwd(lib, out=None) == 1
    assert _fwd(lib, v=MIS) == 5
    assert _fwd(lib, lse=FAKE + 2) == 5
    assert _fwd(lib, order=FAKE + 1) == 5
    assert b"topk" in lib.sol_attn_last_error() or b"aligned" in lib.sol_attn_last_error()
    assert _fwd(lib, scale=float("inf")) == 2
    assert b"softmax_scale" in lib.sol_attn_last_error()
    assert _fwd(lib, scale=float("inf"), B=0) == 2     # an argument error even with nothing to do


def test_fwd_empty_problem_is_a_noop(lib):
    # zero-element problems are valid and enqueue nothing (no GPU needed)
    assert _fwd(lib, B=0, q=None, k=None, v=None, idx=None, out=None) == 0
    assert _fwd(lib, H=0, topk=99) == 0
    assert _fwd(lib, L=0) == 0
    assert lib.sol_attn_last_error() == b""


def test_pool_argument_errors(lib):
    p = lambda **kw: lib.sol_attn_pool(kw.get("q", FAKE), kw.get("k", FAKE), kw.get("dtype", 0), kw.get("B", 1),  # noqa: E731
                                       kw.get("H", 1), kw.get("L", 256), kw.get("d", 128), kw.get("block", 128),
                                       kw.get("qp", FAKE), kw.get("kp", FAKE), None)
    assert p(dtype=3) == 4
    assert p(L=-1) == 2
    assert p(d=12) == 4          # bf16 pool needs d % 8 == 0
    assert p(d=1024) == 4
    assert p(q=None) == 1
    assert p(kp=None) == 1
    assert p(k=MIS) == 5
    assert p(qp=FAKE + 4) == 5
    assert p(B=0, q=None) == 0


def test_select_argument_errors(lib):
    s = lambda **kw: lib.sol_attn_select(kw.get("qp", FAKE), kw.get("kp", FAKE), kw.get("B", 1), kw.get("H", 1),  # noqa: E731
                                         kw.get("nb", 8), kw.get("d", 128), kw.get("topk", 2), kw.get("idx", FAKE),
                                         kw.get("scores", None), None)
    assert s(topk=0) == 3
    assert s(topk=9) == 3
    assert s(nb=-1) == 2
    assert s(d=0) == 2
    assert s(d=1000) == 4
    assert s(nb=8193, topk=1) == 4
    assert s(idx=None) == 1
    assert s(idx=FAKE + 2) == 5
    assert s(scores=FAKE + 4) == 5
    assert s(nb=0, topk=0) == 0


def test_binding_device_check():
    """Every pointer a kernel dereferences must be on the call's HIP device: host tensors
    and tensors on another device are refused before the library is called."""
    import torch
    cpu = torch.zeros(2, dtype=torch.int32)
    with pytest.raises(ValueError, match="HIP device"):
        S._check_on_device(torch.device("cpu"), x=cpu)
    dev0, dev1 = torch.device("cuda", 0), torch.device("cuda", 1)
    with pytest.raises(ValueError, match="block_idx"):
        S._check_on_device(dev0, block_idx=cpu, out=None)
    meta = torch.empty(2, device="meta")
    with pytest.raises(ValueError, match="lse"):
        S._check_on_device(dev0, lse=meta)
    S._check_on_device(dev0, out=None, lse=None)          # absent tensors are fine
    assert dev0 != dev1


def test_binding_refuses_cpu_tensors(lib):
    import torch
    q = torch.zeros(1, 1, 128, 128, dtype=torch.bfloat16)
    with pytest.raises(ValueError):
        S.sol_attn_pool(q, q, 128)
    qp = torch.zeros(1, 1, 4, 128, dtype=torch.float64)
    with pytest.raises(ValueError):
        S.sol_attn_select(qp, qp, 2)
    codes = torch.zeros(1, 1, 4, 128, dtype=torch.uint8)
    with pytest.raises(ValueError):
        S.sol_attn_dequantize(codes, torch.ones(1, 1, 4), S.INT8)


def test_frame_order(lib):
    import numpy as np
    # 2 frames x 4 rows x 32 cols = 256 tokens, blocks of 32 tokens = one row each
    o = S.sol_attn_frame_order(256, 32, 128, 32).numpy()
    assert o.tolist() == [0, 4, 1, 5, 2, 6, 3, 7]          # row-major across frames
    # blocks straddling rows: key = row of the first token
    o = S.sol_attn_frame_order(4 * 84 * 48, 128, 48 * 84, 84).numpy()
    assert sorted(o.tolist()) == list(range(4 * 84 * 48 // 128))   # a permutation
    first = np.array(o) * 128
    rows = (first % (48 * 84)) // 84
    frames = first // (48 * 84)
    keys = list(zip(rows, frames))
    assert keys == sorted(keys)
    assert lib.sol_attn_frame_order(-1, 32, 64, 32, None) == 2         # negative L
    assert S.sol_attn_frame_order(100, 32, 64, 32).numel() == 4        # a short last block counts
    assert lib.sol_attn_frame_order(128, 32, 64, 65, None) == 2        # row > frame
    assert lib.sol_attn_frame_order(0, 32, 64, 32, None) == 0          # empty


def _perm(lib, src=FAKE, dst=FAKE + 0x100000, B=1, H=1, T=4, h=8, w=8, row_bytes=256, bt=2, by=4, bx=4, inv=0):
    return lib.sol_attn_cube_permute(src, dst, B, H, T, h, w, row_bytes, bt, by, bx, inv, None)


def test_cube_permute_argument_checks(lib):
    assert _perm(lib, T=-1) == 2                       # negative size
    assert _perm(lib, row_bytes=0) == 2                # empty rows
    assert _perm(lib, row_bytes=6) == 2                # not a multiple of 4
    assert _perm(lib, bt=3) == 2                       # box does not divide T
    assert _perm(lib, by=3) == 2                       # ... h
    assert _perm(lib, bx=0) == 2                       # ... w
    assert _perm(lib, inv=2) == 2
    assert _perm(lib, B=65536) == 2                    # grid.y limit
    assert _perm(lib, src=None) == 1
    assert _perm(lib, dst=MIS) == 5
    assert _perm(lib, H=0, src=None) == 0              # nothing to do
    assert _perm(lib, T=0, h=0, w=0) == 0
    assert b"does not tile" in (_perm(lib, by=3), lib.sol_attn_last_error())[1]


def test_pool_cube_argument_checks(lib):
    def p(q=FAKE, k=FAKE, dtype=0, B=1, H=1, T=4, h=16, w=16, d=128, bt=2, by=8, bx=8, qp=FAKE, kp=FAKE):
        return lib.sol_attn_pool_cube(q, k, dtype, B, H, T, h, w, d, bt, by, bx, qp, kp, None)
    assert p(T=-1) == 2
    assert p(bt=3) == 2                        # box does not divide T
    assert p(bx=0) == 2
    assert p(dtype=5) == 4
    assert p(d=12) == 4                        # bf16 pool needs d % 8 == 0
    assert p(B=65536) == 2
    assert p(q=None) == 1
    assert p(k=MIS) == 5
    assert p(kp=FAKE + 4) == 5
    assert p(H=0, q=None) == 0                 # nothing to do
    assert b"does not tile" in (p(by=3), lib.sol_attn_last_error())[1]


def test_fwd_cube_argument_checks(lib):
    def f(q=FAKE, k=FAKE, v=FAKE, B=1, H=1, T=4, h=16, w=16, bt=2, by=8, bx=8, topk=2, idx=FAKE, order=None,
          out=FAKE, lse=None):
        return lib.sol_attn_fwd_cube(q, k, v, B, H, T, h, w, bt, by, bx, topk, idx, order, 0.0, out, lse, None)
    assert f(h=-16) == 2
    assert f(by=3) == 2                        # box does not divide h
    assert f(bt=1, by=4, bx=4) == 4            # 16-token boxes: needs 128
    assert f(bt=4, by=8, bx=8) == 4            # 256-token boxes
    assert f(T=1024, h=256, w=256, bt=2) == 4  # a head of 2^31 bytes or more
    assert f(topk=0) == 3
    assert f(topk=9) == 3                      # 8 boxes
    assert f(v=None) == 1
    assert f(idx=None) == 1
    assert f(out=MIS) == 5
    assert f(lse=FAKE + 2) == 5
    assert f(order=FAKE + 1) == 5
    assert lib.sol_attn_fwd_cube(FAKE, FAKE, FAKE, 1, 1, 4, 16, 16, 2, 8, 8, 2, FAKE, None, float("inf"), FAKE,
                                 None, None) == 2
    assert f(B=0, q=None, idx=None) == 0       # nothing to do
    assert f(T=0, topk=99) == 0
    assert lib.sol_attn_last_error() == b""


def test_quantize_argument_checks(lib):
    q = lambda **kw: lib.sol_attn_quantize(kw.get("x", FAKE), kw.get("B", 1), kw.get("H", 1), kw.get("L", 8),
                                           kw.get("d", 128), kw.get("fmt", 0), kw.get("codes", FAKE),
                                           kw.get("scales", FAKE), None)
    dq = lambda **kw: lib.sol_attn_dequantize(kw.get("codes", FAKE), kw.get("scales", FAKE), 1, 1, 8,
                                              kw.get("d", 128), kw.get("fmt", 1), kw.get("out", FAKE), None)
    assert q(L=-1) == 2 and q(d=0) == 2
    assert q(fmt=2) == 4 and q(d=12) == 4 and q(d=520) == 4
    assert q(x=None) == 1 and q(scales=None) == 1
    assert q(x=MIS) == 5 and q(codes=FAKE + 4) == 5 and q(scales=FAKE + 2) == 5
    assert q(B=0, x=None) == 0
    assert dq(out=MIS) == 5 and dq(codes=None) == 1 and dq(d=7) == 4


def test_check_block_idx_argument_checks(lib):
    chk = lambda idx=FAKE, B=1, H=1, nb=8, k=2, bad=FAKE: lib.sol_attn_check_block_idx(idx, B, H, nb, k, bad, None)
    assert chk(B=-1) == 2 and chk(k=-1) == 2
    assert chk(bad=None) == 1 and chk(idx=None) == 1
    assert chk(bad=FAKE + 2) == 5 and chk(idx=FAKE + 1) == 5


def test_probe_mfma_argument_checks(lib):
    assert lib.sol_attn_probe_mfma(0, 10, FAKE, None) == 2
    assert lib.sol_attn_probe_mfma(4, 0, FAKE, None) == 2
    assert lib.sol_attn_probe_mfma(4, 10, None, None) == 1
    assert lib.sol_attn_probe_mfma(4, 10, FAKE + 2, None) == 5


@pytest.mark.parametrize("lang,std", [("c", "c99"), ("c++", "c++17")])
def test_header_is_plain_c(lang, std, tmp_path):
    """include/sol_attn.h is a C-ABI header: it compiles on its own as C99 and as C++17
    (no torch or HIP types in the signatures), and a C program that includes it links
    against the library and reads its version."""
    import shutil
    import subprocess
    cc = shutil.which("gcc" if lang == "c" else "g++")
    if cc is None:
        pytest.skip("no host compiler")
    inc = os.path.join(os.path.dirname(S.HEADER_PATH))
    src = tmp_path / ("v.c" if lang == "c" else "v.cpp")
    src.write_text('#include "sol_attn.h"\n#include <stdio.h>\n'
                   'int main(void) { printf("%d\\n", sol_attn_version()); return 0; }\n')
    exe = tmp_path / "v"
    subprocess.run([cc, f"-std={std}", "-Wall", "-Werror", "-I", inc, str(src), "-o", str(exe),
                    S.LIB_PATH, f"-Wl,-rpath,{os.path.dirname(S.LIB_PATH)}"], check=True)
    res = subprocess.run([str(exe)], capture_output=True, text=True, timeout=60)
    assert res.returncode == 0 and res.stdout.strip() == str(S.load_library().sol_attn_version())
