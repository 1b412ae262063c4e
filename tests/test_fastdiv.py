"""Host check of the multiply-high division the kernels use for box numbers
(block_sparse_attention_attn_amd/csrc/fastdiv.h): compiled with g++ and compared with
the integer quotient, exhaustively for small operands and at the edges (multiples of d
and their neighbours, up to 2^31 - 1) for large ones."""
import os
import shutil
import subprocess

import pytest

HERE = os.path.dirname(os.path.abspath(__file__))
CSRC = os.path.join(os.path.dirname(HERE), "block_sparse_attention_attn_amd", "csrc")

CHECK = r"""
#include <cstdio>
#include <cstdint>
#include "fastdiv.h"
int main() {
  long long bad = 0, n = 0;
  auto check = [&](uint32_t d, uint32_t c) {
    const sol_attn::FastDiv f(d);
    ++n;
    if (f.div(c) != c / d) { if (bad < 5) printf("d=%u c=%u got %u\n", d, c, f.div(c)); ++bad; }
  };
  for (uint32_t d = 1; d <= 2048; ++d)
    for (uint32_t c = 0; c < 8192; ++c) check(d, c);
  const uint32_t top = 0x7fffffffu;
  uint32_t ds[] = {3, 5, 7, 21, 42, 84, 96, 504, 1000, 4095, 4097, 65535, 65536, 65537, 1000003, 0x40000000u, top};
  for (uint32_t d : ds) {
    for (uint64_t q = 0; q * d <= top; q += (top / d) / 4096 + 1)
      for (int r = -1; r <= 1; ++r) {
        const long long c = (long long)(q * d) + r;
        if (c >= 0 && c <= top) check(d, (uint32_t)c);
      }
    check(d, top);
    check(d, top - 1);
  }
  for (uint32_t k = 0; k < 31; ++k) check(1u << k, top), check((1u << k) + 1, top), check(1u << k, (1u << k) - 1);
  printf("checked %lld bad %lld\n", n, bad);
  return bad != 0;
}
"""


@pytest.mark.skipif(shutil.which("g++") is None, reason="no host C++ compiler")
def test_fastdiv_matches_integer_division(tmp_path):
    src = tmp_path / "check.cpp"
    src.write_text(CHECK)
    exe = tmp_path / "check"
    subprocess.run(["g++", "-O2", "-std=c++17", "-I", CSRC, str(src), "-o", str(exe)], check=True)
    res = subprocess.run([str(exe)], capture_output=True, text=True, timeout=120)
    assert res.returncode == 0, res.stdout + res.stderr
    assert "bad 0" in res.stdout
