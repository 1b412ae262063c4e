"""Host check of the box addressing that the in-place cube kernels use
(block_sparse_attention_attn_amd/csrc/launchers.h, BoxGeom): compiled for the host and
compared with the oracle's cube token sets -- box c, row r is token
first_token(c) + row_offset(r) -- on grids with ragged and power-of-two box counts."""
import os
import shutil
import subprocess

import numpy as np
import pytest

import oracle

HERE = os.path.dirname(os.path.abspath(__file__))
CSRC = os.path.join(os.path.dirname(HERE), "block_sparse_attention_attn_amd", "csrc")

PROG = r"""
#include <cstdio>
#include <cstdlib>
#include "launchers.h"
int main(int argc, char** argv) {
  const int T = atoi(argv[1]), h = atoi(argv[2]), w = atoi(argv[3]);
  const int bt = atoi(argv[4]), by = atoi(argv[5]), bx = atoi(argv[6]);
  const sol_attn::BoxGeom g = sol_attn::make_box_geom(h, w, bt, by, bx);
  const int boxes = (T / bt) * (h / by) * (w / bx), V = bt * by * bx;
  for (int c = 0; c < boxes; ++c)
    for (int r = 0; r < V; ++r) printf("%d\n", g.first_token(c) + g.row_offset(r));
  return 0;
}
"""

CASES = [((16, 48, 84), (4, 8, 4)), ((4, 16, 16), (2, 8, 8)), ((4, 6, 10), (2, 3, 5)), ((6, 9, 21), (3, 3, 7)),
         ((2, 8, 128), (1, 1, 128)), ((3, 5, 7), (1, 1, 1))]


@pytest.fixture(scope="module")
def prog(tmp_path_factory):
    hipcc = next((c for c in (os.environ.get("HIPCC"), "/opt/rocm/bin/hipcc", shutil.which("hipcc"))
                  if c and os.path.exists(c)), None)
    if hipcc is None:
        pytest.skip("hipcc not available")
    d = tmp_path_factory.mktemp("boxgeom")
    src, exe = d / "g.cpp", d / "g"
    src.write_text(PROG)
    subprocess.run([hipcc, "-std=c++17", "-O1", "-x", "hip", "--offload-arch=gfx950", "-I", CSRC, str(src), "-o",
                    str(exe)], check=True, capture_output=True)
    return str(exe)


@pytest.mark.parametrize("grid,cube", CASES)
def test_box_addressing_matches_oracle_sets(prog, grid, cube):
    out = subprocess.run([prog, *map(str, grid), *map(str, cube)], check=True, capture_output=True,
                         text=True, timeout=120).stdout
    got = np.array(out.split(), dtype=np.int64).reshape(-1, int(np.prod(cube)))
    assert np.array_equal(got, oracle.cube_blocks(*grid, cube))
