"""CPU oracle for the Sol-Attn block-sparse attention path -- TEST INFRASTRUCTURE ONLY.

Plain, slow, float64 numpy code that computes what the sparse-attention path
computes, written from the definition, so the HIP path can be checked against it.
Only the tests, the smoke check and the benchmark's CPU-baseline leg may import
it; the library's compute path never does, and the two share no code.
"""
from .sol_attn_oracle import (  # noqa: F401
    widen, n_blocks, block_rows, pool, block_scores, select, select_from_scores, attend, attend_block,
    selection_margins, run, window_selection, cube_blocks, pool_sets, attend_sets, run_cube,
)
from . import quant_oracle  # noqa: F401,E402
