"""Sol-Attn block-sparse attention for MI355X (gfx950).

The compute path is the C-ABI library ``libsol_attn.so`` (hand-written HIP
kernels); :mod:`block_sparse_attention_attn_amd.sol_attn` is its thin Python
binding.  Importing this package does not load the library; the binding does,
on first use, and raises if it is missing.
"""
__version__ = "0.1.0"
