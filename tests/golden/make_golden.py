"""Writes the stored regression values under tests/golden/.

* workload_hashes.json -- sha256 of the tiny workload's Q, K, V bytes (generator only);
* tiny_fp32_1k_idx.txt -- the oracle's selected key blocks for the tiny workload at
  k=4, one row per (head, query block).

The pages print no worked example for this path, so nothing here is quoted from
them; expected values come only from the generator and from `oracle/`.
Run: python tests/golden/make_golden.py
"""
import hashlib
import json
import os
import sys

import numpy as np

HERE = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, os.path.dirname(os.path.dirname(HERE)))

import oracle  # noqa: E402
from block_sparse_attention_attn_amd import workloads as W  # noqa: E402


def main():
    wl = W.get("tiny_fp32_1k")
    q, k, v = W.make_qkv(wl)
    hashes = {"tiny_fp32_1k": [hashlib.sha256(np.ascontiguousarray(x).tobytes()).hexdigest()
                               for x in (q, k, v)]}
    with open(os.path.join(HERE, "workload_hashes.json"), "w") as f:
        json.dump(hashes, f, indent=1)
        f.write("\n")
    Q, K = oracle.widen(q, wl.dtype), oracle.widen(k, wl.dtype)
    idx = oracle.select(oracle.pool(Q, wl.block), oracle.pool(K, wl.block), wl.topk)
    with open(os.path.join(HERE, "tiny_fp32_1k_idx.txt"), "w") as f:
        f.write("# oracle selection, tiny_fp32_1k, k=4; row = head*16 + query block\n")
        for row in idx.reshape(-1, wl.topk):
            f.write(" ".join(str(int(x)) for x in row) + "\n")


if __name__ == "__main__":
    main()
