"""On-disk cache of oracle results for the large workloads (test infrastructure).

The oracle's pooled means, selected indices and sampled attention rows of a
full-size workload take minutes of CPU time; with a cache directory named in
SOL_ATTN_CACHE_DIR (unset or empty: no cache) they are stored once and read back
on later runs.  A result is keyed by
  * the generated inputs' key (every workload field and the generator version),
  * a hash of the oracle's source files, so any change to its arithmetic starts afresh,
  * the kind of result and its parameters (top-k, sampled blocks, ...).
Files are plain .npz archives read with allow_pickle=False; each also records the
seconds the oracle took, in the array "oracle_seconds".
"""
import glob
import hashlib
import json
import os
import time

import numpy as np

import oracle
from block_sparse_attention_attn_amd import workloads as W


def oracle_source_hash() -> str:
    h = hashlib.sha256()
    for path in sorted(glob.glob(os.path.join(os.path.dirname(oracle.__file__), "*.py"))):
        h.update(os.path.basename(path).encode())
        with open(path, "rb") as f:
            h.update(f.read())
    return h.hexdigest()[:16]


def result_key(wl, kind: str, params) -> str:
    blob = json.dumps({"inputs": W.input_key(wl), "oracle": oracle_source_hash(), "kind": kind,
                       "params": params}, sort_keys=True, separators=(",", ":"))
    return hashlib.sha256(blob.encode()).hexdigest()[:24]


def cached(wl, kind: str, params, compute, cache_dir=None):
    """compute() -> {name: ndarray}; returned from the cache when an entry with this key exists.

    Returns (arrays, hit)."""
    cache_dir = cache_dir or W.cache_dir_from_env()
    if cache_dir is None:
        return compute(), False
    sub = os.path.join(cache_dir, "oracle")
    os.makedirs(sub, exist_ok=True)
    path = os.path.join(sub, f"{kind}_{result_key(wl, kind, params)}.npz")
    if os.path.exists(path):
        try:
            with np.load(path, allow_pickle=False) as z:
                res = {name: z[name] for name in z.files if name != "oracle_seconds"}
            return res, True
        except (OSError, ValueError, KeyError):
            pass
    t0 = time.perf_counter()
    res = compute()
    seconds = time.perf_counter() - t0
    tmp = f"{path}.{os.getpid()}.tmp"
    with open(tmp, "wb") as f:
        np.savez(f, oracle_seconds=np.float64(seconds), **res)
    os.replace(tmp, path)
    return res, False
