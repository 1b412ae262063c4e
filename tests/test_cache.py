"""The input and oracle-result caches: a hit returns exactly what was stored, and any
change to the workload, the generator version, the oracle's sources or the result's
parameters is a miss."""
import dataclasses
import os

import numpy as np
import pytest

import oracle
import oracle_cache
from block_sparse_attention_attn_amd import workloads as W

TINY = W.get("tiny_fp32_1k")
SMALL_BF16 = dataclasses.replace(W.get("draft_896x512"), name="cache_small", H=2, frames=1, lat_h=8, lat_w=32,
                                 coarse=(1, 2, 2), topk=2, seed=21)


@pytest.fixture(autouse=True)
def no_env_cache(monkeypatch):
    monkeypatch.delenv("SOL_ATTN_CACHE_DIR", raising=False)


def count_generation(monkeypatch):
    calls = []
    real = W.make_tensor

    def counted(wl, which, heads=None):
        calls.append(which)
        return real(wl, which, heads)

    monkeypatch.setattr(W, "make_tensor", counted)
    return calls


@pytest.mark.parametrize("wl", [TINY, SMALL_BF16], ids=["fp32", "bf16"])
def test_input_cache_hit_returns_the_generated_bits(tmp_path, monkeypatch, wl):
    plain = W.make_qkv(wl)
    calls = count_generation(monkeypatch)
    first = W.make_qkv(wl, cache_dir=str(tmp_path))
    assert calls == [0, 1, 2]
    second = W.make_qkv(wl, cache_dir=str(tmp_path))
    assert calls == [0, 1, 2]                       # nothing generated on the second call
    for a, b, c in zip(plain, first, second):
        assert a.dtype == b.dtype == c.dtype and a.shape == b.shape == c.shape
        assert np.array_equal(a.view(np.uint8), c.view(np.uint8))
        assert np.array_equal(b.view(np.uint8), c.view(np.uint8))
    assert len(os.listdir(tmp_path / "inputs")) == 3


def test_input_cache_from_environment(tmp_path, monkeypatch):
    monkeypatch.setenv("SOL_ATTN_CACHE_DIR", str(tmp_path))
    W.make_qkv(TINY)
    key = W.input_key(TINY)
    assert sorted(os.listdir(tmp_path / "inputs")) == [f"{key}_{t}.npy" for t in "kqv"]


def test_no_cache_dir_writes_nothing(tmp_path, monkeypatch):
    monkeypatch.chdir(tmp_path)
    W.make_qkv(TINY)
    assert os.listdir(tmp_path) == []


def test_input_key_changes_with_every_field_and_the_generator_version(monkeypatch):
    base = W.input_key(TINY)
    assert W.input_key(dataclasses.replace(TINY)) == base
    for field, value in [("seed", 1), ("H", 3), ("coarse", (2, 4, 2)), ("topk", 5), ("dtype", "bf16"),
                         ("cube", (1, 8, 8)), ("name", "other")]:
        assert W.input_key(dataclasses.replace(TINY, **{field: value})) != base, field
    monkeypatch.setattr(W, "GENERATOR_VERSION", W.GENERATOR_VERSION + 1)
    assert W.input_key(TINY) != base


def test_generator_version_bump_regenerates(tmp_path, monkeypatch):
    W.make_qkv(TINY, cache_dir=str(tmp_path))
    monkeypatch.setattr(W, "GENERATOR_VERSION", W.GENERATOR_VERSION + 1)
    calls = count_generation(monkeypatch)
    W.make_qkv(TINY, cache_dir=str(tmp_path))
    assert calls == [0, 1, 2]
    assert len(os.listdir(tmp_path / "inputs")) == 6


def test_damaged_cache_file_is_regenerated(tmp_path, monkeypatch):
    q, _, _ = W.make_qkv(TINY, cache_dir=str(tmp_path))
    path = tmp_path / "inputs" / f"{W.input_key(TINY)}_q.npy"
    np.save(path, np.zeros((3, 3), dtype=np.float32))      # wrong shape
    calls = count_generation(monkeypatch)
    q2, _, _ = W.make_qkv(TINY, cache_dir=str(tmp_path))
    assert calls == [0]
    assert np.array_equal(q, q2)
    path.write_bytes(b"not an npy file")
    q3, _, _ = W.make_qkv(TINY, cache_dir=str(tmp_path))
    assert calls == [0, 0] and np.array_equal(q, q3)


def test_oracle_cache_round_trip_and_misses(tmp_path, monkeypatch):
    q, k, v = W.make_qkv(TINY)
    runs = []

    def compute():
        runs.append(1)
        ref = oracle.run(q, k, v, "fp32", TINY.block, TINY.topk)
        return {name: ref[name] for name in ("qbar", "kbar", "idx", "out", "lse")}

    a, hit_a = oracle_cache.cached(TINY, "run", {"topk": TINY.topk}, compute, cache_dir=str(tmp_path))
    b, hit_b = oracle_cache.cached(TINY, "run", {"topk": TINY.topk}, compute, cache_dir=str(tmp_path))
    assert (hit_a, hit_b, len(runs)) == (False, True, 1)
    assert set(a) == set(b)
    for name in a:
        assert a[name].dtype == b[name].dtype and np.array_equal(a[name], b[name]), name
    # the stored file also holds the oracle's time
    (path,) = list((tmp_path / "oracle").iterdir())
    with np.load(path, allow_pickle=False) as z:
        assert float(z["oracle_seconds"]) > 0.0
    # other parameters, another workload, changed oracle sources: all misses
    oracle_cache.cached(TINY, "run", {"topk": 16}, compute, cache_dir=str(tmp_path))
    assert len(runs) == 2
    oracle_cache.cached(dataclasses.replace(TINY, seed=5), "run", {"topk": TINY.topk}, compute,
                        cache_dir=str(tmp_path))
    assert len(runs) == 3
    monkeypatch.setattr(oracle_cache, "oracle_source_hash", lambda: "edited")
    oracle_cache.cached(TINY, "run", {"topk": TINY.topk}, compute, cache_dir=str(tmp_path))
    assert len(runs) == 4


def test_oracle_cache_off_without_a_directory():
    runs = []
    res, hit = oracle_cache.cached(TINY, "x", {}, lambda: runs.append(1) or {"a": np.ones(2)})
    assert not hit and runs == [1] and np.array_equal(res["a"], np.ones(2))


def test_oracle_source_hash_covers_every_oracle_file():
    import glob
    files = glob.glob(os.path.join(os.path.dirname(oracle.__file__), "*.py"))
    assert {os.path.basename(f) for f in files} >= {"sol_attn_oracle.py", "quant_oracle.py", "__init__.py"}
    assert len(oracle_cache.oracle_source_hash()) == 16
