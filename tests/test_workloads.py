"""The seeded input generator: shapes, scaling, rounding and reproducibility."""
import hashlib
import json
import os

import numpy as np
import pytest

from block_sparse_attention_attn_amd import workloads as W

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def test_shapes_match_the_latent_grids():
    expect = {
        "tiny_fp32_1k": (1024, 16, 2, 64),
        "draft_896x512": (28672, 224, 40, 128),
        "refine_1344x768": (64512, 504, 40, 128),
        "clip10s_1344x768": (129024, 1008, 40, 128),
        "refine_2k": (147456, 1152, 40, 128),
    }
    for name, (L, nb, H, d) in expect.items():
        wl = W.get(name)
        assert (wl.L, wl.n_blocks, wl.H, wl.d) == (L, nb, H, d)
        assert wl.L % wl.block == 0
    # pixel sizes / 16
    assert (W.get("draft_896x512").lat_w * 16, W.get("draft_896x512").lat_h * 16) == (896, 512)
    assert (W.get("refine_1344x768").lat_w * 16, W.get("refine_1344x768").lat_h * 16) == (1344, 768)
    assert (W.get("refine_2k").lat_w * 16, W.get("refine_2k").lat_h * 16) == (2048, 1152)
    assert W.get("refine_1344x768").effective_flops() == 4.0 * 40 * 64512 * 76 * 128 * 128


def test_bf16_rounding_is_nearest_even():
    rng = np.random.default_rng(0)
    x = np.concatenate([rng.standard_normal(20000) * 3.0,
                        # exact halfway cases between neighbouring bf16 values
                        (np.arange(128, 256) + 0.5) / 128.0, -(np.arange(128, 256) + 0.5) / 64.0])
    bits = W.f64_to_bf16_bits(x)
    val = W.bf16_bits_to_f32(bits).astype(np.float64)
    up = W.bf16_bits_to_f32(bits + np.uint16(1)).astype(np.float64)
    dn = W.bf16_bits_to_f32(bits - np.uint16(1)).astype(np.float64)
    err = np.abs(x - val)
    assert np.all(err <= np.abs(x - up)) and np.all(err <= np.abs(x - dn))
    tie = (err == np.abs(x - up)) | (err == np.abs(x - dn))
    assert np.any(tie)
    assert np.all((bits[tie] & 1) == 0)          # ties go to the even significand
    assert W.f64_to_bf16_bits(np.array([1.0]))[0] == 0x3F80
    assert W.f64_to_bf16_bits(np.array([-2.0]))[0] == 0xC000


def test_tiny_workload_reproducible_and_hashed():
    wl = W.get("tiny_fp32_1k")
    a = W.make_qkv(wl)
    b = W.make_qkv(wl)
    for x, y in zip(a, b):
        assert x.dtype == np.float32 and x.shape == (1, 2, 1024, 64)
        assert np.array_equal(x, y)
    with open(os.path.join(GOLDEN, "workload_hashes.json")) as f:
        want = json.load(f)
    got = [hashlib.sha256(np.ascontiguousarray(x).tobytes()).hexdigest() for x in a]
    assert got == want["tiny_fp32_1k"]
    # Q, K and V are independent streams
    assert not np.array_equal(a[0], a[1])


@pytest.mark.slow
def test_draft_workload_unit_rms_and_bf16():
    wl = W.get("draft_896x512")
    k = W.make_tensor(wl, 1)
    assert k.dtype == np.uint16 and k.shape == (1, 40, 28672, 128)
    v = W.bf16_bits_to_f32(k).astype(np.float64)
    assert abs(np.sqrt(np.mean(v * v)) - 1.0) < 1e-3
    # smooth field: neighbouring tokens correlate strongly, distant frames much less
    a = v[0, 0, :-1, 0]
    b = v[0, 0, 1:, 0]
    assert np.corrcoef(a, b)[0, 1] > 0.5


def test_cube_boxes_tile_the_grid():
    for wl in W.WORKLOADS.values():
        (T, h, w), (bt, by, bx) = wl.grid, wl.cube
        assert T % bt == 0 and h % by == 0 and w % bx == 0, wl.name
        assert bt * by * bx == wl.block, wl.name
