"""Seeded random sweep of the whole path (pool -> select -> fwd) on the GPU against the
float64 oracle: random batch, heads, sequence length (usually not a multiple of the
block), block count, k, dtype, block size (fp32), softmax scale and query-block
schedule.  Same bar as the other parity tests: pooled means and indices bit-exact,
outputs within the bf16 / fp32 tolerances, log-sum-exp close, rows past L untouched."""
import numpy as np
import pytest
import torch

import oracle

pytestmark = pytest.mark.gpu

BF16_MAX, BF16_MEAN, FP32_MAX = 2e-2, 2e-3, 1e-5


def _bf16_bits(x):
    f = x.astype(np.float32).view(np.uint32).astype(np.uint64)
    return ((f + 0x7FFF + ((f >> 16) & 1)) >> 16).astype(np.uint16)


def _configs(n, seed=2024):
    rng = np.random.default_rng(seed)
    out = []
    for c in range(n):
        dtype = "bf16" if (c % 3 != 2 or c in (5, 11)) else "fp32"
        if dtype == "bf16":
            d, block = 128, 128
        else:
            d = int(rng.choice([64, 128]))
            block = int(rng.choice([16, 32, 50, 64, 128, 256]))
        nb = int(rng.integers(1, 24))
        if c in (5, 11):                       # more than 128 selected blocks: the one-block kernel
            nb = int(rng.integers(131, 140))
        tail = int(rng.integers(1, block + 1)) if rng.random() < 0.7 else block
        L = (nb - 1) * block + tail
        topk = int(rng.integers(1, nb + 1)) if c not in (5, 11) else int(rng.integers(129, nb + 1))
        B, H = (1, 1) if nb > 100 else (int(rng.integers(1, 3)), int(rng.integers(1, 4)))
        scale = None if rng.random() < 0.6 else float(rng.uniform(0.02, 0.3))
        order = rng.random() < 0.5
        out.append((c, dtype, B, H, L, d, block, topk, scale, order))
    return out


@pytest.fixture(scope="module")
def S():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    from block_sparse_attention_attn_amd import sol_attn
    sol_attn.load_library()
    return sol_attn


@pytest.mark.parametrize("cfg", _configs(24), ids=lambda c: f"c{c[0]}-{c[1]}-L{c[4]}-b{c[6]}-k{c[7]}")
def test_random_config_matches_oracle(S, cfg):
    c, dtype, B, H, L, d, block, topk, scale, use_order = cfg
    rng = np.random.default_rng(1000 + c)
    xs = [rng.standard_normal((B, H, L, d)) * s + rng.standard_normal((B, H, 1, d)) * 0.5
          for s in (1.0, 1.3, 0.8)]
    stored = [_bf16_bits(x) for x in xs] if dtype == "bf16" else [x.astype(np.float32) for x in xs]
    q, k, v = stored

    def dev(x):
        x = np.ascontiguousarray(x)
        return (torch.from_numpy(x.view(np.int16)).view(torch.bfloat16) if dtype == "bf16"
                else torch.from_numpy(x)).cuda()

    Q, K, V = dev(q), dev(k), dev(v)
    nb = -(-L // block)
    qp, kp = S.sol_attn_pool(Q, K, block)
    idx = S.sol_attn_select(qp, kp, topk)
    order = None
    if use_order:
        order = torch.from_numpy(rng.permutation(nb).astype(np.int32)).cuda()
    out = torch.full_like(Q, float("nan"))
    _, lse = S.sol_attn_fwd(Q, K, V, idx, block, softmax_scale=scale, return_lse=True, out=out,
                            qblock_order=order)
    torch.cuda.synchronize()

    Qd, Kd, Vd = (oracle.widen(x, dtype) for x in stored)
    qbar, kbar = oracle.pool(Qd, block), oracle.pool(Kd, block)
    assert np.array_equal(qp.cpu().numpy(), qbar) and np.array_equal(kp.cpu().numpy(), kbar)
    want = oracle.select(qbar, kbar, topk)
    assert np.array_equal(idx.cpu().numpy(), want), "selection differs from the oracle"
    O, Ls = oracle.attend(Qd, Kd, Vd, want, block, scale=scale)
    got = out.double().cpu().numpy()
    assert np.isfinite(got).all()
    err = np.abs(got - O)
    lerr = np.abs(lse.double().cpu().numpy() - Ls)
    if dtype == "bf16":
        assert err.max() <= BF16_MAX and err.mean() <= BF16_MEAN, (err.max(), err.mean())
        assert lerr.max() <= 1e-2, lerr.max()
    else:
        assert err.max() <= FP32_MAX, err.max()
        assert lerr.max() <= 1e-4, lerr.max()
