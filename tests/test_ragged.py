"""Short last block (block does not divide L) through the whole path on the GPU, against
the float64 oracle: pooled means and selections bit-exact, outputs within the bf16 /
fp32 tolerances, rows past L never written, the short block met at every position of
the attention kernel's buffer rotation (k from 1 to all blocks).  The oracle's reading of a
short block is pinned on the CPU in test_oracle.py."""
import dataclasses
import math

import numpy as np
import pytest
import torch

import oracle
from block_sparse_attention_attn_amd import workloads as W

pytestmark = pytest.mark.gpu

BF16_MAX, BF16_MEAN, FP32_MAX = 2e-2, 2e-3, 1e-5


@pytest.fixture(scope="module")
def S():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    from block_sparse_attention_attn_amd import sol_attn
    sol_attn.load_library()
    return sol_attn


def _bf16_bits(x):
    """float64 -> bf16 bit patterns (round to nearest even), as the workload generator stores them."""
    f = x.astype(np.float32).view(np.uint32).astype(np.uint64)
    return ((f + 0x7FFF + ((f >> 16) & 1)) >> 16).astype(np.uint16)


def _inputs(B, H, L, d, dtype, seed):
    rng = np.random.default_rng(seed)
    xs = [rng.standard_normal((B, H, L, d)) * (1.0 + 0.5 * i) for i in range(3)]
    if dtype == "bf16":
        return [_bf16_bits(x) for x in xs]
    return [x.astype(np.float32) for x in xs]


def _dev(x, dtype):
    x = np.ascontiguousarray(x)
    if dtype == "bf16":
        return torch.from_numpy(x.view(np.int16)).view(torch.bfloat16).cuda()
    return torch.from_numpy(x).cuda()


def _check_whole_path(S, B, H, L, d, block, topk, dtype, seed, order=None):
    q, k, v = _inputs(B, H, L, d, dtype, seed)
    ref = oracle.run(q, k, v, dtype, block, topk)
    Q, K, V = _dev(q, dtype), _dev(k, dtype), _dev(v, dtype)
    qp, kp = S.sol_attn_pool(Q, K, block)
    nb = -(-L // block)
    assert qp.shape == (B, H, nb, d)
    idx = S.sol_attn_select(qp, kp, topk)
    out = torch.full_like(Q, float("nan"))
    S.sol_attn_fwd(Q, K, V, idx, block, out=out, return_lse=False, qblock_order=order)
    _, lse_c = S.sol_attn_fwd(Q, K, V, idx, block, return_lse=True, qblock_order=order)
    torch.cuda.synchronize()
    assert np.array_equal(qp.cpu().numpy(), ref["qbar"])
    assert np.array_equal(kp.cpu().numpy(), ref["kbar"])
    assert np.array_equal(idx.cpu().numpy(), ref["idx"])
    o = out.float().double().cpu().numpy() if dtype == "bf16" else out.double().cpu().numpy()
    assert not np.isnan(o).any()
    err = np.abs(o - ref["out"])
    if dtype == "bf16":
        assert err.max() <= BF16_MAX and err.mean() <= BF16_MEAN, (L, topk, err.max(), err.mean())
    else:
        assert err.max() <= FP32_MAX, (L, topk, err.max())
    assert np.abs(lse_c.double().cpu().numpy() - ref["lse"]).max() <= (1e-2 if dtype == "bf16" else 1e-5)


@pytest.mark.parametrize("L,topk", [(1025, 3), (1087, 4), (1088, 9), (1089, 2), (1151, 9), (1151, 1), (130, 2),
                                    (1025, 5), (1087, 6), (1151, 7), (1089, 8)])
def test_ragged_bf16_small_k(S, L, topk):
    """Short last block of 1, 63, 64, 65 and 127 tokens; odd and even block counts; k = all."""
    _check_whole_path(S, 1, 2, L, 128, 128, topk, "bf16", seed=L + topk)


def test_ragged_bf16_schedule(S):
    L, topk = 1473, 4                                     # 12 blocks, the last with 65 tokens
    order = torch.randperm(12, generator=torch.Generator().manual_seed(3)).to(torch.int32).cuda()
    _check_whole_path(S, 2, 1, L, 128, 128, topk, "bf16", seed=7, order=order)


@pytest.mark.parametrize("L,block,topk", [(1000, 64, 4), (1000, 64, 16), (777, 100, 8), (65, 64, 2)])
def test_ragged_fp32(S, L, block, topk):
    _check_whole_path(S, 1, 2, L, 64, block, topk, "fp32", seed=L)


def test_ragged_bf16_many_blocks(S):
    """k above 128 with a short last block: 130 blocks,
    the last with 50 tokens, all of them selected (dense), checked on sampled blocks."""
    L, d, block = 129 * 128 + 50, 128, 128
    nb = 130
    q, k, v = _inputs(1, 1, L, d, "bf16", 11)
    Q, K, V = _dev(q, "bf16"), _dev(k, "bf16"), _dev(v, "bf16")
    idx = S.sol_attn_select(*S.sol_attn_pool(Q, K, block), nb)
    out = torch.full_like(Q, float("nan"))
    S.sol_attn_fwd(Q, K, V, idx, block, out=out)
    torch.cuda.synchronize()
    assert torch.equal(idx[0, 0, 5].cpu(), torch.arange(nb, dtype=torch.int32))
    assert not torch.isnan(out).any().item()
    Qd, Kd, Vd = (oracle.widen(x, "bf16")[0, 0] for x in (q, k, v))
    o = out.float().double().cpu().numpy()[0, 0]
    for i in (0, 77, nb - 1):
        s = oracle.block_rows(i, L, block)
        Oi, _ = oracle.attend_block(Qd[s], Kd, Vd, np.arange(nb), block, 1.0 / math.sqrt(d))
        e = np.abs(o[s] - Oi)
        assert e.max() <= BF16_MAX and e.mean() <= BF16_MEAN, (i, e.max(), e.mean())


@pytest.mark.timeout(900)
def test_ragged_full_size(S):
    """The 1344x768 workload cut to 64,475 tokens (503 full blocks and one of 91): pooled
    means and every head's selection in full; O and lse of the short block and two
    seeded blocks in every head, each against the oracle's own selection."""
    import concurrent.futures as cf
    import os
    wl = W.get("refine_1344x768")
    q, k, v = (x[..., :wl.L - 37, :] for x in W.make_qkv(wl))
    L = wl.L - 37
    nb = -(-L // wl.block)
    Q, K, V = _dev(q, "bf16"), _dev(k, "bf16"), _dev(v, "bf16")
    order = S.sol_attn_frame_order(L, wl.block, wl.lat_h * wl.lat_w, wl.lat_w).cuda()
    qp, kp = S.sol_attn_pool(Q, K, wl.block)
    idx = S.sol_attn_select(qp, kp, wl.topk)
    out = torch.full_like(Q, float("nan"))
    _, lse = S.sol_attn_fwd(Q, K, V, idx, wl.block, out=out, qblock_order=order, return_lse=True)
    torch.cuda.synchronize()
    Qd, Kd, Vd = (oracle.widen(x, "bf16") for x in (q, k, v))
    qbar, kbar = oracle.pool(Qd, wl.block), oracle.pool(Kd, wl.block)
    assert np.array_equal(qp.cpu().numpy(), qbar) and np.array_equal(kp.cpu().numpy(), kbar)
    BH = wl.B * wl.H
    qf, kf = qbar.reshape(BH, nb, wl.d), kbar.reshape(BH, nb, wl.d)
    with cf.ThreadPoolExecutor(max_workers=min(16, os.cpu_count() or 1)) as ex:
        want = np.stack(list(ex.map(lambda bh: oracle.select(qf[bh], kf[bh], wl.topk), range(BH))))
    assert np.array_equal(idx.cpu().numpy().reshape(BH, nb, wl.topk), want)
    assert not torch.isnan(out).any().item()
    o, ls = out.view(BH, L, wl.d), lse.view(BH, L)
    Qf, Kf, Vf = (x.reshape(BH, L, wl.d) for x in (Qd, Kd, Vd))
    rng = np.random.default_rng(1)
    jobs = [(bh, i) for bh in range(BH) for i in [nb - 1] + list(rng.choice(nb - 1, 2, replace=False))]

    def one(job):
        bh, i = job
        s = oracle.block_rows(i, L, wl.block)
        return job, oracle.attend_block(Qf[bh, s], Kf[bh], Vf[bh], want[bh, i], wl.block, 1.0 / math.sqrt(wl.d))

    with cf.ThreadPoolExecutor(max_workers=min(16, os.cpu_count() or 1)) as ex:
        ref = dict(ex.map(one, jobs))
    errs, lerrs = [], []
    for (bh, i), (Oi, lsei) in ref.items():
        s = oracle.block_rows(i, L, wl.block)
        errs.append(np.abs(o[bh, s].float().double().cpu().numpy() - Oi))
        lerrs.append(np.abs(ls[bh, s].double().cpu().numpy() - lsei))
    err, lerr = np.concatenate(errs), np.concatenate(lerrs)
    assert err.max() <= BF16_MAX and err.mean() <= BF16_MEAN, (err.max(), err.mean())
    assert lerr.max() <= 1e-3, lerr.max()
