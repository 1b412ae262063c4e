"""Parity of the HIP path (through the C ABI) with the float64 CPU oracle.

Bar: pooled means and selected block indices bit-exact; outputs within
max|err| <= 2e-2 and mean|err| <= 2e-3 (absolute, vs the float64 oracle) for bf16
inputs, and max|err| <= 1e-5 for fp32 inputs.  The full-size workloads run in the
launch configuration the benchmark times and are checked on sampled query blocks
(every pooled value and every index is checked in full).
"""
import concurrent.futures as cf
import dataclasses
import hashlib
import math
import os

import numpy as np
import pytest
import torch

import oracle
from block_sparse_attention_attn_amd import workloads as W
from oracle_cache import cached

pytestmark = pytest.mark.gpu

BF16_MAX, BF16_MEAN, FP32_MAX = 2e-2, 2e-3, 1e-5
GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


@pytest.fixture(scope="module")
def S():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    from block_sparse_attention_attn_amd import sol_attn
    sol_attn.load_library()
    return sol_attn


def dev(stored, dtype):
    x = np.ascontiguousarray(stored)
    if dtype == "bf16":
        return torch.from_numpy(x.view(np.int16)).view(torch.bfloat16).cuda()
    return torch.from_numpy(x).cuda()


def host_f64(t):
    return t.float().double().cpu().numpy() if t.dtype == torch.bfloat16 else t.double().cpu().numpy()


def log(msg):
    print(msg, flush=True)


def oracle_select_parallel(qbar, kbar, topk):
    """Oracle selection head by head on a thread pool (same arithmetic, just parallel)."""
    B, H, nb, d = qbar.shape
    qf, kf = qbar.reshape(B * H, nb, d), kbar.reshape(B * H, nb, d)
    with cf.ThreadPoolExecutor(max_workers=min(16, os.cpu_count() or 1)) as ex:
        parts = list(ex.map(lambda i: oracle.select(qf[i], kf[i], topk), range(B * H)))
    return np.stack(parts).reshape(B, H, nb, topk)


# ----------------------------------------------------------------------------- tiny fp32
@pytest.mark.parametrize("topk", [4, 16])
def test_tiny_fp32_matches_oracle(S, topk):
    wl = W.get("tiny_fp32_1k")
    log(f"tiny fp32 topk={topk}")
    q, k, v = W.make_qkv(wl)
    ref = oracle.run(q, k, v, "fp32", wl.block, topk)
    Q, K, V = dev(q, "fp32"), dev(k, "fp32"), dev(v, "fp32")
    qp, kp = S.sol_attn_pool(Q, K, wl.block)
    idx = S.sol_attn_select(qp, kp, topk)
    out, lse = S.sol_attn_fwd(Q, K, V, idx, wl.block, return_lse=True)
    torch.cuda.synchronize()
    assert np.array_equal(qp.cpu().numpy(), ref["qbar"])
    assert np.array_equal(kp.cpu().numpy(), ref["kbar"])
    assert np.array_equal(idx.cpu().numpy(), ref["idx"])
    if topk == 4:
        gold = np.loadtxt(os.path.join(GOLDEN, "tiny_fp32_1k_idx.txt"), dtype=np.int32)
        assert np.array_equal(idx.cpu().numpy().reshape(-1, 4), gold)
    else:
        assert np.array_equal(idx.cpu().numpy()[0, 0, 0], np.arange(16))
    err = np.abs(out.cpu().numpy().astype(np.float64) - ref["out"])
    assert err.max() <= FP32_MAX, err.max()
    assert np.abs(lse.cpu().numpy() - ref["lse"]).max() <= FP32_MAX


# ----------------------------------------------------------------------------- small bf16
SMALL = [
    # (B, H, frames, lat_h, lat_w, topk): L = frames*lat_h*lat_w, a multiple of 128
    (1, 1, 1, 8, 16, 1),      # one block, k = 1
    (2, 3, 2, 8, 104, 5),     # 13 blocks: ragged against the 8-way work split
    (1, 2, 3, 16, 24, 9),     # 9 blocks, k = n_blocks (dense)
    (1, 1, 4, 16, 34, 6),     # 17 blocks, odd k
    (1, 2, 2, 32, 40, 2),     # 20 blocks, k = 2 (tail of the 2-step loop)
]


@pytest.mark.parametrize("B,H,T,h,w,topk", SMALL)
def test_small_bf16_matches_oracle(S, B, H, T, h, w, topk):
    wl = dataclasses.replace(W.get("draft_896x512"), name="small", B=B, H=H, frames=T, lat_h=h, lat_w=w,
                             topk=topk, coarse=(1, 2, 3), seed=100 + topk)
    log(f"small bf16 {B}x{H}x{wl.L} k={topk}")
    q, k, v = W.make_qkv(wl)
    ref = oracle.run(q, k, v, "bf16", 128, topk)
    Q, K, V = dev(q, "bf16"), dev(k, "bf16"), dev(v, "bf16")
    qp, kp = S.sol_attn_pool(Q, K, 128)
    idx = S.sol_attn_select(qp, kp, topk)
    out = torch.full_like(Q, float("nan"))
    _, lse = S.sol_attn_fwd(Q, K, V, idx, 128, return_lse=True, out=out)
    torch.cuda.synchronize()
    assert np.array_equal(qp.cpu().numpy(), ref["qbar"])
    assert np.array_equal(kp.cpu().numpy(), ref["kbar"])
    assert np.array_equal(idx.cpu().numpy(), ref["idx"])
    o = host_f64(out)
    assert not np.isnan(o).any()
    err = np.abs(o - ref["out"])
    assert err.max() <= BF16_MAX and err.mean() <= BF16_MEAN, (err.max(), err.mean())
    assert np.abs(lse.cpu().numpy() - ref["lse"]).max() <= 1e-3


def test_bf16_custom_scale_and_given_indices(S):
    """fwd honours softmax_scale and an arbitrary (unsorted, non-top-k) index list."""
    wl = dataclasses.replace(W.get("draft_896x512"), name="s", H=2, frames=1, lat_h=8, lat_w=96, coarse=(1, 2, 3),
                             seed=7)
    q, k, v = W.make_qkv(wl)
    nb = wl.L // 128
    rng = np.random.default_rng(3)
    sel = np.stack([np.stack([rng.permutation(nb)[:3] for _ in range(nb)]) for _ in range(2)])[None].astype(np.int32)
    Qd, Kd, Vd = (oracle.widen(x, "bf16") for x in (q, k, v))
    O, lse = oracle.attend(Qd, Kd, Vd, sel, 128, scale=0.05)
    out, glse = S.sol_attn_fwd(dev(q, "bf16"), dev(k, "bf16"), dev(v, "bf16"), torch.from_numpy(sel).cuda(), 128,
                               softmax_scale=0.05, return_lse=True)
    err = np.abs(host_f64(out) - O)
    assert err.max() <= BF16_MAX and err.mean() <= BF16_MEAN
    assert np.abs(glse.cpu().numpy() - lse).max() <= 1e-3


# ----------------------------------------------------------------------------- selection
def test_select_exact_ties_prefer_lower_index(S):
    # small-integer pooled values: every score is exact, duplicates tie exactly
    rng = np.random.default_rng(5)
    nb, d = 70, 16
    qb = rng.integers(-3, 4, size=(1, 2, nb, d)).astype(np.float64)
    kb = rng.integers(-3, 4, size=(1, 2, nb, d)).astype(np.float64)
    kb[..., 40, :] = kb[..., 3, :]
    kb[..., 41, :] = kb[..., 3, :]
    kb[..., 69, :] = kb[..., 0, :]
    for topk in (1, 7, 33, 70):
        want = oracle.select(qb, kb, topk)
        got = S.sol_attn_select(torch.from_numpy(qb).cuda(), torch.from_numpy(kb).cuda(), topk).cpu().numpy()
        assert np.array_equal(got, want), topk
    # all-equal scores: the first k blocks win
    z = np.zeros((1, 1, 50, 8))
    got = S.sol_attn_select(torch.from_numpy(z).cuda(), torch.from_numpy(z).cuda(), 11).cpu().numpy()
    assert np.array_equal(got[0, 0], np.tile(np.arange(11), (50, 1)))


def test_select_scores_output(S):
    rng = np.random.default_rng(6)
    qb = rng.standard_normal((2, 1, 33, 128))
    kb = rng.standard_normal((2, 1, 33, 128))
    idx, sc = S.sol_attn_select(torch.from_numpy(qb).cuda(), torch.from_numpy(kb).cuda(), 5, return_scores=True)
    r = oracle.block_scores(qb, kb) / math.sqrt(128)
    np.testing.assert_allclose(sc.cpu().numpy(), r, rtol=1e-13, atol=1e-13)
    assert np.array_equal(idx.cpu().numpy(), oracle.select(qb, kb, 5))


@pytest.mark.parametrize("nb,d", [(3000, 128), (700, 64), (129, 8)])
def test_select_many_blocks(S, nb, d):
    """Row counts that shrink the per-workgroup row group and ragged lane ranges."""
    rng = np.random.default_rng(nb)
    qb = rng.standard_normal((1, 2, nb, d))
    kb = rng.standard_normal((1, 2, nb, d))
    for topk in (1, nb // 7 + 1, nb):
        want = oracle_select_parallel(qb, kb, topk)
        got = S.sol_attn_select(torch.from_numpy(qb).cuda(), torch.from_numpy(kb).cuda(), topk).cpu().numpy()
        assert np.array_equal(got, want), topk


def test_selection_invariant_under_within_block_permutation(S):
    wl = dataclasses.replace(W.get("draft_896x512"), name="p", H=2, frames=2, lat_h=16, lat_w=64, coarse=(1, 2, 4),
                             topk=4, seed=9)
    q, k, _ = W.make_qkv(wl)[:3]
    Q, K = dev(q, "bf16"), dev(k, "bf16")
    base = S.sol_attn_select(*S.sol_attn_pool(Q, K, 128), 4).cpu().numpy()
    rng = np.random.default_rng(2)
    perm = np.concatenate([i * 128 + rng.permutation(128) for i in range(wl.L // 128)])
    Kp = dev(np.ascontiguousarray(k[..., perm, :]), "bf16")
    assert np.array_equal(S.sol_attn_select(*S.sol_attn_pool(Q, Kp, 128), 4).cpu().numpy(), base)


@pytest.mark.parametrize("dtype", ["bf16", "fp32"])
def test_schedule_order(S, dtype):
    """The query-block schedule changes only which blocks run together (and, for bf16,
    which two blocks share their common key tiles): any permutation gives bit-identical
    outputs, and every schedule matches the oracle."""
    base = W.get("draft_896x512") if dtype == "bf16" else W.get("tiny_fp32_1k")
    wl = dataclasses.replace(base, name="ord", H=2, frames=4, lat_h=8, lat_w=48 if dtype == "bf16" else 16,
                             coarse=(2, 2, 3), topk=3, seed=13)
    q, k, v = W.make_qkv(wl)
    Q, K, V = dev(q, dtype), dev(k, dtype), dev(v, dtype)
    idx = S.sol_attn_select(*S.sol_attn_pool(Q, K, wl.block), 3)
    nb = wl.L // wl.block
    ref = oracle.run(q, k, v, dtype, wl.block, 3)
    assert np.array_equal(idx.cpu().numpy(), ref["idx"])
    a = S.sol_attn_fwd(Q, K, V, idx, wl.block)
    for order in (None, S.sol_attn_frame_order(wl.L, wl.block, wl.lat_h * wl.lat_w, wl.lat_w),
                  torch.randperm(nb, generator=torch.Generator().manual_seed(1)).to(torch.int32)):
        b, lse = S.sol_attn_fwd(Q, K, V, idx, wl.block, qblock_order=None if order is None else order.cuda(),
                                return_lse=True)
        torch.cuda.synchronize()
        err = np.abs(host_f64(b) - ref["out"])
        lerr = np.abs(lse.double().cpu().numpy() - ref["lse"])
        if dtype == "fp32":
            assert torch.equal(a, b)
            assert err.max() <= FP32_MAX
        else:
            assert torch.equal(a.view(torch.int16), b.view(torch.int16))
            assert err.max() <= BF16_MAX and err.mean() <= BF16_MEAN, (err.max(), err.mean())
            assert lerr.max() <= 1e-2, lerr.max()


def test_fwd_deterministic(S):
    wl = dataclasses.replace(W.get("draft_896x512"), name="det", H=3, frames=2, lat_h=16, lat_w=64, coarse=(1, 2, 4),
                             topk=3, seed=11)
    Q, K, V = (dev(x, "bf16") for x in W.make_qkv(wl))
    idx = S.sol_attn_select(*S.sol_attn_pool(Q, K, 128), 3)
    a = S.sol_attn_fwd(Q, K, V, idx, 128)
    b = S.sol_attn_fwd(Q, K, V, idx, 128)
    assert torch.equal(a.view(torch.int16), b.view(torch.int16))


# ----------------------------------------------------------------------------- full size
FULL = ["draft_896x512", "refine_1344x768", "clip10s_1344x768", "refine_2k"]


def sample_blocks(nb, order, rng, extra=1):
    """Query blocks checked in every head: the first and last block, the two blocks on
    either side of the first boundary between XCD work ranges in the launch schedule
    (position per_xcd - 1 and per_xcd of `order`), and `extra` seeded random ones."""
    per_xcd = -(-nb // 8)
    picks = {0, nb - 1}
    if per_xcd < nb:
        picks |= {int(order[per_xcd - 1]), int(order[per_xcd])}
    picks |= {int(i) for i in rng.choice(nb, extra, replace=False)}
    return sorted(picks)


def sampled_attention(Qd, Kd, Vd, sel, block, picks_per_head):
    """Oracle O and lse of the given query blocks of every head (a thread pool over
    blocks; numpy releases the GIL in matmul and exp).  Returns {(bh, i): (O_i, lse_i)}."""
    BH, L, d = Qd.shape
    jobs = [(bh, i) for bh in range(BH) for i in picks_per_head[bh]]

    def one(job):
        bh, i = job
        s = oracle.block_rows(i, L, block)
        return job, oracle.attend_block(Qd[bh, s], Kd[bh], Vd[bh], sel[bh, i], block, 1.0 / math.sqrt(d))

    with cf.ThreadPoolExecutor(max_workers=min(16, os.cpu_count() or 1)) as ex:
        return dict(ex.map(one, jobs))


def cached_sampled_attention(wl, kind, Qf, Kf, Vf, sel, picks_per_head):
    """sampled_attention through the oracle-result cache (keyed by the workload, the
    selection's hash and the sampled blocks)."""
    params = {"sel": hashlib.sha256(np.ascontiguousarray(sel).tobytes()).hexdigest()[:16],
              "picks": [list(map(int, p)) for p in picks_per_head]}

    def compute():
        ref = sampled_attention(Qf, Kf, Vf, sel, wl.block, picks_per_head)
        arrays = {}
        for (bh, i), (Oi, lsei) in ref.items():
            arrays[f"O_{bh}_{i}"], arrays[f"lse_{bh}_{i}"] = Oi, lsei
        return arrays

    arrays, hit = cached(wl, kind, params, compute)
    if hit:
        log(f"{kind}: oracle rows from the cache")
    return {(bh, i): (arrays[f"O_{bh}_{i}"], arrays[f"lse_{bh}_{i}"])
            for bh, p in enumerate(picks_per_head) for i in p}


def check_sampled(out, lse, ref, L, block, what):
    o = out.view(-1, L, out.shape[-1])
    ls = lse.view(-1, L)
    errs, lerrs = [], []
    for (bh, i), (Oi, lsei) in ref.items():
        s = oracle.block_rows(i, L, block)
        errs.append(np.abs(host_f64(o[bh, s]) - Oi))
        lerrs.append(np.abs(ls[bh, s].double().cpu().numpy() - lsei))
    err, lerr = np.concatenate(errs), np.concatenate(lerrs)
    log(f"{what}: {len(ref)} query blocks, max|err| {err.max():.3e} mean|err| {err.mean():.3e} "
        f"max|lse err| {lerr.max():.3e}")
    assert err.max() <= BF16_MAX and err.mean() <= BF16_MEAN, (what, err.max(), err.mean())
    assert lerr.max() <= 1e-3, (what, lerr.max())


@pytest.mark.timeout(900)
@pytest.mark.parametrize("name", FULL)
def test_full_size_workload(S, name):
    """Full-size workload in the launch configuration the benchmark times: pooled means
    and every selected index bit-exact; every output row written; O and lse of four or
    more query blocks in every head against the oracle; a second launch bit-identical
    to the first (the kernel's waits and barriers leave no race)."""
    wl = W.get(name)
    log(f"full {name}: generating")
    q, k, v = W.make_qkv(wl)
    Q, K, V = dev(q, "bf16"), dev(k, "bf16"), dev(v, "bf16")
    log(f"full {name}: gpu pool/select/fwd")
    order = S.sol_attn_frame_order(wl.L, wl.block, wl.lat_h * wl.lat_w, wl.lat_w)
    order_d = order.cuda()
    qp, kp = S.sol_attn_pool(Q, K, wl.block)
    idx = S.sol_attn_select(qp, kp, wl.topk)
    out = torch.full_like(Q, float("nan"))
    lse = torch.full(Q.shape[:3], float("nan"), dtype=torch.float32, device="cuda")
    S.sol_attn_fwd(Q, K, V, idx, wl.block, out=out, lse=lse, qblock_order=order_d)
    torch.cuda.synchronize()
    log(f"full {name}: second launch (race check)")
    out2 = torch.full_like(Q, float("nan"))
    lse2 = torch.full_like(lse, float("nan"))
    S.sol_attn_fwd(Q, K, V, idx, wl.block, out=out2, lse=lse2, qblock_order=order_d)
    torch.cuda.synchronize()
    assert torch.equal(out.view(torch.int16), out2.view(torch.int16))
    assert torch.equal(lse.view(torch.int32), lse2.view(torch.int32))
    del out2, lse2
    log(f"full {name}: oracle pool/select")
    Qd = oracle.widen(q, "bf16")
    Kd = oracle.widen(k, "bf16")

    def pool_select():
        qbar, kbar = oracle.pool(Qd, wl.block), oracle.pool(Kd, wl.block)
        return {"qbar": qbar, "kbar": kbar, "idx": oracle_select_parallel(qbar, kbar, wl.topk)}

    ps, hit = cached(wl, "pool_select", {"topk": wl.topk}, pool_select)
    if hit:
        log(f"full {name}: oracle pool/select from the cache")
    assert np.array_equal(qp.cpu().numpy(), ps["qbar"])
    assert np.array_equal(kp.cpu().numpy(), ps["kbar"])
    want = ps["idx"]
    got = idx.cpu().numpy()
    assert np.array_equal(got, want)
    # every output row written, finite
    assert not torch.isnan(out).any().item() and not torch.isnan(lse).any().item()
    log(f"full {name}: sampled attention")
    Vd = oracle.widen(v, "bf16")
    BH, nb = wl.B * wl.H, wl.n_blocks
    Qf, Kf, Vf = (x.reshape(BH, wl.L, wl.d) for x in (Qd, Kd, Vd))
    rng = np.random.default_rng(wl.seed)
    picks = [sample_blocks(nb, order, rng) for _ in range(BH)]
    ref = cached_sampled_attention(wl, "sampled", Qf, Kf, Vf, want.reshape(BH, nb, wl.topk), picks)
    check_sampled(out, lse, ref, wl.L, wl.block, f"full {name}")
    if name == "refine_2k":
        # the dense (k = all blocks) run, into freshly NaN-filled outputs
        log("full refine_2k: dense k=1152")
        kd = nb
        idx_d = S.sol_attn_select(qp, kp, kd)
        assert torch.equal(idx_d.cpu(), torch.arange(kd, dtype=torch.int32).expand(wl.B, wl.H, kd, kd))
        out.fill_(float("nan"))
        lse.fill_(float("nan"))
        S.sol_attn_fwd(Q, K, V, idx_d, wl.block, out=out, lse=lse, qblock_order=order_d)
        torch.cuda.synchronize()
        assert not torch.isnan(out).any().item() and not torch.isnan(lse).any().item()
        del idx_d
        dense = np.broadcast_to(np.arange(kd, dtype=np.int32), (BH, nb, kd))
        rng = np.random.default_rng(44)
        picks = [sample_blocks(nb, order, rng, extra=0) for _ in range(BH)]
        ref = cached_sampled_attention(wl, "sampled_dense", Qf, Kf, Vf, dense, picks)
        check_sampled(out, lse, ref, wl.L, wl.block, "full refine_2k dense")


def test_binding_refuses_host_index_lists(S):
    """An index list (or output) on the host with Q/K/V on the device is refused before any
    launch: the kernels would otherwise dereference a host pointer."""
    wl = dataclasses.replace(W.get("draft_896x512"), name="hostidx", H=1, frames=1, lat_h=8, lat_w=32,
                             coarse=(1, 2, 2), topk=2, seed=5)
    q, k, v = W.make_qkv(wl)
    Q, K, V = dev(q, "bf16"), dev(k, "bf16"), dev(v, "bf16")
    idx = S.sol_attn_select(*S.sol_attn_pool(Q, K, 128), 2)
    with pytest.raises(ValueError, match="block_idx"):
        S.sol_attn_fwd(Q, K, V, idx.cpu(), 128)
    with pytest.raises(ValueError, match="lse"):
        S.sol_attn_fwd(Q, K, V, idx, 128, lse=torch.empty(1, 1, wl.L))
    with pytest.raises(ValueError, match="block_idx"):
        S.sol_attn_fwd_cube(Q, K, V, idx.cpu(), wl.grid, (1, 4, 32))
    qp, kp = S.sol_attn_pool(Q, K, 128)
    with pytest.raises(ValueError, match="k_pooled"):
        S.sol_attn_select(qp, kp.cpu(), 2)
    torch.cuda.synchronize()
    out = S.sol_attn_fwd(Q, K, V, idx, 128)          # the same call with device tensors runs
    torch.cuda.synchronize()
    assert not torch.isnan(out).any().item()
