"""Static window pattern (the decoder's windowed attention as a fixed key-block list,
Sol-H3-VAE model card, opening paragraph) through the same sparse-attention path.

CPU: the oracle's window (a search over all window starts) is pinned to the properties
that define it, and the library's host helper (a closed form) must equal it.  GPU
(marked): sol_attn_fwd with the pattern against the oracle's attention with the same
key blocks."""
import math

import numpy as np
import pytest
import torch

import oracle
from block_sparse_attention_attn_amd import sol_attn as S
from block_sparse_attention_attn_amd import workloads as W


def test_oracle_window_properties():
    for nb in range(1, 30):
        for k in range(1, nb + 1):
            w = oracle.window_selection(nb, k)
            assert w.shape == (nb, k)
            for i in range(nb):
                row = w[i]
                assert i in row                                    # the query block itself
                assert np.array_equal(row, np.arange(row[0], row[0] + k))   # contiguous, ascending
                assert 0 <= row[0] and row[-1] < nb                # inside the sequence
                before, after = i - row[0], row[-1] - i
                if row[0] > 0 and row[-1] < nb - 1:                # interior: centred, later on a tie
                    assert after - before in (0, 1)
                    assert after - before == (1 - k % 2)
    assert np.array_equal(oracle.window_selection(7, 7), np.tile(np.arange(7), (7, 1)))
    assert np.array_equal(oracle.window_selection(5, 1), np.arange(5)[:, None])


def test_host_helper_equals_oracle():
    for nb in range(1, 41):
        for k in range(1, nb + 1):
            assert np.array_equal(S.sol_attn_window_blocks(nb, k).numpy(), oracle.window_selection(nb, k)), (nb, k)
    assert np.array_equal(S.sol_attn_window_blocks(504, 76).numpy(), oracle.window_selection(504, 76))


def test_host_helper_rejects_bad_arguments():
    lib = S.load_library()
    assert lib.sol_attn_window_blocks(-1, 1, None) == 2          # ERR_SHAPE
    assert lib.sol_attn_window_blocks(8, 0, None) == 3           # ERR_K
    assert lib.sol_attn_window_blocks(8, 9, None) == 3           # ERR_K
    assert lib.sol_attn_window_blocks(8, 2, None) == 1           # ERR_NULL
    assert lib.sol_attn_window_blocks(0, 0, None) == 0


def _dev(x):
    return torch.from_numpy(np.ascontiguousarray(x).view(np.int16)).view(torch.bfloat16).cuda()


@pytest.mark.gpu
@pytest.mark.parametrize("topk", [1, 4, 9])
def test_window_pattern_fwd_matches_oracle(topk):
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import dataclasses
    wl = dataclasses.replace(W.get("draft_896x512"), name="win", H=2, frames=3, lat_h=8, lat_w=48,
                             coarse=(1, 2, 3), topk=topk, seed=21)          # L = 1152 = 9 blocks
    q, k, v = W.make_qkv(wl)
    nb = wl.n_blocks
    pat = S.sol_attn_window_blocks(nb, topk)
    idx = pat.view(1, 1, nb, topk).expand(wl.B, wl.H, nb, topk).contiguous().cuda()
    out, lse = S.sol_attn_fwd(_dev(q), _dev(k), _dev(v), idx, wl.block, return_lse=True)
    torch.cuda.synchronize()
    sel = np.broadcast_to(oracle.window_selection(nb, topk), (wl.B, wl.H, nb, topk))
    O, L = oracle.attend(oracle.widen(q, "bf16"), oracle.widen(k, "bf16"), oracle.widen(v, "bf16"), sel, wl.block)
    err = np.abs(out.float().double().cpu().numpy() - O)
    assert err.max() <= 2e-2 and err.mean() <= 2e-3, (err.max(), err.mean())
    assert np.abs(lse.double().cpu().numpy() - L).max() <= 1e-2


@pytest.mark.gpu
@pytest.mark.timeout(600)
def test_window_pattern_full_size():
    """1344x768 workload (64,512 tokens, 40 heads), window of 76 blocks, sampled query blocks."""
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    wl = W.get("refine_1344x768")
    q, k, v = W.make_qkv(wl)
    nb = wl.n_blocks
    idx = S.sol_attn_window_blocks(nb, wl.topk).view(1, 1, nb, wl.topk).expand(wl.B, wl.H, nb, wl.topk)
    order = S.sol_attn_frame_order(wl.L, wl.block, wl.lat_h * wl.lat_w, wl.lat_w).cuda()
    Q, K, V = _dev(q), _dev(k), _dev(v)
    out = torch.full_like(Q, float("nan"))
    S.sol_attn_fwd(Q, K, V, idx.contiguous().cuda(), wl.block, out=out, qblock_order=order)
    torch.cuda.synchronize()
    assert not torch.isnan(out).any().item()
    sel = oracle.window_selection(nb, wl.topk)
    Qd, Kd, Vd = (oracle.widen(x, "bf16").reshape(-1, wl.L, wl.d) for x in (q, k, v))
    o = out.view(-1, wl.L, wl.d)
    rng = np.random.default_rng(5)
    errs = []
    for bh in rng.choice(wl.B * wl.H, 3, replace=False):
        for i in [0, nb - 1] + list(rng.choice(nb, 2, replace=False)):
            s = slice(i * wl.block, (i + 1) * wl.block)
            Oi, _ = oracle.attend_block(Qd[bh, s], Kd[bh], Vd[bh], sel[i], wl.block, 1.0 / math.sqrt(wl.d))
            errs.append(np.abs(o[bh, s].float().double().cpu().numpy() - Oi))
    err = np.concatenate(errs)
    assert err.max() <= 2e-2 and err.mean() <= 2e-3, (err.max(), err.mean())
