"""The bf16 attention kernel keeps a running max per key half and re-scales O and the weight
sum only when a lane's weights for a tile add up to more than 2^15 (or are not finite).
These inputs make that path fire after the first tile: the scores of later tiles rise far
above everything seen before (in log2 units, 20 per tile and a single jump of 120), fall
(no re-scale after the first tile), or do both for different query rows.  Outputs and lse
are compared with the float64 oracle on every row.

Construction: dimension 0 of every query row is +A or -A and dimension 0 of every key row
of key block j is c_j, so block j adds about +-A c_j / sqrt(d) to the scores of a row; the
other dimensions are small noise.  The given index lists run over every block in a chosen
order, so the order decides when the large scores arrive.
"""
import math

import numpy as np
import pytest
import torch

import oracle

pytestmark = pytest.mark.gpu

BF16_MAX, BF16_MEAN = 2e-2, 2e-3
NB, BS, D, H = 8, 128, 128, 2
A = 8.0


@pytest.fixture(scope="module")
def S():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    from block_sparse_attention_attn_amd import sol_attn
    sol_attn.load_library()
    return sol_attn


def to_bf16_bits(x):
    return torch.from_numpy(np.ascontiguousarray(x, dtype=np.float32)).to(torch.bfloat16).view(torch.int16).numpy()


def make_case(log2_steps, signs, seed):
    """q, k, v as bf16 bit patterns; log2_steps[j] = score offset (log2 units, for a + row) of key block j."""
    rng = np.random.default_rng(seed)
    L = NB * BS
    q = 0.3 * rng.standard_normal((1, H, L, D))
    k = 0.3 * rng.standard_normal((1, H, L, D))
    v = rng.standard_normal((1, H, L, D))
    q[..., 0] = A * signs[None, None, :]
    per_unit = A / math.sqrt(D) / math.log(2.0)      # log2 units added per unit of c_j
    for j, step in enumerate(log2_steps):
        k[:, :, j * BS:(j + 1) * BS, 0] = step / per_unit
    return to_bf16_bits(q), to_bf16_bits(k), to_bf16_bits(v)


CASES = {
    # tile t of the list (ascending blocks) is 20 log2 units above tile t-1 for + rows
    "rising": (np.arange(NB) * 20.0, np.ones(NB * BS), np.arange(NB)),
    # one jump of 120 log2 units at the last tile of the list
    "jump_last": (np.r_[np.zeros(NB - 1), 120.0], np.ones(NB * BS), np.arange(NB)),
    # the largest scores come first: after the first tile no re-scale is needed
    "falling": (np.arange(NB) * 20.0, np.ones(NB * BS), np.arange(NB)[::-1].copy()),
    # half the rows see rising scores, half falling ones, in the same tile order
    "mixed_rows": (np.arange(NB) * 20.0, np.where(np.arange(NB * BS) % 3 == 0, -1.0, 1.0), np.arange(NB)),
}


@pytest.mark.parametrize("name", sorted(CASES))
def test_running_max_rescale_matches_oracle(S, name):
    steps, signs, order = CASES[name]
    q, k, v = make_case(steps, signs, seed=11)
    sel = np.broadcast_to(order.astype(np.int32), (1, H, NB, NB)).copy()
    Qd, Kd, Vd = (oracle.widen(x, "bf16") for x in (q, k, v))
    O, lse = oracle.attend(Qd, Kd, Vd, sel, BS)
    dev = lambda x: torch.from_numpy(np.ascontiguousarray(x)).view(torch.bfloat16).cuda()
    out, glse = S.sol_attn_fwd(dev(q), dev(k), dev(v), torch.from_numpy(sel).cuda(), BS, return_lse=True)
    torch.cuda.synchronize()
    got = out.float().double().cpu().numpy()
    assert np.isfinite(got).all()
    err = np.abs(got - O)
    print(f"{name}: max|err| {err.max():.3e} mean {err.mean():.3e} lse range [{lse.min():.1f}, {lse.max():.1f}]", flush=True)
    assert err.max() <= BF16_MAX and err.mean() <= BF16_MEAN, (err.max(), err.mean())
    gl = glse.cpu().numpy().astype(np.float64)
    assert (np.abs(gl - lse) <= 1e-3 * np.maximum(1.0, np.abs(lse))).all(), np.abs(gl - lse).max()
