"""The whole step (pool -> select -> fwd, through the C ABI) captured into a HIP graph and
replayed: every replay reproduces the eager results bit for bit, also when the outputs were
overwritten between replays, when other work runs on the device in between, and when the
inputs are rewritten in place (the graph reads them, it does not keep their values).
The step records kernel launches only: no allocation, memset or copy inside the calls."""
import dataclasses

import numpy as np
import pytest
import torch

from block_sparse_attention_attn_amd import workloads as W

pytestmark = pytest.mark.gpu

REPLAYS = 4


@pytest.fixture(scope="module")
def S():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    from block_sparse_attention_attn_amd import sol_attn
    sol_attn.load_library()
    return sol_attn


def dev_bf16(bits):
    return torch.from_numpy(np.ascontiguousarray(bits).view(np.int16)).view(torch.bfloat16).cuda()


def same_bits(a, b):
    if a.dtype in (torch.bfloat16, torch.float16):
        return torch.equal(a.view(torch.int16), b.view(torch.int16))
    if a.dtype == torch.float32:
        return torch.equal(a.view(torch.int32), b.view(torch.int32))
    if a.dtype == torch.float64:
        return torch.equal(a.view(torch.int64), b.view(torch.int64))
    return torch.equal(a, b)


@pytest.mark.parametrize("route", ["blocks", "ragged_scheduled", "cube_in_place"])
def test_step_graph_replays_match_eager(S, route):
    """blocks: 128-token blocks; ragged_scheduled: a short last block and the frame-aware
    query-block schedule; cube_in_place: 2x8x8 boxes read in place."""
    wl = dataclasses.replace(W.get("draft_896x512"), name="graph", H=4, frames=4, lat_h=32, lat_w=56, topk=14,
                             coarse=(2, 4, 7), seed=31)
    q, k, v = W.make_qkv(wl)
    if route == "ragged_scheduled":   # a short last block: 7168 - 77 tokens
        q, k, v = (x[..., : wl.L - 77, :] for x in (q, k, v))
    Q, K, V = dev_bf16(q), dev_bf16(k), dev_bf16(v)
    L = Q.shape[2]
    order = None
    if route == "ragged_scheduled":
        order = S.sol_attn_frame_order(L, wl.block, wl.lat_h * wl.lat_w, wl.lat_w).cuda()
    grid, box = wl.grid, (2, 8, 8)
    print(f"graph capture: route={route} L={L} k={wl.topk}", flush=True)

    def step():
        if route == "cube_in_place":
            qp, kp = S.sol_attn_pool_cube(Q, K, grid, box)
            idx = S.sol_attn_select(qp, kp, wl.topk)
            out, lse = S.sol_attn_fwd_cube(Q, K, V, idx, grid, box, return_lse=True)
        else:
            qp, kp = S.sol_attn_pool(Q, K, wl.block)
            idx = S.sol_attn_select(qp, kp, wl.topk)
            out, lse = S.sol_attn_fwd(Q, K, V, idx, wl.block, return_lse=True, qblock_order=order)
        return qp, kp, idx, out, lse

    ref = step()   # eager (also the warm-up: every one-time set-up happens here)
    torch.cuda.synchronize()

    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        step()
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()

    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        static = step()
    torch.cuda.synchronize()

    other = torch.randn(512, 512, device="cuda")
    for rep in range(REPLAYS):
        # overwrite every output so that a replay that skipped a write would show
        for t in static:
            if t.dtype.is_floating_point:
                t.fill_(float("nan"))
            else:
                t.fill_(-7)
        other = other @ other.T / 512.0          # unrelated eager work between replays
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        for name, a, b in zip(("qbar", "kbar", "idx", "out", "lse"), static, ref):
            assert same_bits(a, b), (rep, name)

    # inputs rewritten in place: the replay follows them
    q2, k2, v2 = (np.ascontiguousarray(x[..., ::-1, :]) for x in (q, k, v))   # tokens in reverse order
    Q.copy_(dev_bf16(q2))
    K.copy_(dev_bf16(k2))
    V.copy_(dev_bf16(v2))
    ref2 = step()
    torch.cuda.synchronize()
    g.replay()
    torch.cuda.synchronize()
    for name, a, b in zip(("qbar", "kbar", "idx", "out", "lse"), static, ref2):
        assert same_bits(a, b), ("rewritten inputs", name)
    assert not same_bits(static[3], ref[3])
