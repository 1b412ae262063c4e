"""Calls from several host threads, each on its own stream, with different inputs: every
result equals the sequential, single-stream result bit for bit (the library keeps no
per-call state, and its one-time per-device set-up is safe to race)."""
import dataclasses
import threading

import numpy as np
import pytest
import torch

from block_sparse_attention_attn_amd import workloads as W

pytestmark = pytest.mark.gpu

ROUNDS = 3


@pytest.fixture(scope="module")
def S():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    from block_sparse_attention_attn_amd import sol_attn
    sol_attn.load_library()
    return sol_attn


def dev_bf16(bits):
    return torch.from_numpy(np.ascontiguousarray(bits).view(np.int16)).view(torch.bfloat16).cuda()


def test_concurrent_streams_match_sequential(S):
    cases = []
    for seed in (41, 42, 43):
        wl = dataclasses.replace(W.get("draft_896x512"), name=f"thr{seed}", H=3, frames=2, lat_h=32, lat_w=56,
                                 topk=9, coarse=(1, 4, 7), seed=seed)
        cases.append((wl, tuple(dev_bf16(x) for x in W.make_qkv(wl))))

    def step(wl, Q, K, V):
        qp, kp = S.sol_attn_pool(Q, K, wl.block)
        idx = S.sol_attn_select(qp, kp, wl.topk)
        out, lse = S.sol_attn_fwd(Q, K, V, idx, wl.block, return_lse=True)
        return idx, out, lse

    ref = [step(wl, *qkv) for wl, qkv in cases]
    torch.cuda.synchronize()
    print(f"threads: {len(cases)} cases, {ROUNDS} rounds", flush=True)

    results = [[None] * ROUNDS for _ in cases]
    errors = []

    def worker(n):
        try:
            wl, qkv = cases[n]
            stream = torch.cuda.Stream()
            for r in range(ROUNDS):
                with torch.cuda.stream(stream):
                    res = step(wl, *qkv)
                stream.synchronize()
                results[n][r] = res
        except Exception as exc:  # reported below, in the main thread
            errors.append((n, repr(exc)))

    threads = [threading.Thread(target=worker, args=(n,)) for n in range(len(cases))]
    for t in threads:
        t.start()
    for t in threads:
        t.join(timeout=120)
    assert not any(t.is_alive() for t in threads), "a worker thread did not finish"
    assert not errors, errors
    torch.cuda.synchronize()
    for n, (idx0, out0, lse0) in enumerate(ref):
        for r in range(ROUNDS):
            idx, out, lse = results[n][r]
            assert torch.equal(idx, idx0), (n, r)
            assert torch.equal(out.view(torch.int16), out0.view(torch.int16)), (n, r)
            assert torch.equal(lse.view(torch.int32), lse0.view(torch.int32)), (n, r)
