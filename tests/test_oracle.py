"""Pins of the float64 CPU oracle against facts that do not come from the oracle itself:
closed forms, brute force, library routines that compute the same quantity a
different way, and invariants of the definition.  Each check is chosen so that a
plausible slip in the oracle (a dropped term, a wrong sign, index or scale, a
transposed operand, a wrong tie rule) fails at least one of them.

The reading under test: mean-pooled blocks, pooled score Qbar.Kbar^T/sqrt(d),
top-k key blocks per query block (ties to the lower index, ascending output),
then exact softmax attention over the selected blocks.
"""
import itertools
import math

import numpy as np
import pytest
import torch

import oracle
from block_sparse_attention_attn_amd import workloads as W

pytestmark = pytest.mark.filterwarnings("ignore::DeprecationWarning")


def _rand(shape, seed):
    return np.random.default_rng(seed).standard_normal(shape)


# ----------------------------------------------------------------------------- pool
def test_pool_constant_block_gives_constant():
    X = np.zeros((1, 1, 8, 3))
    X[..., :4, :] = 2.5
    X[..., 4:, :] = -7.0
    P = oracle.pool(X, 4)
    assert P.shape == (1, 1, 2, 3)
    assert np.all(P[..., 0, :] == 2.5) and np.all(P[..., 1, :] == -7.0)


def test_pool_ramp_gives_midpoint():
    # token-linear ramp a + b*t over a block of Bs tokens has mean a + b*(Bs-1)/2
    Bs, nb = 16, 3
    t = np.arange(nb * Bs, dtype=np.float64)
    X = np.stack([3.0 + 0.5 * t, -1.0 - 2.0 * t], axis=-1)[None, None]
    P = oracle.pool(X, Bs)
    for i in range(nb):
        start = i * Bs
        assert P[0, 0, i, 0] == 3.0 + 0.5 * (start + (Bs - 1) / 2)
        assert P[0, 0, i, 1] == -1.0 - 2.0 * (start + (Bs - 1) / 2)


def test_pool_uses_block_not_stride():
    # a transposed reshape (tokens i, i+nb, ...) would mix blocks: make that visible
    X = np.arange(12, dtype=np.float64).reshape(1, 1, 12, 1)
    P = oracle.pool(X, 4)[0, 0, :, 0]
    assert list(P) == [1.5, 5.5, 9.5]


@pytest.mark.parametrize("name", ["tiny_fp32_1k", "draft_896x512"])
def test_pool_is_exact_fsum(name):
    """bf16/fp32 block sums are exact in float64 for the generated data: the oracle's
    mean equals math.fsum(block)/Bs (a correctly rounded sum) on every sampled block."""
    wl = W.get(name)
    Kst = W.make_tensor(wl, 1)
    K = oracle.widen(Kst, wl.dtype)
    P = oracle.pool(K, wl.block)
    rng = np.random.default_rng(7)
    heads = range(wl.B * wl.H) if wl.H <= 2 else rng.choice(wl.B * wl.H, 3, replace=False)
    Kf = K.reshape(-1, wl.L, wl.d)
    Pf = P.reshape(-1, wl.n_blocks, wl.d)
    for bh in heads:
        blocks = range(wl.n_blocks) if wl.n_blocks <= 16 else rng.choice(wl.n_blocks, 12, replace=False)
        for i in blocks:
            blk = Kf[bh, i * wl.block:(i + 1) * wl.block]
            for e in range(wl.d):
                col = blk[:, e]
                assert Pf[bh, i, e] == math.fsum(col) / wl.block
                # exactness: any summation order gives the same float64 value
                assert float(np.sum(col[::-1])) * 1.0 == math.fsum(col)


# ----------------------------------------------------------------------------- scores
def test_scores_match_matmul_and_dot():
    Qb, Kb = _rand((2, 5, 7), 1), _rand((2, 6, 7), 2)
    r = oracle.block_scores(Qb, Kb)
    assert r.shape == (2, 5, 6)
    ref = np.matmul(Qb, np.swapaxes(Kb, -1, -2))
    np.testing.assert_allclose(r, ref, rtol=1e-14, atol=1e-14)
    # a single pair by an explicit fsum of products
    assert abs(r[1, 3, 4] - math.fsum(Qb[1, 3] * Kb[1, 4])) <= 1e-15 * 10


def test_scores_symmetric_and_scale_exact():
    A = _rand((9, 16), 3)
    r = oracle.block_scores(A, A)
    assert np.array_equal(r, r.T)
    r2 = oracle.block_scores(A * 2.0 ** 5, A)
    assert np.array_equal(r2, r * 2.0 ** 5)


def test_identical_key_blocks_score_identically():
    Qb = _rand((4, 32), 4)
    Kb = _rand((6, 32), 5)
    Kb[4] = Kb[1]
    r = oracle.block_scores(Qb, Kb)
    assert np.array_equal(r[:, 4], r[:, 1])


# ----------------------------------------------------------------------------- select
def test_select_bruteforce_subsets_tiny_workload():
    """On the tiny workload the selected set is the unique k-subset maximising sum r
    (no ties occur), found by enumerating all C(16,4) = 1820 subsets."""
    wl = W.get("tiny_fp32_1k")
    Q = oracle.widen(W.make_tensor(wl, 0), wl.dtype)
    K = oracle.widen(W.make_tensor(wl, 1), wl.dtype)
    qb, kb = oracle.pool(Q, wl.block), oracle.pool(K, wl.block)
    idx = oracle.select(qb, kb, wl.topk)
    r = np.einsum("bhid,bhjd->bhij", qb, kb)
    for b, h, i in itertools.product(range(wl.B), range(wl.H), range(wl.n_blocks)):
        best, best_val, second = None, -np.inf, -np.inf
        for sub in itertools.combinations(range(wl.n_blocks), wl.topk):
            v = r[b, h, i, list(sub)].sum()
            if v > best_val:
                best, second, best_val = sub, best_val, v
            elif v > second:
                second = v
        assert best_val > second  # unique maximiser
        assert tuple(idx[b, h, i]) == best


def test_select_ascending_and_matches_stable_argsort():
    r = _rand((3, 11, 40), 6)
    for k in (1, 5, 17, 40):
        sel = oracle.select_from_scores(r, k)
        assert np.all(np.diff(sel, axis=-1) > 0)
        alt = np.sort(np.argsort(-r, axis=-1, kind="stable")[..., :k], axis=-1)
        assert np.array_equal(sel, alt)


def test_select_k_all_and_k_one():
    r = _rand((5, 9), 8)
    assert np.array_equal(oracle.select_from_scores(r, 9), np.tile(np.arange(9), (5, 1)))
    assert np.array_equal(oracle.select_from_scores(r, 1)[:, 0], np.argmax(r, axis=-1))


def test_select_ties_go_to_lower_index():
    # small-integer pooled blocks: every product and sum is exact, so duplicates tie exactly
    Qb = np.array([[1.0, 2.0, 0.0, -1.0]])
    Kb = np.array([[0, 0, 0, 0],      # r = 0
                   [1, 1, 0, 0],      # r = 3
                   [3, 0, 0, 0],      # r = 3  (tie with 1)
                   [0, 0, 5, 0],      # r = 0
                   [1, 1, 0, 0],      # r = 3  (tie with 1, 2)
                   [2, 2, 0, 0],      # r = 6
                   [0, 0, 0, -1]], dtype=np.float64)  # r = 1
    r = oracle.block_scores(Qb, Kb)[0]
    assert list(r) == [0, 3, 3, 0, 3, 6, 1]
    sel = lambda k: list(oracle.select(Qb, Kb, k)[0])  # noqa: E731
    assert sel(1) == [5]
    assert sel(2) == [1, 5]
    assert sel(3) == [1, 2, 5]
    assert sel(4) == [1, 2, 4, 5]
    assert sel(5) == [1, 2, 4, 5, 6]
    assert sel(6) == [0, 1, 2, 4, 5, 6]
    assert sel(7) == [0, 1, 2, 3, 4, 5, 6]
    # negative zero ties with positive zero (lower index wins)
    r0 = np.array([[-0.0, 0.0, -1.0]])
    assert list(oracle.select_from_scores(r0, 1)[0]) == [0]
    r1 = np.array([[0.0, -0.0, -1.0]])
    assert list(oracle.select_from_scores(r1, 1)[0]) == [0]


def test_select_invariant_under_within_block_permutation():
    """Permuting keys (or queries) inside a block leaves the selection bit-identical."""
    wl = W.get("tiny_fp32_1k")
    Q = oracle.widen(W.make_tensor(wl, 0), wl.dtype)
    K = oracle.widen(W.make_tensor(wl, 1), wl.dtype)
    base = oracle.select(oracle.pool(Q, wl.block), oracle.pool(K, wl.block), wl.topk)
    rng = np.random.default_rng(11)
    perm = np.concatenate([i * wl.block + rng.permutation(wl.block) for i in range(wl.n_blocks)])
    Kp, Qp = K[..., perm, :], Q[..., perm, :]
    assert np.array_equal(oracle.select(oracle.pool(Q, wl.block), oracle.pool(Kp, wl.block), wl.topk), base)
    assert np.array_equal(oracle.select(oracle.pool(Qp, wl.block), oracle.pool(K, wl.block), wl.topk), base)
    # while a permutation ACROSS blocks does change the pooled scores
    cross = rng.permutation(wl.L)
    assert not np.array_equal(oracle.pool(K[..., cross, :], wl.block), oracle.pool(K, wl.block))


# ----------------------------------------------------------------------------- attention
def _dense_sdpa(Q, K, V):
    """Brute-force dense attention by torch's own routine, float64 on the CPU."""
    q, k, v = (torch.from_numpy(np.ascontiguousarray(x)) for x in (Q, K, V))
    return torch.nn.functional.scaled_dot_product_attention(q, k, v).numpy()


def test_k_all_equals_dense_attention():
    """With k = nB every query sees every key: the oracle must equal dense softmax attention."""
    wl = W.get("tiny_fp32_1k")
    Q, K, V = (oracle.widen(W.make_tensor(wl, i), wl.dtype) for i in range(3))
    qb, kb = oracle.pool(Q, wl.block), oracle.pool(K, wl.block)
    idx = oracle.select(qb, kb, wl.n_blocks)
    O, lse = oracle.attend(Q, K, V, idx, wl.block)
    ref = _dense_sdpa(Q, K, V)
    assert np.max(np.abs(O - ref)) <= 1e-12
    # dense logsumexp by an independent library routine
    z = np.einsum("bhld,bhmd->bhlm", Q, K) / math.sqrt(wl.d)
    ref_lse = torch.logsumexp(torch.from_numpy(z), dim=-1).numpy()
    assert np.max(np.abs(lse - ref_lse)) <= 1e-12


def test_sparse_equals_dense_on_gathered_keys():
    """For one query block, sparse attention equals dense attention over the gathered keys."""
    rng = np.random.default_rng(12)
    L, d, Bs, k = 96, 8, 16, 2
    Q, K, V = (rng.standard_normal((1, 1, L, d)) for _ in range(3))
    sel = np.array([[[1, 4]] * (L // Bs)], dtype=np.int32)
    O, _ = oracle.attend(Q, K, V, sel, Bs)
    rows = np.r_[16:32, 64:80]
    ref = _dense_sdpa(Q, K[..., rows, :], V[..., rows, :])
    assert np.max(np.abs(O - ref)) <= 1e-12


def test_softmax_weights_sum_to_one():
    wl = W.get("tiny_fp32_1k")
    Q, K, V = (oracle.widen(W.make_tensor(wl, i), wl.dtype) for i in range(3))
    idx = oracle.select(oracle.pool(Q, wl.block), oracle.pool(K, wl.block), wl.topk)
    _, lse = oracle.attend(Q, K, V, idx, wl.block)
    for b, h, i in itertools.product(range(wl.B), range(wl.H), range(wl.n_blocks)):
        rows = (idx[b, h, i][:, None] * wl.block + np.arange(wl.block)).reshape(-1)
        s = slice(i * wl.block, (i + 1) * wl.block)
        z = Q[b, h, s] @ K[b, h, rows].T / math.sqrt(wl.d)
        w = np.exp(z - lse[b, h, s][:, None])
        assert np.max(np.abs(w.sum(axis=1) - 1.0)) <= 1e-12


def test_constant_values_give_constant_output():
    rng = np.random.default_rng(13)
    Q, K = rng.standard_normal((1, 2, 64, 4)), rng.standard_normal((1, 2, 64, 4))
    V = np.full((1, 2, 64, 4), 0.625)
    idx = oracle.select(oracle.pool(Q, 16), oracle.pool(K, 16), 2)
    O, _ = oracle.attend(Q, K, V, idx, 16)
    assert np.max(np.abs(O - 0.625)) <= 1e-15


def test_equal_keys_give_mean_of_selected_values():
    rng = np.random.default_rng(14)
    Q = rng.standard_normal((1, 1, 64, 4))
    K = np.tile(rng.standard_normal(4), (1, 1, 64, 1))
    V = rng.standard_normal((1, 1, 64, 4))
    sel = np.array([[[0, 3], [1, 2], [2, 3], [0, 1]]], dtype=np.int32)
    O, lse = oracle.attend(Q, K, V, sel, 16)
    for i in range(4):
        rows = np.r_[sel[0, i, 0] * 16:(sel[0, i, 0] + 1) * 16, sel[0, i, 1] * 16:(sel[0, i, 1] + 1) * 16]
        want = V[0, 0, rows].mean(axis=0)
        assert np.max(np.abs(O[0, 0, i * 16:(i + 1) * 16] - want)) <= 1e-14
        # all 32 logits equal z: lse = z + ln 32
        z = Q[0, 0, i * 16:(i + 1) * 16] @ K[0, 0, 0] / 2.0
        assert np.max(np.abs(lse[0, 0, i * 16:(i + 1) * 16] - (z + math.log(32)))) <= 1e-13


def test_within_block_permutation_of_keys_leaves_output():
    rng = np.random.default_rng(15)
    L, d, Bs = 128, 8, 16
    Q, K, V = (rng.standard_normal((1, 1, L, d)) for _ in range(3))
    idx = oracle.select(oracle.pool(Q, Bs), oracle.pool(K, Bs), 3)
    O, _ = oracle.attend(Q, K, V, idx, Bs)
    perm = np.concatenate([i * Bs + rng.permutation(Bs) for i in range(L // Bs)])
    idx2 = oracle.select(oracle.pool(Q, Bs), oracle.pool(K[..., perm, :], Bs), 3)
    assert np.array_equal(idx, idx2)
    O2, _ = oracle.attend(Q, K[..., perm, :], V[..., perm, :], idx2, Bs)
    assert np.max(np.abs(O - O2)) <= 1e-12


def test_hand_worked_example_closed_form():
    """L=4, Bs=2, d=2, k=1, worked out by hand:
    Qbar = [[1,0],[0,1]], Kbar = [[1,0],[0,2]] so block 0 picks key block 0 and
    block 1 picks key block 1.  Row 0 (q=[1,0]) sees keys [2,0],[0,0]: logits
    sqrt2, 0.  Row 2 (q=[0,1]) sees keys [0,0],[0,4]: logits 0, 2*sqrt2."""
    Q = np.array([[1, 0], [1, 0], [0, 1], [0, 1]], dtype=np.float64)[None, None]
    K = np.array([[2, 0], [0, 0], [0, 0], [0, 4]], dtype=np.float64)[None, None]
    V = np.array([[1, 2], [3, 4], [5, 6], [7, 8]], dtype=np.float64)[None, None]
    res = oracle.run(Q.astype(np.float32), K.astype(np.float32), V.astype(np.float32), "fp32", 2, 1)
    assert res["idx"][0, 0].tolist() == [[0], [1]]
    assert res["qbar"][0, 0].tolist() == [[1, 0], [0, 1]]
    assert res["kbar"][0, 0].tolist() == [[1, 0], [0, 2]]
    e1, e2 = math.exp(math.sqrt(2)), math.exp(2 * math.sqrt(2))
    o0 = [(1 * e1 + 3) / (1 + e1), (2 * e1 + 4) / (1 + e1)]
    o2 = [(5 + 7 * e2) / (1 + e2), (6 + 8 * e2) / (1 + e2)]
    O, lse = res["out"][0, 0], res["lse"][0, 0]
    assert np.max(np.abs(O[0] - o0)) <= 1e-15 and np.max(np.abs(O[1] - o0)) <= 1e-15
    assert np.max(np.abs(O[2] - o2)) <= 1e-14 and np.max(np.abs(O[3] - o2)) <= 1e-14
    assert abs(lse[0] - math.log(e1 + 1)) <= 1e-15
    assert abs(lse[2] - math.log(1 + e2)) <= 1e-15


def test_scale_argument_and_default():
    rng = np.random.default_rng(16)
    Q, K, V = (rng.standard_normal((1, 1, 32, 16)) for _ in range(3))
    sel = np.array([[[0, 1]] * 2], dtype=np.int32)
    O_default, _ = oracle.attend(Q, K, V, sel, 16)
    O_quarter, _ = oracle.attend(Q, K, V, sel, 16, scale=0.25)    # 1/sqrt(16)
    assert np.array_equal(O_default, O_quarter)
    O_other, _ = oracle.attend(Q, K, V, sel, 16, scale=0.5)
    ref = _dense_sdpa(Q * 2.0, K, V)      # scale 0.5 == default scale on 2*Q
    assert np.max(np.abs(O_other - ref)) <= 1e-12


# ----------------------------------------------------------------------------- margins
def test_margin_certificate_on_tiny_and_ties():
    wl = W.get("tiny_fp32_1k")
    Q = oracle.widen(W.make_tensor(wl, 0), wl.dtype)
    K = oracle.widen(W.make_tensor(wl, 1), wl.dtype)
    rel, amb, ties = oracle.selection_margins(oracle.pool(Q, wl.block), oracle.pool(K, wl.block), wl.topk)
    assert amb == 0 and ties == 0 and rel > 1e-10
    Qb = np.array([[1.0, 2.0]])
    Kb = np.array([[1.0, 1.0], [3.0, 0.0], [0.0, 0.0]])
    assert oracle.selection_margins(Qb, Kb, 1)[2] == 1     # r = 3, 3, 0: exact tie at k=1


# ----------------------------------------------------------------------------- ragged last block
@pytest.mark.parametrize("L", [97, 100, 111, 113])
def test_ragged_pool_is_mean_of_remaining_tokens(L):
    """Block size 16 that does not divide L: the last block is the remaining L - 16(nB-1)
    tokens and its mean is their exact sum (math.fsum) divided by their count."""
    Bs, d = 16, 5
    X = np.round(_rand((2, L, d), 7) * 64) / 64          # dyadic values: sums are exact
    P = oracle.pool(X, Bs)
    nb = -(-L // Bs)
    assert P.shape == (2, nb, d) and oracle.n_blocks(L, Bs) == nb
    last = L - (nb - 1) * Bs
    for b in range(2):
        for e in range(d):
            assert P[b, nb - 1, e] == math.fsum(X[b, L - last:, e]) / last
            for i in range(nb - 1):
                assert P[b, i, e] == math.fsum(X[b, i * Bs:(i + 1) * Bs, e]) / Bs


@pytest.mark.parametrize("L", [97, 120, 127])
def test_ragged_k_all_equals_dense_attention(L):
    """Short last block and k = nB: every query (all L rows) sees exactly the L keys, so the
    oracle must equal dense softmax attention over the L tokens (torch, float64)."""
    Bs, d = 16, 8
    rng = np.random.default_rng(L)
    Q, K, V = (rng.standard_normal((1, 2, L, d)) for _ in range(3))
    nb = oracle.n_blocks(L, Bs)
    idx = oracle.select(oracle.pool(Q, Bs), oracle.pool(K, Bs), nb)
    assert np.array_equal(idx[0, 0, 0], np.arange(nb))
    O, lse = oracle.attend(Q, K, V, idx, Bs)
    assert not np.isnan(O).any()
    assert np.max(np.abs(O - _dense_sdpa(Q, K, V))) <= 1e-12
    z = np.einsum("bhld,bhmd->bhlm", Q, K) / math.sqrt(d)
    assert np.max(np.abs(lse - torch.logsumexp(torch.from_numpy(z), dim=-1).numpy())) <= 1e-12


def test_ragged_selected_short_block_contributes_only_its_tokens():
    """A query block that selects the short last block attends to exactly its tokens plus
    those of its other blocks: dense attention over that gathered key set."""
    Bs, d, L = 16, 6, 70                                 # blocks 0..4, the last one has 6 tokens
    rng = np.random.default_rng(3)
    Q, K, V = (rng.standard_normal((1, 1, L, d)) for _ in range(3))
    sel = np.array([[[1, 4]] * 5], dtype=np.int32)
    O, _ = oracle.attend(Q, K, V, sel, Bs)
    rows = np.r_[16:32, 64:70]
    assert np.max(np.abs(O - _dense_sdpa(Q, K[..., rows, :], V[..., rows, :]))) <= 1e-12
