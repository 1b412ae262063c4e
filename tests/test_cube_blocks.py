"""3-D cube blocks (a block is a bt x by x bx box of the T x h x w latent grid instead
of a run of consecutive frame-major tokens).

CPU: the oracle's cube blocking is pinned to facts that do not come from it -- a
partition of the tokens into aligned boxes, the same boxes obtained by a reshape and
axis transpose of the grid, the 1-D blocking it reduces to for boxes that are whole
latent rows, the exact fsum mean, and dense attention when every block is kept."""
import math

import numpy as np
import pytest
import torch

import oracle


def _rand(shape, seed):
    return np.random.default_rng(seed).standard_normal(shape)


def _by_reshape(X, grid, cube):
    """Cube-major token order derived independently: split each grid axis into
    (box index, offset in box), move the three box indices in front, flatten."""
    T, h, w = grid
    bt, by, bx = cube
    *lead, L, d = X.shape
    n = len(lead)
    Y = X.reshape(*lead, T // bt, bt, h // by, by, w // bx, bx, d)
    perm = list(range(n)) + [n + 0, n + 2, n + 4, n + 1, n + 3, n + 5, n + 6]
    return Y.transpose(perm).reshape(*lead, L, d)


@pytest.mark.parametrize("grid,cube", [((4, 16, 16), (4, 4, 4)), ((4, 6, 10), (2, 3, 5)),
                                       ((3, 4, 6), (1, 2, 3)), ((16, 48, 84), (4, 8, 4)),
                                       ((2, 3, 4), (2, 3, 4)), ((2, 3, 4), (1, 1, 1))])
def test_cube_blocks_partition_into_aligned_boxes(grid, cube):
    T, h, w = grid
    bt, by, bx = cube
    sets = oracle.cube_blocks(T, h, w, cube)
    L = T * h * w
    assert sets.shape == (L // (bt * by * bx), bt * by * bx)
    assert np.array_equal(np.sort(sets.reshape(-1)), np.arange(L))          # every token exactly once
    t, rem = np.divmod(sets, h * w)
    y, x = np.divmod(rem, w)
    for arr, b in ((t, bt), (y, by), (x, bx)):                                # inside one aligned box
        lo = arr.min(axis=1)
        assert np.all(lo % b == 0) and np.all(arr.max(axis=1) - lo == b - 1)
    assert np.all(np.diff(sets, axis=1) > 0)                                  # frame-major inside a box
    boxes = np.stack([t[:, 0] // bt, y[:, 0] // by, x[:, 0] // bx], axis=1)
    key = (boxes[:, 0] * (h // by) + boxes[:, 1]) * (w // bx) + boxes[:, 2]
    assert np.array_equal(key, np.arange(sets.shape[0]))                     # numbered time, row, col


@pytest.mark.parametrize("grid,cube", [((4, 6, 10), (2, 3, 5)), ((4, 16, 16), (4, 4, 4)), ((6, 4, 9), (3, 2, 3))])
def test_cube_order_equals_reshape_transpose(grid, cube):
    L = int(np.prod(grid))
    X = _rand((2, L, 3), 1)
    sets = oracle.cube_blocks(*grid, cube)
    assert np.array_equal(X[:, sets.reshape(-1)], _by_reshape(X, grid, cube))


def test_cube_rejects_non_dividing_boxes():
    for cube in [(3, 1, 1), (1, 4, 1), (1, 1, 4), (0, 1, 1)]:
        with pytest.raises(ValueError):
            oracle.cube_blocks(4, 10, 14, cube)


def test_cube_pool_is_exact_fsum_of_the_box():
    grid, cube = (4, 6, 10), (2, 3, 5)
    T, h, w = grid
    X = np.round(_rand((T * h * w, 4), 2) * 64) / 64 + 1e3       # exactly summable magnitudes
    sets = oracle.cube_blocks(T, h, w, cube)
    P = oracle.pool_sets(X, sets)
    i = 0
    for tc in range(T // 2):
        for yc in range(h // 3):
            for xc in range(w // 5):
                for e in range(4):
                    vals = [X[(t * h + y) * w + x, e] for t in range(2 * tc, 2 * tc + 2)
                            for y in range(3 * yc, 3 * yc + 3) for x in range(5 * xc, 5 * xc + 5)]
                    assert P[i, e] == math.fsum(vals) / 30
                i += 1


def test_row_boxes_reduce_to_one_dimensional_blocks():
    """A box of whole latent rows (1 x by x w) is a run of by*w consecutive tokens, so
    the cube path must give exactly the 1-D path with block = by*w."""
    grid = (4, 6, 8)
    L = int(np.prod(grid))
    q, k, v = (_rand((1, 2, L, 16), s).astype(np.float32) for s in (3, 4, 5))
    for by, topk in ((1, 5), (2, 3), (3, 8)):
        a = oracle.run_cube(q, k, v, "fp32", grid, (1, by, 8), topk)
        b = oracle.run(q, k, v, "fp32", by * 8, topk)
        for key in ("qbar", "kbar", "idx", "out", "lse"):
            assert np.array_equal(a[key], b[key]), (by, key)


@pytest.mark.parametrize("grid,cube,topk", [((4, 6, 10), (2, 3, 5), 3), ((4, 16, 16), (4, 4, 4), 4),
                                            ((4, 16, 16), (1, 8, 8), 6)])
def test_cube_path_equals_one_dimensional_path_on_reordered_tokens(grid, cube, topk):
    """Reordering Q, K, V into cube-major order (by reshape) and blocking consecutively
    must give the same selection, and the same outputs once reordered back."""
    L = int(np.prod(grid))
    q, k, v = (_rand((1, 2, L, 16), s).astype(np.float32) for s in (6, 7, 8))
    V = int(np.prod(cube))
    a = oracle.run_cube(q, k, v, "fp32", grid, cube, topk)
    b = oracle.run(*(_by_reshape(x, grid, cube) for x in (q, k, v)), "fp32", V, topk)
    assert np.array_equal(a["idx"], b["idx"])
    assert np.array_equal(a["qbar"], b["qbar"])
    back = np.empty_like(b["out"])
    back[..., a["sets"].reshape(-1), :] = b["out"]
    assert np.array_equal(a["out"], back)


def test_cube_k_all_equals_dense_attention():
    grid, cube = (2, 6, 10), (2, 3, 5)
    L = int(np.prod(grid))
    q, k, v = (_rand((1, 2, L, 8), s).astype(np.float32) for s in (9, 10, 11))
    res = oracle.run_cube(q, k, v, "fp32", grid, cube, L // 30)
    Q, K, V = (torch.from_numpy(x.astype(np.float64)) for x in (q, k, v))
    ref = torch.nn.functional.scaled_dot_product_attention(Q, K, V).numpy()
    assert np.abs(res["out"] - ref).max() <= 1e-12
    z = np.einsum("bhld,bhmd->bhlm", q.astype(np.float64), k.astype(np.float64)) / math.sqrt(8)
    lse = np.log(np.exp(z).sum(-1))
    assert np.abs(res["lse"] - lse).max() <= 1e-12


def test_cube_selection_follows_the_box_means():
    """Keys constant on each box with a one-hot direction: the best box for a query box
    is the one whose direction matches its own, which a wrong box membership breaks."""
    grid, cube = (2, 4, 6), (1, 2, 3)          # 8 boxes of 6 tokens
    T, h, w = grid
    L, d = T * h * w, 8
    sets = oracle.cube_blocks(T, h, w, cube)
    K = np.zeros((L, d))
    Q = np.zeros((L, d))
    for i, rows in enumerate(sets):
        K[rows, i] = 1.0 + i
        Q[rows, i] = 1.0
    idx = oracle.select(oracle.pool_sets(Q, sets), oracle.pool_sets(K, sets), 1)
    assert np.array_equal(idx[:, 0], np.arange(8))
