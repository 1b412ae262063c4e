"""Float64 CPU oracle of Sol-Attn block-sparse attention (test infrastructure only).

What the pages fix
------------------
Sol-Attn is the largest single source of the Sol-H3 runtime's speed-up: a sparse
attention that decides, per query, which parts of the attention computation
matter, and that needs no retraining ("Videomodel MiniMax-H3 rendert sneller dan
afspelen", section "Waar de snelheidswinst vandaan komt").  The same section says
the *preparation* of the sparse attention was made faster, i.e. there is a
selection step before the attention proper.  In the two-stage schedule it runs in
the high-resolution refinement steps ("NVIDIA Adds Two-Stage Generation for
MiniMax H3 ...", first paragraph).

The concrete reading implemented (the pages give no formula)
-----------------------------------------------------------
* tokens are frame-major; the sequence is cut into contiguous blocks of Bs tokens;
  when Bs does not divide L the last block holds the remaining L - (nB-1) Bs tokens
  (nB = ceil(L / Bs));
* every query block and key block is mean-pooled (block sum / number of its tokens);
* pooled score of (query block i, key block j) is r_ij / sqrt(d), r_ij = Qbar_i . Kbar_j;
* each query block keeps the k key blocks with the largest score, ties going to
  the lower key-block index; indices are emitted in ascending order;
* every query of block i then attends with exact softmax(q k^T / sqrt(d)) over
  the union of the selected key blocks' tokens, with no mask.

Second blocking (cube_blocks, run_cube): on a T x h x w latent grid a block may be
a bt x by x bx box of latents instead of a run of consecutive tokens; pooling,
selection and attention are then the same definitions over those token sets.

Ranking uses the unscaled r_ij: multiplying by the positive constant 1/sqrt(d)
preserves the order in exact arithmetic, and not applying it avoids creating
rounding ties.  Everything is float64; inputs are the exact widenings of the
stored bf16/fp32 values.

Every function below is the definition written out step by step.  Library
primitives used as single steps: numpy sum, lexsort and matmul.
"""
from __future__ import annotations

import math
from typing import Optional, Tuple

import numpy as np

__all__ = ["widen", "n_blocks", "block_rows", "pool", "block_scores", "select", "select_from_scores",
           "attend", "attend_block", "selection_margins", "run", "window_selection",
           "cube_blocks", "pool_sets", "attend_sets", "run_cube"]


def widen(stored: np.ndarray, dtype: str) -> np.ndarray:
    """Exact float64 value of stored inputs: bf16 given as uint16 bit patterns, or float32."""
    if dtype == "bf16":
        bits = np.asarray(stored, dtype=np.uint16).astype(np.uint32) << 16
        return bits.view(np.float32).astype(np.float64)
    if dtype == "fp32":
        return np.asarray(stored, dtype=np.float32).astype(np.float64)
    raise ValueError(dtype)


def n_blocks(L: int, block: int) -> int:
    """Number of blocks: the last one may be shorter (ceil(L / block))."""
    return -(-L // block)


def block_rows(i: int, L: int, block: int) -> slice:
    """Token rows of block i: [i*block, min((i+1)*block, L))."""
    return slice(i * block, min((i + 1) * block, L))


def pool(X: np.ndarray, block: int) -> np.ndarray:
    """Block mean: [..., L, d] -> [..., nB, d], Xbar_i = (sum of block i's rows) / (its row count)."""
    *lead, L, d = X.shape
    nb = n_blocks(L, block)
    out = np.empty((*lead, nb, d), dtype=np.float64)
    for i in range(nb):
        rows = X[..., block_rows(i, L, block), :]
        out[..., i, :] = rows.sum(axis=-2) / rows.shape[-2]
    return out


def block_scores(Qbar: np.ndarray, Kbar: np.ndarray, chunk: int = 64) -> np.ndarray:
    """r_ij = sum_e Qbar_ie * Kbar_je for all block pairs: [..., nq, d] x [..., nk, d] -> [..., nq, nk].

    Each r_ij is evaluated the same way (elementwise product, then a sum over e),
    so two identical key blocks always get identical scores.
    """
    *lead, nq, d = Qbar.shape
    nk = Kbar.shape[-2]
    r = np.empty((*lead, nq, nk), dtype=np.float64)
    for i0 in range(0, nq, chunk):
        i1 = min(nq, i0 + chunk)
        prod = Qbar[..., i0:i1, None, :] * Kbar[..., None, :, :]
        r[..., i0:i1, :] = prod.sum(axis=-1)
    return r


def select_from_scores(r: np.ndarray, topk: int) -> np.ndarray:
    """Per row of r (the last axis indexes key blocks j): the first `topk` j in the order
    (r desc, j asc), returned in ascending j.  int32 [..., topk]."""
    *lead, nk = r.shape
    if not 1 <= topk <= nk:
        raise ValueError("topk out of range")
    flat = r.reshape(-1, nk)
    out = np.empty((flat.shape[0], topk), dtype=np.int32)
    j = np.arange(nk)
    for row in range(flat.shape[0]):
        order = np.lexsort((j, -flat[row]))     # primary: -r ascending, secondary: j ascending
        out[row] = np.sort(order[:topk])
    return out.reshape(*lead, topk)


def select(Qbar: np.ndarray, Kbar: np.ndarray, topk: int) -> np.ndarray:
    """Top-k key blocks per query block by pooled score (see module docstring)."""
    return select_from_scores(block_scores(Qbar, Kbar), topk)


def attend_block(Qi: np.ndarray, K: np.ndarray, V: np.ndarray, sel_i: np.ndarray, block: int,
                 scale: float) -> Tuple[np.ndarray, np.ndarray]:
    """Exact softmax attention of the rows of one query block over its selected key blocks.

    Qi [rows of the block, d]; K, V [L, d] of the same (b, h); sel_i [k] key-block indices.
    Returns (O_i [Bs, d], lse_i [Bs]) with lse = m + ln(sum exp(z - m)).
    """
    rows = (sel_i[:, None] * block + np.arange(block)[None, :]).reshape(-1)
    rows = rows[rows < K.shape[0]]           # a short last block has only its own tokens
    return _softmax_attend(Qi, K[rows], V[rows], scale)


def _softmax_attend(Qi: np.ndarray, Kc: np.ndarray, Vc: np.ndarray, scale: float):
    """softmax(Qi Kc^T * scale) Vc and its log-sum-exp, for query rows Qi and key/value rows Kc, Vc."""
    z = (Qi @ Kc.T) * scale                  # [rows, keys]
    m = z.max(axis=1, keepdims=True)
    p = np.exp(z - m)
    l = p.sum(axis=1, keepdims=True)
    O = (p @ Vc) / l
    lse = (m + np.log(l))[:, 0]
    return O, lse


def attend(Q: np.ndarray, K: np.ndarray, V: np.ndarray, sel: np.ndarray, block: int,
           scale: Optional[float] = None, qblocks: Optional[np.ndarray] = None):
    """Block-sparse attention for [..., L, d] inputs and sel [..., nB, k].

    scale defaults to 1/sqrt(d).  `qblocks` (optional) restricts the query blocks
    computed (same set for every leading index); other rows of O are NaN.
    Returns (O [..., L, d], lse [..., L]).
    """
    *lead, L, d = Q.shape
    if scale is None:
        scale = 1.0 / math.sqrt(d)
    nb = n_blocks(L, block)
    Qf = Q.reshape(-1, L, d)
    Kf = K.reshape(-1, L, d)
    Vf = V.reshape(-1, L, d)
    sf = sel.reshape(-1, nb, sel.shape[-1])
    O = np.full(Qf.shape, np.nan)
    lse = np.full(Qf.shape[:2], np.nan)
    blocks = range(nb) if qblocks is None else qblocks
    for bh in range(Qf.shape[0]):
        for i in blocks:
            s = block_rows(i, L, block)
            O[bh, s], lse[bh, s] = attend_block(Qf[bh, s], Kf[bh], Vf[bh], sf[bh, i], block, scale)
    return O.reshape(*lead, L, d), lse.reshape(*lead, L)


def window_selection(n_blocks: int, topk: int) -> np.ndarray:
    """Static window pattern (the decoder's windowed attention as a fixed key-block list;
    Sol-H3-VAE model card, opening paragraph).  Reading: row i holds the topk consecutive
    key blocks whose centre is nearest to i -- for even topk two windows are equally
    near and the later one is taken (one more block after i than before it) -- shifted
    inwards at the two ends of the sequence.  Written as a search over all starts."""
    starts = np.arange(n_blocks - topk + 1)
    centres = starts + (topk - 1) / 2.0
    out = np.empty((n_blocks, topk), dtype=np.int32)
    for i in range(n_blocks):
        dist = np.abs(centres - i)
        s = starts[np.flatnonzero(dist == dist.min())[-1]]
        out[i] = np.arange(s, s + topk)
    return out


def cube_blocks(T: int, h: int, w: int, cube) -> np.ndarray:
    """3-D blocking of a T x h x w latent token grid (the latent of a clip is frames x
    rows x cols, Sol-H3-VAE model card, section "Usage"; token n = (t*h + y)*w + x).

    Reading: a block is a box of bt x by x bx latents (cube = (bt, by, bx)), which must
    divide (T, h, w); boxes are numbered like the tokens themselves (time slowest, then
    row, then column), and inside a box its tokens keep their frame-major order.
    Returns int64 [nB, bt*by*bx]: row i lists the token indices of block i."""
    bt, by, bx = cube
    if min(bt, by, bx) < 1 or T % bt or h % by or w % bx:
        raise ValueError("cube does not tile the latent grid")
    blocks = []
    for tc in range(T // bt):
        for yc in range(h // by):
            for xc in range(w // bx):
                blocks.append([(t * h + y) * w + x
                               for t in range(tc * bt, (tc + 1) * bt)
                               for y in range(yc * by, (yc + 1) * by)
                               for x in range(xc * bx, (xc + 1) * bx)])
    return np.asarray(blocks, dtype=np.int64).reshape(-1, bt * by * bx)


def pool_sets(X: np.ndarray, sets: np.ndarray) -> np.ndarray:
    """Block mean over arbitrary token sets: [..., L, d] -> [..., nB, d], block i = mean of X[..., sets[i], :]."""
    *lead, L, d = X.shape
    out = np.empty((*lead, sets.shape[0], d), dtype=np.float64)
    for i, rows in enumerate(sets):
        out[..., i, :] = X[..., rows, :].sum(axis=-2) / len(rows)
    return out


def attend_sets(Q: np.ndarray, K: np.ndarray, V: np.ndarray, sets: np.ndarray, sel: np.ndarray,
                scale: Optional[float] = None, qblocks: Optional[np.ndarray] = None):
    """Block-sparse attention with blocks given as token sets: the rows sets[i] of query
    block i attend over the tokens of the key blocks sel[..., i, :].  Inputs and outputs
    keep the token order of Q (for cube blocks: frame-major).  Other arguments as attend()."""
    *lead, L, d = Q.shape
    if scale is None:
        scale = 1.0 / math.sqrt(d)
    nb = sets.shape[0]
    Qf, Kf, Vf = (x.reshape(-1, L, d) for x in (Q, K, V))
    sf = sel.reshape(-1, nb, sel.shape[-1])
    O = np.full(Qf.shape, np.nan)
    lse = np.full(Qf.shape[:2], np.nan)
    blocks = range(nb) if qblocks is None else qblocks
    for bh in range(Qf.shape[0]):
        for i in blocks:
            rows = sets[i]
            keys = sets[sf[bh, i]].reshape(-1)
            O[bh, rows], lse[bh, rows] = _softmax_attend(Qf[bh, rows], Kf[bh, keys], Vf[bh, keys], scale)
    return O.reshape(*lead, L, d), lse.reshape(*lead, L)


def run_cube(q_stored, k_stored, v_stored, dtype: str, grid, cube, topk: int,
             qblocks: Optional[np.ndarray] = None):
    """Whole path with 3-D cube blocks on stored frame-major inputs [B,H,L,d], L = T*h*w:
    returns dict(sets, qbar, kbar, idx, out, lse); idx indexes cubes, out/lse are frame-major."""
    T, h, w = grid
    sets = cube_blocks(T, h, w, cube)
    Q, K, V = widen(q_stored, dtype), widen(k_stored, dtype), widen(v_stored, dtype)
    qbar, kbar = pool_sets(Q, sets), pool_sets(K, sets)
    idx = select(qbar, kbar, topk)
    out, lse = attend_sets(Q, K, V, sets, idx, qblocks=qblocks)
    return dict(sets=sets, qbar=qbar, kbar=kbar, idx=idx, out=out, lse=lse)


def selection_margins(Qbar: np.ndarray, Kbar: np.ndarray, topk: int):
    """Certificate that the float64 selection equals the exact-arithmetic selection.

    For every row: gap = r_(k) - r_(k+1) between the k-th and (k+1)-th largest
    scores (inf when k = nB), and a rounding bound on |computed r - exact r| of
    2 * gamma_d * sum_e |Qbar_ie||Kbar_je| with gamma_d = d*u/(1-d*u), u = 2^-53
    (the standard bound for a d-term dot product; the factor 2 covers the two
    scores being compared).  A row with gap == 0 is an exact tie, resolved by
    index; a row with 0 < gap <= bound is ambiguous.

    Returns (min relative gap over rows with gap > 0, number of ambiguous rows,
    number of rows whose k-th/(k+1)-th scores tie exactly).
    """
    r = block_scores(Qbar, Kbar)
    mag = block_scores(np.abs(Qbar), np.abs(Kbar))
    d = Qbar.shape[-1]
    u = 2.0 ** -53
    gamma = d * u / (1 - d * u)
    *lead, nq, nk = r.shape
    rf = r.reshape(-1, nk)
    mf = mag.reshape(-1, nk)
    min_rel = math.inf
    ambiguous = 0
    ties = 0
    if topk >= nk:
        return math.inf, 0, 0
    for row in range(rf.shape[0]):
        srt = np.sort(rf[row])[::-1]
        gap = srt[topk - 1] - srt[topk]
        bound = 2.0 * gamma * mf[row].max()
        if gap == 0:
            ties += 1
            continue
        if gap <= bound:
            ambiguous += 1
        scale_row = max(abs(srt[topk - 1]), abs(srt[topk]), 1e-300)
        min_rel = min(min_rel, gap / scale_row)
    return min_rel, ambiguous, ties


def run(q_stored, k_stored, v_stored, dtype: str, block: int, topk: int,
        qblocks: Optional[np.ndarray] = None):
    """Whole path on stored inputs [B,H,L,d]: returns dict(qbar, kbar, idx, out, lse)."""
    Q, K, V = widen(q_stored, dtype), widen(k_stored, dtype), widen(v_stored, dtype)
    qbar, kbar = pool(Q, block), pool(K, block)
    idx = select(qbar, kbar, topk)
    out, lse = attend(Q, K, V, idx, block, qblocks=qblocks)
    return dict(qbar=qbar, kbar=kbar, idx=idx, out=out, lse=lse)
