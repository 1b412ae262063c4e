"""Seeded synthetic Q/K/V workloads shaped like the Sol-H3 latent token grids.

This module only *makes inputs*. It holds none of the sparse-attention arithmetic
(no pooling, scoring, selection or softmax) and is the one module shared by the
HIP path's tests/benchmark and the CPU oracle's tests.

Shapes follow the Sol-H3 pipeline described on the pages:

* the two-stage schedule runs a draft at 896x512 and refines at 1344x768, 1080p
  or 2K ("NVIDIA Adds Two-Stage Generation for MiniMax H3 ...", first and second
  paragraphs), and Sol-H3 renders 5 s and 10 s clips at 1344x768 ("Videomodel
  MiniMax-H3 rendert sneller dan afspelen", section "De cijfers achter Sol-H3");
* the video latent is a (T, H/16, W/16) grid (Sol-H3-VAE model card, section
  "Usage"), so the tokens of one clip are T x (H/16) x (W/16).

Tokens are frame-major and row-major inside a frame: token n = (t*h + y)*w + x.

Values: per (tensor, batch, head, channel) an N(0,1) field on a coarse
(Tc, hc, wc) grid is upsampled trilinearly (corner-aligned) to (T, h, w), then
0.3*N(0,1) i.i.d. noise is added.  Large workloads are divided by the tensor's
global root-mean-square; the tiny fp32 workload is left unscaled.  The fp64
result is rounded once, to nearest-even, to bf16 (returned as uint16 bit
patterns) or to fp32.

Random streams: numpy PCG64 seeded with SeedSequence(seed); it spawns one child
per tensor (Q, K, V), and each child spawns one grandchild per (b, h).  Inside a
head the coarse field [d, Tc, hc, wc] is drawn first, then the noise [L, d].

Cache: when a cache directory is named (the `cache_dir` argument, else the
SOL_ATTN_CACHE_DIR environment variable; unset or empty means no cache), make_qkv
stores each tensor's bits as a plain .npy file named by `input_key` -- a hash of
every field of the workload and GENERATOR_VERSION -- and later calls with the same
key load them instead of generating.  Bump GENERATOR_VERSION whenever the values
this module produces change, so that stale files are never read.
"""
from __future__ import annotations

import concurrent.futures as cf
import dataclasses
import hashlib
import json
import math
import os
from typing import Dict, Optional, Sequence, Tuple

import numpy as np

__all__ = [
    "Workload", "WORKLOADS", "get", "make_qkv", "make_tensor", "f64_to_bf16_bits",
    "bf16_bits_to_f32", "GENERATOR_VERSION", "input_key", "cache_dir_from_env",
]

GENERATOR_VERSION = 1


@dataclasses.dataclass(frozen=True)
class Workload:
    name: str
    B: int
    H: int
    d: int
    dtype: str            # "bf16" or "fp32"
    frames: int           # latent frames T
    lat_h: int            # latent rows  (pixel height / 16)
    lat_w: int            # latent cols  (pixel width / 16)
    block: int            # tokens per block Bs
    topk: int             # key blocks kept per query block
    coarse: Tuple[int, int, int]   # (Tc, hc, wc) grid of the smooth field
    unit_rms: bool
    seed: int
    extra_topk: Tuple[int, ...] = ()   # further k values run on the same tensors
    cube: Tuple[int, int, int] = (1, 1, 1)   # (bt, by, bx) box for 3-D cube blocks, bt*by*bx == block

    @property
    def grid(self) -> Tuple[int, int, int]:
        return (self.frames, self.lat_h, self.lat_w)

    @property
    def L(self) -> int:
        return self.frames * self.lat_h * self.lat_w

    @property
    def n_blocks(self) -> int:
        return -(-self.L // self.block)          # the last block may be short

    def effective_flops(self, topk: Optional[int] = None) -> float:
        """4*B*H*L*(k*Bs)*d: the two contractions over the selected key blocks."""
        k = self.topk if topk is None else topk
        return 4.0 * self.B * self.H * self.L * (k * self.block) * self.d


# The five workloads: a tiny fp32 case the oracle finishes instantly, the
# 896x512 draft stage, the 1344x768 refinement stage (the headline size,
# 64,512 tokens), a 10 s clip at 1344x768 and a 2K (2048x1152) refinement.
# `cube` is the box used when the same tokens are cut into 3-D blocks: one block's
# worth of latents (bt*by*bx == block) that tiles the grid -- 2x8x8 where 8 divides
# the latent width, 4x8x4 at 1344x768, whose 84 latent columns 8 does not divide.
WORKLOADS: Dict[str, Workload] = {
    w.name: w for w in [
        Workload("tiny_fp32_1k", 1, 2, 64, "fp32", 4, 16, 16, 64, 4, (2, 4, 4), False, 0,
                 extra_topk=(16,), cube=(4, 4, 4)),
        Workload("draft_896x512", 1, 40, 128, "bf16", 16, 32, 56, 128, 56, (4, 8, 14), True, 1, cube=(2, 8, 8)),
        Workload("refine_1344x768", 1, 40, 128, "bf16", 16, 48, 84, 128, 76, (4, 12, 21), True, 2,
                 cube=(4, 8, 4)),
        Workload("clip10s_1344x768", 1, 40, 128, "bf16", 32, 48, 84, 128, 101, (8, 12, 21), True, 3,
                 cube=(4, 8, 4)),
        Workload("refine_2k", 1, 40, 128, "bf16", 16, 72, 128, 128, 92, (4, 18, 32), True, 4,
                 extra_topk=(1152,), cube=(2, 8, 8)),
    ]
}
HEADLINE = "refine_1344x768"


def get(name: str) -> Workload:
    return WORKLOADS[name]


def _workers() -> int:
    return max(1, min(16, os.cpu_count() or 1))


def _interp_matrix(n_out: int, n_in: int) -> np.ndarray:
    """Linear interpolation weights, corner-aligned: out[i] samples in[i*(n_in-1)/(n_out-1)]."""
    U = np.zeros((n_out, n_in), dtype=np.float64)
    if n_in == 1 or n_out == 1:
        U[:, 0] = 1.0
        return U
    for i in range(n_out):
        pos = i * (n_in - 1) / (n_out - 1)
        i0 = min(int(np.floor(pos)), n_in - 2)
        f = pos - i0
        U[i, i0] += 1.0 - f
        U[i, i0 + 1] += f
    return U


def _head_field(rng: np.random.Generator, d: int, grid: Tuple[int, int, int],
                coarse: Tuple[int, int, int], noise: float = 0.3) -> np.ndarray:
    """One head: [L, d] float64 = upsampled coarse N(0,1) field + noise*N(0,1)."""
    T, h, w = grid
    Tc, hc, wc = coarse
    c = rng.standard_normal((d, Tc, hc, wc))
    Ut, Uy, Ux = _interp_matrix(T, Tc), _interp_matrix(h, hc), _interp_matrix(w, wc)
    a = np.tensordot(Ut, c, axes=([1], [1]))        # [T, d, hc, wc]
    a = np.tensordot(Uy, a, axes=([1], [2]))        # [h, T, d, wc]
    a = np.tensordot(Ux, a, axes=([1], [3]))        # [w, h, T, d]
    field = np.ascontiguousarray(a.transpose(2, 1, 0, 3)).reshape(T * h * w, d)
    field += noise * rng.standard_normal((T * h * w, d))
    return field


def f64_to_bf16_bits(x: np.ndarray) -> np.ndarray:
    """Round float64 to bfloat16 (round to nearest, ties to even) in ONE step.

    Returns uint16 bit patterns.  Going through float32 first could round twice;
    here the 8-bit significand is rounded directly with np.rint (ties-to-even).
    Values whose bf16 result would be subnormal, infinite or NaN are rejected.
    """
    x = np.asarray(x, dtype=np.float64)
    m, e = np.frexp(x)                       # x = m * 2**e, 0.5 <= |m| < 1
    r = np.rint(np.ldexp(m, 8))              # integer significand, |r| in [128, 256]
    v = np.ldexp(r, e - 8)                   # exactly representable in bf16
    nz = v != 0
    if np.any(~np.isfinite(v)) or np.any(np.abs(v[nz]) < 2.0 ** -126) or np.any(np.abs(v) > 3.0e38):
        raise ValueError("value outside the normal bf16 range")
    bits32 = v.astype(np.float32).view(np.uint32)   # exact: v has <= 8 significant bits
    return (bits32 >> 16).astype(np.uint16)


def bf16_bits_to_f32(bits: np.ndarray) -> np.ndarray:
    return (np.asarray(bits, dtype=np.uint16).astype(np.uint32) << 16).view(np.float32)


def make_tensor(wl: Workload, which: int, heads: Optional[Sequence[int]] = None) -> np.ndarray:
    """Tensor `which` (0=Q, 1=K, 2=V) as stored bits: uint16 [B,H,L,d] (bf16) or float32.

    `heads` restricts generation to a subset of head indices (b*H + h) and returns
    [len(heads), L, d]; only valid for unscaled workloads or when the global RMS is
    supplied through the full tensor (the RMS needs every head).
    """
    grid = (wl.frames, wl.lat_h, wl.lat_w)
    tensor_seq = np.random.SeedSequence(wl.seed).spawn(3)[which]
    head_seqs = tensor_seq.spawn(wl.B * wl.H)
    sel = list(range(wl.B * wl.H)) if heads is None else list(heads)
    if heads is not None and wl.unit_rms:
        raise ValueError("a head subset of a unit-RMS workload needs the full tensor's RMS")
    out = np.empty((len(sel), wl.L, wl.d), dtype=np.float64)

    def gen(n):
        out[n] = _head_field(np.random.Generator(np.random.PCG64(head_seqs[sel[n]])), wl.d, grid, wl.coarse)
        return float(np.sum(np.square(out[n])))

    # heads are independent streams: generate them on a thread pool (numpy releases the GIL)
    with cf.ThreadPoolExecutor(max_workers=_workers()) as ex:
        sumsq = list(ex.map(gen, range(len(sel))))
    if wl.unit_rms:
        rms = np.sqrt(math.fsum(sumsq) / out.size)
    else:
        rms = 1.0
    if wl.dtype == "bf16":
        res = np.empty(out.shape, dtype=np.uint16)

        def rnd(n):
            res[n] = f64_to_bf16_bits(out[n] / rms)

        with cf.ThreadPoolExecutor(max_workers=_workers()) as ex:
            list(ex.map(rnd, range(len(sel))))
    else:
        res = (out / rms).astype(np.float32)
    if heads is None:
        res = res.reshape(wl.B, wl.H, wl.L, wl.d)
    return res


def input_key(wl: Workload) -> str:
    """Hex key naming the generated tensors: every workload field plus GENERATOR_VERSION."""
    fields = dataclasses.asdict(wl)
    fields["generator_version"] = GENERATOR_VERSION
    blob = json.dumps(fields, sort_keys=True, separators=(",", ":"))
    return hashlib.sha256(blob.encode()).hexdigest()[:24]


def cache_dir_from_env() -> Optional[str]:
    d = os.environ.get("SOL_ATTN_CACHE_DIR", "")
    return d or None


def _expected(wl: Workload):
    return (wl.B, wl.H, wl.L, wl.d), np.dtype(np.uint16 if wl.dtype == "bf16" else np.float32)


def _load_cached(path: str, wl: Workload) -> Optional[np.ndarray]:
    """The cached tensor, or None when the file is missing or does not have the workload's shape/type."""
    if not os.path.exists(path):
        return None
    try:
        x = np.load(path, allow_pickle=False)
    except (OSError, ValueError):
        return None
    shape, dtype = _expected(wl)
    return x if x.shape == shape and x.dtype == dtype else None


def _store(path: str, x: np.ndarray) -> None:
    """Write through a temporary name and rename, so a reader never sees half a file."""
    tmp = f"{path}.{os.getpid()}.tmp"
    with open(tmp, "wb") as f:
        np.save(f, x, allow_pickle=False)
    os.replace(tmp, path)


def make_qkv(wl: Workload, cache_dir: Optional[str] = None):
    """(Q, K, V) stored bits for the workload, each [B,H,L,d].

    With a cache directory (argument, else SOL_ATTN_CACHE_DIR) the tensors are read
    from / written to <dir>/inputs/<input_key>_{q,k,v}.npy."""
    cache_dir = cache_dir or cache_dir_from_env()
    if cache_dir is None:
        return tuple(make_tensor(wl, i) for i in range(3))
    sub = os.path.join(cache_dir, "inputs")
    os.makedirs(sub, exist_ok=True)
    key = input_key(wl)
    out = []
    for i, tag in enumerate("qkv"):
        path = os.path.join(sub, f"{key}_{tag}.npy")
        x = _load_cached(path, wl)
        if x is None:
            x = make_tensor(wl, i)
            _store(path, x)
        out.append(x)
    return tuple(out)
