"""Thin ctypes binding of libsol_attn.so (argument marshalling only).

Every step of the computation runs in the library's HIP kernels; this module
only checks torch tensors, allocates outputs with torch on the inputs' device and
passes raw device pointers plus the current HIP stream.  It never falls back to
another implementation: if the library is missing, calls raise.

Calls (same names as the C ABI):
  sol_attn_pool(q, k, block)                         -> (q_pooled, k_pooled) float64 [B,H,nB,d]
                                                        (nB = ceil(L/block); a last block may be short)
  sol_attn_select(q_pooled, k_pooled, topk, ...)     -> block_idx int32 [B,H,nB,topk] (+ scores)
  sol_attn_fwd(q, k, v, block_idx, block, ...)       -> out [B,H,L,d] (+ lse float32 [B,H,L])
  sol_attn_frame_order(L, block, frame_tokens, row_tokens) -> int32 schedule of the query blocks
  sol_attn_window_blocks(n_blocks, topk)             -> int32 [n_blocks, topk] static window pattern
  sol_attn_check_block_idx(block_idx)                -> rows of an index list sol_attn_fwd does not accept
  sol_attn_cube_permute(x, grid, cube, inverse)      -> x with its tokens in cube-major (or frame-major) order
  sol_attn_pool_cube(q, k, grid, cube)               -> box means of frame-major q, k (read in place)
  sol_attn_fwd_cube(q, k, v, block_idx, grid, cube)  -> bf16 attention over boxes, frame-major in and out
  sparse_attention(q, k, v, block, topk)             -> the three calls in sequence
  cube_sparse_attention(q, k, v, grid, cube, topk)   -> the same with 3-D cube blocks
  sol_attn_probe_mfma()                              -> sustained bf16 matrix-core TFLOP/s (diagnostic)
  sol_attn_quantize(x, fmt) / sol_attn_dequantize(codes, scales, fmt)
                                                     -> 8-bit exchange formats (INT8, FP8_E4M3)
"""
from __future__ import annotations

import ctypes
import os
import re
from typing import Optional, Tuple

import torch

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "libsol_attn.so")
HEADER_PATH = os.path.join(os.path.dirname(_HERE), "include", "sol_attn.h")

BF16, FP32 = 0, 1
STATUS = {0: "OK", 1: "ERR_NULL", 2: "ERR_SHAPE", 3: "ERR_K", 4: "ERR_UNSUPPORTED", 5: "ERR_ALIGN", 6: "ERR_HIP"}

_lib = None


class SolAttnError(RuntimeError):
    def __init__(self, call: str, code: int, msg: str):
        super().__init__(f"{call} failed with {STATUS.get(code, code)}: {msg}")
        self.code = code


def load_library(path: str = LIB_PATH) -> ctypes.CDLL:
    """Load (once) and type the C ABI.  Raises if the library has not been built."""
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(path):
        raise RuntimeError(f"{path} not found: build it with `python -m block_sparse_attention_attn_amd.build`")
    lib = ctypes.CDLL(path)
    vp, i, d = ctypes.c_void_p, ctypes.c_int, ctypes.c_double
    lib.sol_attn_pool.argtypes = [vp, vp, i, i, i, i, i, i, vp, vp, vp]
    lib.sol_attn_pool.restype = i
    lib.sol_attn_select.argtypes = [vp, vp, i, i, i, i, i, vp, vp, vp]
    lib.sol_attn_select.restype = i
    lib.sol_attn_fwd.argtypes = [vp, vp, vp, i, i, i, i, i, i, i, vp, vp, ctypes.c_float, vp, vp, vp]
    lib.sol_attn_fwd.restype = i
    lib.sol_attn_frame_order.argtypes = [i, i, i, i, vp]
    lib.sol_attn_frame_order.restype = i
    lib.sol_attn_window_blocks.argtypes = [i, i, vp]
    lib.sol_attn_window_blocks.restype = i
    lib.sol_attn_cube_permute.argtypes = [vp, vp, i, i, i, i, i, i, i, i, i, i, vp]
    lib.sol_attn_pool_cube.restype = i
    lib.sol_attn_pool_cube.argtypes = [vp, vp, i, i, i, i, i, i, i, i, i, i, vp, vp, vp]
    lib.sol_attn_fwd_cube.restype = i
    lib.sol_attn_fwd_cube.argtypes = [vp, vp, vp, i, i, i, i, i, i, i, i, i, vp, vp, ctypes.c_float, vp, vp, vp]
    lib.sol_attn_cube_permute.restype = i
    lib.sol_attn_quantize.argtypes = [vp, i, i, i, i, i, vp, vp, vp]
    lib.sol_attn_quantize.restype = i
    lib.sol_attn_dequantize.argtypes = [vp, vp, i, i, i, i, i, vp, vp]
    lib.sol_attn_dequantize.restype = i
    lib.sol_attn_check_block_idx.argtypes = [vp, i, i, i, i, vp, vp]
    lib.sol_attn_check_block_idx.restype = i
    lib.sol_attn_probe_mfma.argtypes = [i, i, vp, vp]
    lib.sol_attn_probe_mfma.restype = i
    lib.sol_attn_last_error.argtypes = []
    lib.sol_attn_last_error.restype = ctypes.c_char_p
    lib.sol_attn_version.argtypes = []
    lib.sol_attn_version.restype = i
    _lib = lib
    return lib


def header_symbols(path: str = HEADER_PATH):
    """Names of the functions the public header declares."""
    text = open(path).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(sol_attn_\w+)\s*\(", text)))


def _check(call: str, code: int):
    if code != 0:
        raise SolAttnError(call, code, _lib.sol_attn_last_error().decode())


def _dtype_code(t: torch.Tensor) -> int:
    if t.dtype == torch.bfloat16:
        return BF16
    if t.dtype == torch.float32:
        return FP32
    raise TypeError(f"unsupported dtype {t.dtype} (bfloat16 or float32)")


def _ptr(t: Optional[torch.Tensor]) -> Optional[int]:
    return None if t is None else t.data_ptr()


def _stream(t: torch.Tensor) -> int:
    return torch.cuda.current_stream(t.device).cuda_stream


def _check_on_device(device: torch.device, **tensors: Optional[torch.Tensor]):
    """Every given tensor (None = absent) lives on `device`, a HIP device: the kernels
    dereference these pointers, and a host or other-device pointer would fault there."""
    if device.type != "cuda":
        raise ValueError(f"tensors must be on a HIP device, not {device}")
    for name, t in tensors.items():
        if t is not None and t.device != device:
            raise ValueError(f"{name} must be on {device} (it is on {t.device})")


def _check_qkv(*ts: torch.Tensor):
    ref = ts[0]
    if ref.dim() != 4:
        raise ValueError("tensors must be [B, H, L, d]")
    for t in ts:
        if not t.is_cuda:
            raise ValueError("tensors must be on a HIP device")
        if t.shape != ref.shape or t.dtype != ref.dtype or t.device != ref.device:
            raise ValueError("q, k, v must share shape, dtype and device")
        if not t.is_contiguous():
            raise ValueError("tensors must be contiguous")


def sol_attn_pool(q: torch.Tensor, k: torch.Tensor, block: int) -> Tuple[torch.Tensor, torch.Tensor]:
    lib = load_library()
    _check_qkv(q, k)
    B, H, L, d = q.shape
    nb = -(-L // block) if block > 0 else 0
    qp = torch.empty((B, H, nb, d), dtype=torch.float64, device=q.device)
    kp = torch.empty_like(qp)
    _check("sol_attn_pool", lib.sol_attn_pool(_ptr(q), _ptr(k), _dtype_code(q), B, H, L, d, block,
                                              _ptr(qp), _ptr(kp), _stream(q)))
    return qp, kp


def sol_attn_select(q_pooled: torch.Tensor, k_pooled: torch.Tensor, topk: int, return_scores: bool = False):
    lib = load_library()
    if q_pooled.dtype != torch.float64 or k_pooled.dtype != torch.float64:
        raise TypeError("pooled tensors must be float64")
    if (q_pooled.dim() != 4 or q_pooled.shape != k_pooled.shape
            or not (q_pooled.is_contiguous() and k_pooled.is_contiguous())):
        raise ValueError("pooled tensors must be contiguous [B,H,nB,d] of equal shape")
    _check_on_device(q_pooled.device, k_pooled=k_pooled)
    B, H, nb, d = q_pooled.shape
    idx = torch.empty((B, H, nb, max(topk, 0)), dtype=torch.int32, device=q_pooled.device)
    scores = torch.empty((B, H, nb, nb), dtype=torch.float64, device=q_pooled.device) if return_scores else None
    _check("sol_attn_select", lib.sol_attn_select(_ptr(q_pooled), _ptr(k_pooled), B, H, nb, d, topk, _ptr(idx),
                                                  _ptr(scores), _stream(q_pooled)))
    return (idx, scores) if return_scores else idx


def sol_attn_check_block_idx(block_idx: torch.Tensor, n_blocks: Optional[int] = None) -> int:
    """Number of rows of an int32 [B,H,nB,topk] device list that sol_attn_fwd does not accept
    (an entry outside [0, nB) or not strictly ascending); synchronises the stream."""
    lib = load_library()
    if block_idx.dtype != torch.int32 or block_idx.dim() != 4 or not block_idx.is_contiguous() or not block_idx.is_cuda:
        raise ValueError("block_idx must be a contiguous int32 device tensor [B,H,nB,topk]")
    B, H, nb, topk = block_idx.shape
    bad = torch.empty(1, dtype=torch.int32, device=block_idx.device)
    _check("sol_attn_check_block_idx", lib.sol_attn_check_block_idx(_ptr(block_idx), B, H, nb if n_blocks is None
                                                                    else n_blocks, topk, _ptr(bad),
                                                                    _stream(block_idx)))
    return int(bad.item())


def sol_attn_frame_order(L: int, block: int, frame_tokens: int, row_tokens: int) -> torch.Tensor:
    """Host-computed query-block schedule for frame-major video tokens (int32 CPU tensor)."""
    lib = load_library()
    nb = -(-L // block) if block > 0 else 0
    order = torch.empty(max(nb, 0), dtype=torch.int32)
    _check("sol_attn_frame_order", lib.sol_attn_frame_order(L, block, frame_tokens, row_tokens,
                                                            order.data_ptr() if nb else None))
    return order


def sol_attn_window_blocks(n_blocks: int, topk: int) -> torch.Tensor:
    """Host-computed static window pattern: int32 CPU tensor [n_blocks, topk] (see the C header)."""
    lib = load_library()
    idx = torch.empty((max(n_blocks, 0), max(topk, 0)), dtype=torch.int32)
    _check("sol_attn_window_blocks", lib.sol_attn_window_blocks(n_blocks, topk,
                                                                idx.data_ptr() if idx.numel() else None))
    return idx


def sol_attn_fwd(q: torch.Tensor, k: torch.Tensor, v: torch.Tensor, block_idx: torch.Tensor, block: int,
                 softmax_scale: Optional[float] = None, return_lse: bool = False,
                 out: Optional[torch.Tensor] = None, qblock_order: Optional[torch.Tensor] = None,
                 lse: Optional[torch.Tensor] = None):
    """`out` / `lse` (optional): caller-provided outputs; passing `lse` implies return_lse."""
    lib = load_library()
    _check_qkv(q, k, v)
    B, H, L, d = q.shape
    if block_idx.dtype != torch.int32 or not block_idx.is_contiguous() or block_idx.dim() != 4:
        raise ValueError("block_idx must be contiguous int32 [B,H,nB,topk]")
    _check_on_device(q.device, block_idx=block_idx, out=out, lse=lse, qblock_order=qblock_order)
    topk = block_idx.shape[-1]
    if block > 0 and tuple(block_idx.shape[:3]) != (B, H, -(-L // block)):
        raise ValueError("block_idx leading dims must be [B,H,L/block]")
    if out is None:
        out = torch.empty_like(q)
    elif out.shape != q.shape or out.dtype != q.dtype or out.device != q.device or not out.is_contiguous():
        raise ValueError("out must be a contiguous tensor like q")
    if lse is not None:
        if (tuple(lse.shape) != (B, H, L) or lse.dtype != torch.float32 or lse.device != q.device
                or not lse.is_contiguous()):
            raise ValueError("lse must be a contiguous float32 [B,H,L] tensor on q's device")
        return_lse = True
    elif return_lse:
        lse = torch.empty((B, H, L), dtype=torch.float32, device=q.device)
    if qblock_order is not None:
        if (qblock_order.dtype != torch.int32 or qblock_order.device != q.device or
                qblock_order.numel() != (-(-L // block) if block > 0 else 0) or not qblock_order.is_contiguous()):
            raise ValueError("qblock_order must be a contiguous int32 device tensor of L/block entries")
    scale = 0.0 if softmax_scale is None else float(softmax_scale)
    _check("sol_attn_fwd", lib.sol_attn_fwd(_ptr(q), _ptr(k), _ptr(v), _dtype_code(q), B, H, L, d, block, topk,
                                            _ptr(block_idx), _ptr(qblock_order), scale, _ptr(out), _ptr(lse),
                                            _stream(q)))
    return (out, lse) if return_lse else out


def sparse_attention(q: torch.Tensor, k: torch.Tensor, v: torch.Tensor, block: int, topk: int,
                     softmax_scale: Optional[float] = None, return_lse: bool = False,
                     qblock_order: Optional[torch.Tensor] = None):
    """Pool -> select -> fwd.  Returns out (and lse); use the individual calls to
    inspect the pooled tensors or the selected blocks."""
    qp, kp = sol_attn_pool(q, k, block)
    idx = sol_attn_select(qp, kp, topk)
    return sol_attn_fwd(q, k, v, idx, block, softmax_scale, return_lse, qblock_order=qblock_order)


def sol_attn_cube_permute(x: torch.Tensor, grid: Tuple[int, int, int], cube: Tuple[int, int, int],
                          inverse: bool = False, out: Optional[torch.Tensor] = None) -> torch.Tensor:
    """Reorder the tokens of x ([B,H,L,d] or [B,H,L], L = T*h*w for grid = (T,h,w)) from
    frame-major to cube-major order for boxes cube = (bt,by,bx), or back with inverse=True."""
    lib = load_library()
    if not x.is_cuda or not x.is_contiguous() or x.dim() not in (3, 4):
        raise ValueError("x must be a contiguous device tensor [B,H,L,d] or [B,H,L]")
    B, H, L = x.shape[:3]
    T, h, w = grid
    if T * h * w != L:
        raise ValueError(f"grid {grid} does not hold L={L} tokens")
    row_bytes = (x.shape[3] if x.dim() == 4 else 1) * x.element_size()
    if out is None:
        out = torch.empty_like(x)
    elif out.shape != x.shape or out.dtype != x.dtype or not out.is_contiguous() or out.device != x.device:
        raise ValueError("out must match x")
    bt, by, bx = cube
    _check("sol_attn_cube_permute", lib.sol_attn_cube_permute(_ptr(x), _ptr(out), B, H, T, h, w, row_bytes, bt, by,
                                                              bx, int(bool(inverse)), _stream(x)))
    return out


def _check_grid(L: int, grid: Tuple[int, int, int]):
    T, h, w = grid
    if T * h * w != L:
        raise ValueError(f"grid {grid} does not hold L={L} tokens")


def sol_attn_pool_cube(q: torch.Tensor, k: torch.Tensor, grid: Tuple[int, int, int],
                       cube: Tuple[int, int, int]) -> Tuple[torch.Tensor, torch.Tensor]:
    """Mean of every bt x by x bx box of frame-major q, k ([B,H,T*h*w,d]), read in place:
    float64 [B,H,n_boxes,d] with boxes numbered time, row, column."""
    lib = load_library()
    _check_qkv(q, k)
    B, H, L, d = q.shape
    _check_grid(L, grid)
    T, h, w = grid
    bt, by, bx = cube
    nb = (T // bt) * (h // by) * (w // bx) if min(bt, by, bx) > 0 else 0
    qp = torch.empty((B, H, nb, d), dtype=torch.float64, device=q.device)
    kp = torch.empty_like(qp)
    _check("sol_attn_pool_cube", lib.sol_attn_pool_cube(_ptr(q), _ptr(k), _dtype_code(q), B, H, T, h, w, d, bt, by,
                                                        bx, _ptr(qp), _ptr(kp), _stream(q)))
    return qp, kp


def sol_attn_fwd_cube(q: torch.Tensor, k: torch.Tensor, v: torch.Tensor, block_idx: torch.Tensor,
                      grid: Tuple[int, int, int], cube: Tuple[int, int, int], softmax_scale: Optional[float] = None,
                      return_lse: bool = False, out: Optional[torch.Tensor] = None,
                      qblock_order: Optional[torch.Tensor] = None):
    """bf16 sparse attention (d = 128) with query/key block c = box c (128 tokens) of the
    frame-major latent grid, read and written in place."""
    lib = load_library()
    _check_qkv(q, k, v)
    B, H, L, d = q.shape
    _check_grid(L, grid)
    T, h, w = grid
    bt, by, bx = cube
    if block_idx.dtype != torch.int32 or not block_idx.is_contiguous() or block_idx.dim() != 4:
        raise ValueError("block_idx must be contiguous int32 [B,H,n_boxes,topk]")
    _check_on_device(q.device, block_idx=block_idx, out=out, qblock_order=qblock_order)
    nb = L // (bt * by * bx) if min(bt, by, bx) > 0 else 0
    if tuple(block_idx.shape[:3]) != (B, H, nb):
        raise ValueError("block_idx leading dims must be [B,H,n_boxes]")
    if out is None:
        out = torch.empty_like(q)
    elif out.shape != q.shape or out.dtype != q.dtype or not out.is_contiguous():
        raise ValueError("out must be a contiguous tensor like q")
    lse = torch.empty((B, H, L), dtype=torch.float32, device=q.device) if return_lse else None
    if qblock_order is not None:
        if (qblock_order.dtype != torch.int32 or qblock_order.device != q.device or qblock_order.numel() != nb
                or not qblock_order.is_contiguous()):
            raise ValueError("qblock_order must be a contiguous int32 device tensor of n_boxes entries")
    scale = 0.0 if softmax_scale is None else float(softmax_scale)
    _check("sol_attn_fwd_cube", lib.sol_attn_fwd_cube(_ptr(q), _ptr(k), _ptr(v), B, H, T, h, w, bt, by, bx,
                                                      block_idx.shape[-1], _ptr(block_idx), _ptr(qblock_order),
                                                      scale, _ptr(out), _ptr(lse), _stream(q)))
    return (out, lse) if return_lse else out


def cube_sparse_attention(q: torch.Tensor, k: torch.Tensor, v: torch.Tensor, grid: Tuple[int, int, int],
                          cube: Tuple[int, int, int], topk: int, softmax_scale: Optional[float] = None,
                          return_lse: bool = False, return_idx: bool = False, reorder: bool = False):
    """Sparse attention with 3-D cube blocks on frame-major q, k, v.  block_idx (if
    returned) indexes boxes in cube-major numbering.

    bf16 with 128-token boxes and d = 128 reads the boxes in place (pool_cube,
    select, fwd_cube); otherwise, or with reorder=True, q, k, v are reordered to
    cube-major order, pooled, selected and attended with block = bt*by*bx, and the
    outputs reordered back.  Both routes give the same bits."""
    T, h, w = grid
    bt, by, bx = cube
    V = bt * by * bx
    order = sol_attn_frame_order(q.shape[2], V, V * (h // by) * (w // bx), V * (w // bx)).to(q.device)
    if not reorder and q.dtype == torch.bfloat16 and V == 128 and q.shape[-1] == 128:
        qp, kp = sol_attn_pool_cube(q, k, grid, cube)
        idx = sol_attn_select(qp, kp, topk)
        res = sol_attn_fwd_cube(q, k, v, idx, grid, cube, softmax_scale, return_lse, qblock_order=order)
        out = list(res) if return_lse else [res]
    else:
        qc, kc, vc = (sol_attn_cube_permute(x, grid, cube) for x in (q, k, v))
        qp, kp = sol_attn_pool(qc, kc, V)
        idx = sol_attn_select(qp, kp, topk)
        res = sol_attn_fwd(qc, kc, vc, idx, V, softmax_scale, return_lse, qblock_order=order)
        oc, lc = res if return_lse else (res, None)
        out = [sol_attn_cube_permute(oc, grid, cube, inverse=True)]
        if return_lse:
            out.append(sol_attn_cube_permute(lc, grid, cube, inverse=True))
    if return_idx:
        out.append(idx)
    return out[0] if len(out) == 1 else tuple(out)


INT8, FP8_E4M3 = 0, 1


def sol_attn_quantize(x: torch.Tensor, fmt: int) -> Tuple[torch.Tensor, torch.Tensor]:
    """bf16 [B,H,L,d] -> (codes uint8 [B,H,L,d] (int8 bit patterns for INT8), scales float32 [B,H,L])."""
    lib = load_library()
    if x.dtype != torch.bfloat16 or x.dim() != 4 or not x.is_cuda or not x.is_contiguous():
        raise ValueError("x must be a contiguous bfloat16 device tensor [B,H,L,d]")
    B, H, L, d = x.shape
    codes = torch.empty((B, H, L, d), dtype=torch.uint8, device=x.device)
    scales = torch.empty((B, H, L), dtype=torch.float32, device=x.device)
    _check("sol_attn_quantize", lib.sol_attn_quantize(_ptr(x), B, H, L, d, fmt, _ptr(codes), _ptr(scales),
                                                      _stream(x)))
    return codes, scales


def sol_attn_dequantize(codes: torch.Tensor, scales: torch.Tensor, fmt: int,
                        out: Optional[torch.Tensor] = None) -> torch.Tensor:
    """(codes uint8 [B,H,L,d], scales float32 [B,H,L]) -> bf16 [B,H,L,d]."""
    lib = load_library()
    if codes.dtype not in (torch.uint8, torch.int8) or codes.dim() != 4 or not codes.is_contiguous():
        raise ValueError("codes must be contiguous 1-byte [B,H,L,d]")
    B, H, L, d = codes.shape
    if scales.dtype != torch.float32 or tuple(scales.shape) != (B, H, L) or not scales.is_contiguous():
        raise ValueError("scales must be contiguous float32 [B,H,L]")
    _check_on_device(codes.device, scales=scales, out=out)
    if out is None:
        out = torch.empty((B, H, L, d), dtype=torch.bfloat16, device=codes.device)
    elif out.dtype != torch.bfloat16 or tuple(out.shape) != (B, H, L, d) or not out.is_contiguous():
        raise ValueError("out must be a contiguous bfloat16 [B,H,L,d] tensor")
    _check("sol_attn_dequantize", lib.sol_attn_dequantize(_ptr(codes), _ptr(scales), B, H, L, d, fmt, _ptr(out),
                                                          _stream(codes)))
    return out


def sol_attn_probe_mfma(workgroups: int = 1024, iters: int = 20000, repeats: int = 5) -> float:
    """Sustained bf16 matrix-core rate (TFLOP/s) of the current device, from timing the
    diagnostic kernel (best of `repeats` launches after one warm-up)."""
    lib = load_library()
    sink = torch.empty(workgroups, dtype=torch.float32, device="cuda")
    stream = torch.cuda.current_stream()
    call = lambda: _check("sol_attn_probe_mfma", lib.sol_attn_probe_mfma(workgroups, iters, _ptr(sink),
                                                                         stream.cuda_stream))
    call()
    best = None
    for _ in range(repeats):
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record(stream)
        call()
        e1.record(stream)
        e1.synchronize()
        ms = e0.elapsed_time(e1)
        best = ms if best is None else min(best, ms)
    return workgroups * 4 * iters * 4 * 32768.0 / (best * 1e-3) / 1e12


def version() -> int:
    return load_library().sol_attn_version()
