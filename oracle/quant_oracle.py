"""CPU oracle of the 8-bit exchange formats (test infrastructure only).

What the pages fix
------------------
Between the eight GPUs of the Sol-H3 runtime the Q, K and V tensors travel as INT8
and the attention output as FP8, which shrinks the exchanged data by 51.6 percent
("Videomodel MiniMax-H3 rendert sneller dan afspelen", section "Waar de
snelheidswinst vandaan komt").  Nothing else is given.

The reading implemented
-----------------------
* Granularity: one float32 scale per token row of one head (d values), symmetric.
  With d = 128 a row then costs d + 4 = 132 bytes against 2d = 256 in bf16: 51.56 %
  of the bf16 bytes, the page's figure read as the size that remains (a cut *by*
  51.6 % would leave less than one byte per value, which 8-bit codes cannot reach).
* INT8 (Q, K, V): with amax = max |x| over the row, the stored scale is amax / 127 and
  code = round-half-even(x * (127 / amax)), clamped to [-127, 127].
* FP8 (the output): OCP E4M3 ("e4m3fn": 4 exponent bits with bias 7, 3 mantissa bits,
  subnormals, largest finite 448, no infinities, S.1111.111 = NaN);
  stored scale amax / 448; code = x * (448 / amax) rounded to nearest-even E4M3,
  saturated to +-448.
* The page fixes no rounding order.  The reading taken is the published absmax
  scheme of LLM.int8() (Dettmers et al., 2022, section on absmax quantization): a
  per-row scaling constant qmax/amax, and code = round(constant * x).  So the value
  coded is fl32(x * fl32(qmax/amax)); the stored scale amax/qmax is what the receiver
  multiplies by.  Dividing each value by the stored scale is the other possible order
  and gives different codes on ordinary rows; tests/test_oracle_exact_pins.py pins
  this reading against exact rational arithmetic and shows the two orders differ.
* A row of zeros gets scale 0 and all-zero codes.
* Decoding: value = code * scale, rounded to bf16 (nearest-even).
* Every quantity that decides a code is float32 with IEEE-rounded float32 division
  and multiplication (the exchanged scale is a float32).

Library primitives used as single steps: numpy float32 arithmetic, rint, abs/max.
"""
from __future__ import annotations

import numpy as np

__all__ = ["INT8_MAX", "E4M3_MAX", "int8_quantize", "int8_dequantize", "e4m3_decode", "e4m3_encode",
           "fp8_quantize", "fp8_dequantize", "bf16_bits_round", "bf16_bits_to_f32"]

INT8_MAX = np.float32(127.0)
E4M3_MAX = np.float32(448.0)


def bf16_bits_to_f32(bits: np.ndarray) -> np.ndarray:
    """Exact float32 value of bf16 bit patterns (uint16)."""
    return (np.asarray(bits, dtype=np.uint16).astype(np.uint32) << 16).view(np.float32)


def bf16_bits_round(x: np.ndarray) -> np.ndarray:
    """float32 -> bf16 bit patterns, round to nearest, ties to even (finite inputs)."""
    u = np.asarray(x, dtype=np.float32).view(np.uint32).astype(np.uint64)
    return ((u + 0x7FFF + ((u >> 16) & 1)) >> 16).astype(np.uint16)


def _row_scale(x32: np.ndarray, qmax: np.float32) -> np.ndarray:
    amax = np.max(np.abs(x32), axis=-1)
    return (amax / qmax).astype(np.float32)


def _scaled(x32: np.ndarray, qmax: np.float32) -> np.ndarray:
    """x * (qmax / amax) per row in float32; rows of zeros give 0."""
    amax = np.max(np.abs(x32), axis=-1)
    safe = np.where(amax == 0, np.float32(1), amax).astype(np.float32)
    inv = (qmax / safe).astype(np.float32)
    v = (x32 * inv[..., None]).astype(np.float32)
    return np.where((amax == 0)[..., None], np.float32(0), v)


def int8_quantize(x_bits: np.ndarray):
    """bf16 rows [..., d] (uint16 bit patterns) -> (int8 codes [..., d], float32 scales [...])."""
    x32 = bf16_bits_to_f32(x_bits)
    scale = _row_scale(x32, INT8_MAX)
    v = _scaled(x32, INT8_MAX)
    codes = np.clip(np.rint(v), -127, 127).astype(np.int8)
    return codes, scale


def int8_dequantize(codes: np.ndarray, scales: np.ndarray) -> np.ndarray:
    """(int8 codes, float32 scales) -> bf16 bit patterns of code * scale."""
    v = (np.asarray(codes).astype(np.float32) * np.asarray(scales, np.float32)[..., None]).astype(np.float32)
    return bf16_bits_round(v)


def e4m3_decode(codes: np.ndarray) -> np.ndarray:
    """OCP E4M3 codes (uint8) -> float64 values (NaN for the two NaN codes)."""
    c = np.asarray(codes, dtype=np.uint8).astype(np.int64)
    sign = np.where(c & 0x80, -1.0, 1.0)
    e = (c >> 3) & 0xF
    m = c & 0x7
    mag = np.where(e == 0, m / 8.0 * 2.0 ** -6, (1.0 + m / 8.0) * 2.0 ** (e - 7))
    mag = np.where((e == 15) & (m == 7), np.nan, mag)
    return sign * mag


def e4m3_encode(v: np.ndarray) -> np.ndarray:
    """float32 values -> OCP E4M3 codes, round to nearest even, saturated to +-448.

    |v| >= 2^-6 lies in a binade [2^e, 2^(e+1)) whose E4M3 spacing is 2^(e-3); below
    2^-6 the spacing is the subnormal step 2^-9.  Rounding |v| to an integer multiple
    of the spacing with ties to even is round-to-nearest-even on the 3-bit mantissa."""
    v = np.asarray(v, dtype=np.float32).astype(np.float64)     # exact
    mag = np.minimum(np.abs(v), 448.0)
    e = np.floor(np.log2(np.where(mag > 0, mag, 1.0)))
    e = np.maximum(e, -6.0)
    step = 2.0 ** (e - 3)
    q = np.rint(mag / step) * step                             # exact: power-of-two scaling
    q = np.minimum(q, 448.0)
    # encode the rounded magnitude
    qe = np.floor(np.log2(np.where(q > 0, q, 1.0)))
    normal = q >= 2.0 ** -6
    exp_field = np.where(normal, qe + 7, 0).astype(np.int64)
    mant = np.where(normal, q / 2.0 ** qe - 1.0, q / 2.0 ** -6) * 8.0
    code = (exp_field << 3) | np.rint(mant).astype(np.int64)
    code = np.where(np.signbit(v), code | 0x80, code)
    return code.astype(np.uint8)


def fp8_quantize(x_bits: np.ndarray):
    """bf16 rows [..., d] (uint16 bit patterns) -> (E4M3 codes uint8 [..., d], float32 scales [...])."""
    x32 = bf16_bits_to_f32(x_bits)
    scale = _row_scale(x32, E4M3_MAX)
    v = _scaled(x32, E4M3_MAX)
    return e4m3_encode(v), scale


def fp8_dequantize(codes: np.ndarray, scales: np.ndarray) -> np.ndarray:
    """(E4M3 codes, float32 scales) -> bf16 bit patterns of value * scale."""
    vals = e4m3_decode(codes).astype(np.float32)               # exact: 4 significant bits
    v = (vals * np.asarray(scales, np.float32)[..., None]).astype(np.float32)
    return bf16_bits_round(v)
