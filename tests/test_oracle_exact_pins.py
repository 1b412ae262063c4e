"""Pins of oracle parts whose correctness is a statement about rounding, checked against
exact rational arithmetic (fractions.Fraction) and against torch's own conversions,
never against the GPU kernels:

* the 8-bit coding step (oracle/quant_oracle.py): the code of x is x times the per-row
  multiplier qmax/amax, each float32 rounding applied explicitly to exact rationals;
  a second test shows that this reading and division by the stored scale give
  different codes on real rows, so the pin tells the two apart;
* the selection-margin certificate (oracle.selection_margins): its rounding bound
  holds against exact scores, and its ambiguity threshold sits where the bound says
  (a constant off by a factor of 8 either way fails);
* oracle.widen for bf16 and quant_oracle.bf16_bits_round against torch.bfloat16.
"""
from fractions import Fraction

import numpy as np
import pytest
import torch

import oracle
from oracle import quant_oracle as Qo


# ----------------------------------------------------------------------------- exact helpers
def _floor_log2(x: Fraction) -> int:
    """floor(log2(x)) for a positive rational, exactly."""
    n, d = x.numerator, x.denominator
    e = n.bit_length() - d.bit_length()
    if Fraction(2) ** e > x:
        e -= 1
    return e


def _rne_int(x: Fraction) -> int:
    """Round a rational to the nearest integer, ties to even."""
    f = x.numerator // x.denominator          # floor
    r = x - f
    if r > Fraction(1, 2) or (r == Fraction(1, 2) and f % 2 == 1):
        return f + 1
    return f


def _to_f32(x: Fraction) -> Fraction:
    """Nearest IEEE binary32 value (ties to even), subnormals included; no overflow here."""
    if x == 0:
        return Fraction(0)
    s = -1 if x < 0 else 1
    a = abs(x)
    e = max(_floor_log2(a), -126)
    ulp = Fraction(2) ** (e - 23)
    return s * _rne_int(a / ulp) * ulp


def _f32_exact(v) -> Fraction:
    return Fraction(float(np.float32(v)))


# ----------------------------------------------------------------------------- 8-bit coding step
def _rows(seed, n=64, d=128):
    """bf16 rows whose maxima are not powers of two (the multiplier is then inexact)."""
    rng = np.random.default_rng(seed)
    x = rng.standard_normal((n, d)) * rng.uniform(0.003, 40.0, (n, 1))
    return Qo.bf16_bits_round(x.astype(np.float32))


def _int8_codes_exact(row_f32, reading):
    amax = max(abs(_f32_exact(v)) for v in row_f32)
    if amax == 0:
        return [0] * len(row_f32)
    if reading == "multiplier":            # x * fl(127 / amax)
        inv = _to_f32(Fraction(127) / amax)
        vals = [_to_f32(_f32_exact(v) * inv) for v in row_f32]
    else:                                  # x / fl(amax / 127), the stored scale
        scale = _to_f32(amax / 127)
        vals = [_to_f32(_f32_exact(v) / scale) for v in row_f32]
    return [max(-127, min(127, _rne_int(v))) for v in vals]


def test_int8_codes_equal_exact_multiplier_reading():
    """Every code of 64 rows at non-unit scales equals round-half-even of
    fl32(x * fl32(127/amax)) computed in exact rationals; the stored scale is fl32(amax/127)."""
    bits = _rows(11)
    codes, scale = Qo.int8_quantize(bits)
    xf = Qo.bf16_bits_to_f32(bits)
    for r in range(bits.shape[0]):
        assert codes[r].tolist() == _int8_codes_exact(xf[r], "multiplier"), r
        amax = max(abs(_f32_exact(v)) for v in xf[r])
        assert Fraction(float(scale[r])) == _to_f32(amax / 127)


def test_int8_multiplier_and_division_readings_differ():
    """The two rounding orders the page leaves open give different codes on ordinary rows,
    so the previous test pins the reading taken, not just the format."""
    bits = _rows(12, n=256)
    xf = Qo.bf16_bits_to_f32(bits)
    differ = sum(_int8_codes_exact(xf[r], "multiplier") != _int8_codes_exact(xf[r], "division")
                 for r in range(bits.shape[0]))
    assert differ > 0
    codes, _ = Qo.int8_quantize(bits)
    div_rows = [r for r in range(bits.shape[0])
                if _int8_codes_exact(xf[r], "multiplier") != _int8_codes_exact(xf[r], "division")]
    for r in div_rows:     # the oracle takes the multiplier reading on exactly those rows too
        assert codes[r].tolist() == _int8_codes_exact(xf[r], "multiplier")


def _e4m3_table():
    """(value, code) of the 127 non-negative finite E4M3 codes, from the decoder that the
    hand-decoded table in tests/test_quant.py pins."""
    codes = np.arange(0, 0x7F, dtype=np.uint8)
    return [(Fraction(float(v)), int(c)) for v, c in zip(Qo.e4m3_decode(codes), codes)]


def _e4m3_nearest(v: Fraction, table):
    """Nearest E4M3 value to v by brute force over the table, ties to the even code,
    magnitudes above 448 saturated."""
    a = min(abs(v), Fraction(448))
    best = min(table, key=lambda t: (abs(t[0] - a), t[1] % 2))
    return best[0] if v >= 0 else -best[0]


def test_fp8_codes_equal_exact_multiplier_reading():
    """FP8 codes decode to the E4M3 value nearest (ties to even) to fl32(x * fl32(448/amax)),
    found by brute force over the format's values in exact rationals."""
    table = _e4m3_table()
    bits = _rows(13, n=24)
    codes, scale = Qo.fp8_quantize(bits)
    xf = Qo.bf16_bits_to_f32(bits)
    dec = Qo.e4m3_decode(codes)
    for r in range(bits.shape[0]):
        amax = max(abs(_f32_exact(v)) for v in xf[r])
        inv = _to_f32(Fraction(448) / amax)
        assert Fraction(float(scale[r])) == _to_f32(amax / 448)
        for e in range(bits.shape[1]):
            want = _e4m3_nearest(_to_f32(_f32_exact(xf[r, e]) * inv), table)
            assert Fraction(float(dec[r, e])) == want, (r, e)


def test_fp8_multiplier_and_division_readings_differ():
    table = _e4m3_table()
    xf = Qo.bf16_bits_to_f32(_rows(14, n=48))
    differ = 0
    for r in range(xf.shape[0]):
        amax = max(abs(_f32_exact(v)) for v in xf[r])
        inv, scale = _to_f32(Fraction(448) / amax), _to_f32(amax / 448)
        for v in xf[r]:
            a = _e4m3_nearest(_to_f32(_f32_exact(v) * inv), table)
            b = _e4m3_nearest(_to_f32(_f32_exact(v) / scale), table)
            differ += a != b
    assert differ > 0


# ----------------------------------------------------------------------------- margin certificate
def _exact_scores(Qb, Kb):
    return [[sum(Fraction(float(a)) * Fraction(float(b)) for a, b in zip(q, k)) for k in Kb] for q in Qb]


def test_margin_rounding_bound_holds_against_exact_scores():
    """|float64 score - exact score| <= gamma_d * sum_e |Qbar_ie Kbar_je| for every pair:
    the per-score bound the certificate doubles when it compares two scores."""
    rng = np.random.default_rng(21)
    d = 64
    Qb = rng.standard_normal((6, d)) * 3
    Kb = rng.standard_normal((40, d)) * 3
    Kb[7] = -Kb[3] + 1e-9                       # heavy cancellation against row 3
    r = oracle.block_scores(Qb, Kb)
    ex = _exact_scores(Qb, Kb)
    u = Fraction(1, 2 ** 53)
    gamma = d * u / (1 - d * u)
    for i in range(Qb.shape[0]):
        for j in range(Kb.shape[0]):
            mag = sum(abs(Fraction(float(a)) * Fraction(float(b))) for a, b in zip(Qb[i], Kb[j]))
            assert abs(Fraction(float(r[i, j])) - ex[i][j]) <= gamma * mag


@pytest.mark.parametrize("gap_exp,ambiguous", [(-27, 0), (-33, 1)])
def test_margin_ambiguity_threshold_constructed(gap_exp, ambiguous):
    """Query row (1, 1) against key rows (A, -A + g): the exact score is g while
    sum |Qbar||Kbar| is about 2A, so the certificate's bound is about 8 u A = 2^-30 at
    A = 2^20.  A k-th/(k+1)-th gap of 2^-27 (8x the bound) is certified and one of 2^-33
    (1/8 of it) is reported ambiguous; a bound constant off by 8x either way fails."""
    A = 2.0 ** 20
    g_hi, g_lo = 2.0 ** -20, 2.0 ** -20 - 2.0 ** gap_exp
    Qb = np.array([[1.0, 1.0]])
    Kb = np.array([[A, -A + g_hi], [A, -A + g_lo], [A, -A - 1.0], [0.5, 0.25]])
    ex = _exact_scores(Qb, Kb)[0]
    assert ex[0] == Fraction(g_hi) and ex[1] == Fraction(g_lo)       # the construction is exact
    # scores g_hi, g_lo, -1, 0.75: descending 0.75, g_hi, g_lo, -1
    rel, amb, ties = oracle.selection_margins(Qb, Kb, 3)              # compares g_lo with -1
    assert amb == 0 and ties == 0
    rel, amb, ties = oracle.selection_margins(Qb, Kb, 2)              # compares g_hi with g_lo
    assert ties == 0 and amb == ambiguous
    assert rel == (g_hi - g_lo) / g_hi


def test_margin_exact_tie_counted_not_ambiguous():
    Qb = np.array([[1.0, 1.0]])
    Kb = np.array([[2.0 ** 20, -2.0 ** 20 + 1.0], [3.0, -2.0], [0.0, 0.0]])
    rel, amb, ties = oracle.selection_margins(Qb, Kb, 1)
    assert ties == 1 and amb == 0


# ----------------------------------------------------------------------------- bf16 conversions
@pytest.mark.filterwarnings("ignore::RuntimeWarning")
def test_widen_bf16_equals_torch_for_every_pattern():
    bits = np.arange(1 << 16, dtype=np.uint32).astype(np.uint16)
    ours = oracle.widen(bits, "bf16")
    ref = torch.from_numpy(bits.view(np.int16)).view(torch.bfloat16).double().numpy()
    fin = np.isfinite(ref)
    assert np.array_equal(ours[fin], ref[fin])
    assert np.array_equal(np.signbit(ours[fin]), np.signbit(ref[fin]))     # -0.0 stays negative
    assert np.array_equal(np.isnan(ours), np.isnan(ref))
    assert np.array_equal(np.isinf(ours), np.isinf(ref))


def test_bf16_bits_round_equals_torch_including_ties():
    rng = np.random.default_rng(31)
    hi = rng.integers(0, 0x7F7F, 200000, dtype=np.uint32)          # finite, below the overflow edge
    lo = rng.integers(0, 1 << 16, 200000, dtype=np.uint32)
    lo[:50000] = 0x8000                                              # exact ties, even and odd upper halves
    lo[50000:60000] = 0x7FFF
    lo[60000:70000] = 0x8001
    u = (hi << 16) | lo
    sign = (rng.integers(0, 2, u.size, dtype=np.uint32) << 31)
    x = (u | sign).view(np.float32)
    ours = Qo.bf16_bits_round(x)
    ref = torch.from_numpy(x).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    assert np.array_equal(ours, ref)
