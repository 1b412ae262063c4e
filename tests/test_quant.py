"""8-bit exchange formats: INT8 for Q/K/V and FP8 (OCP E4M3) for the attention output,
one float32 scale per token row ("Videomodel MiniMax-H3 rendert sneller dan afspelen",
section "Waar de snelheidswinst vandaan komt": the traffic between the GPUs goes in
INT8 for QKV and FP8 for the output).

CPU: the oracle is pinned to the E4M3 format definition (hand-decoded codes), to torch's
own float8_e4m3fn conversion (a library routine computing the same rounding), to exactly
representable INT8 cases with ties, and to the error bounds of the formats."""
import math

import numpy as np
import pytest
import torch

from oracle import quant_oracle as Qo


def _bits(x):
    return Qo.bf16_bits_round(np.asarray(x, dtype=np.float32))


# ----------------------------------------------------------------------------- E4M3 format
def test_e4m3_decode_hand_values():
    table = {0x00: 0.0, 0x01: 2.0 ** -9, 0x07: 7 * 2.0 ** -9, 0x08: 2.0 ** -6, 0x0F: 1.875 * 2.0 ** -6,
             0x38: 1.0, 0x3C: 1.5, 0x40: 2.0, 0x47: 3.75, 0x78: 256.0, 0x7E: 448.0,
             0x80: -0.0, 0xB8: -1.0, 0xFE: -448.0}
    for c, v in table.items():
        got = Qo.e4m3_decode(np.array([c], np.uint8))[0]
        assert got == v and np.signbit(got) == np.signbit(v), hex(c)
    assert np.isnan(Qo.e4m3_decode(np.array([0x7F, 0xFF], np.uint8))).all()


def test_e4m3_every_finite_code_round_trips():
    codes = np.array([c for c in range(256) if c & 0x7F != 0x7F], np.uint8)
    vals = Qo.e4m3_decode(codes).astype(np.float32)
    assert np.array_equal(Qo.e4m3_encode(vals), codes)
    pos = np.sort(Qo.e4m3_decode(np.arange(0, 0x7F, dtype=np.uint8)))
    assert np.all(np.diff(pos) > 0) and pos[-1] == 448.0          # 127 distinct, ordered magnitudes


def test_e4m3_midpoints_round_to_even_and_saturate():
    pos = Qo.e4m3_decode(np.arange(0, 0x7F, dtype=np.uint8))
    mids = ((pos[:-1] + pos[1:]) / 2).astype(np.float32)
    assert np.array_equal(mids.astype(np.float64), (pos[:-1] + pos[1:]) / 2)    # exact in float32
    got = Qo.e4m3_encode(mids)
    lo = np.arange(0, 0x7E)
    want = np.where(lo % 2 == 0, lo, lo + 1)                      # the even code of the two neighbours
    assert np.array_equal(got, want.astype(np.uint8))
    assert Qo.e4m3_encode(np.float32([500.0, -1e6]))[0] == 0x7E
    assert Qo.e4m3_encode(np.float32([500.0, -1e6]))[1] == 0xFE


def test_e4m3_encode_equals_torch_float8_e4m3fn():
    rng = np.random.default_rng(0)
    v = np.concatenate([rng.standard_normal(200000) * s for s in (1e-3, 0.05, 1, 30, 150)]).astype(np.float32)
    v = np.clip(v, -448, 448)
    ours = Qo.e4m3_encode(v)
    ref = torch.from_numpy(v).to(torch.float8_e4m3fn).view(torch.uint8).numpy()
    assert np.array_equal(ours, ref)


# ----------------------------------------------------------------------------- INT8
def test_int8_unit_scale_rounds_half_even():
    x = _bits([[127.0, -3.5, 2.5, 0.5, 1.5, -0.5, 0.25, -127.0]])   # amax 127 -> scale exactly 1
    codes, scale = Qo.int8_quantize(x)
    assert scale[0] == 1.0
    assert codes[0].tolist() == [127, -4, 2, 0, 2, 0, 0, -127]


def test_int8_extremes_and_zero_rows():
    rng = np.random.default_rng(1)
    x = _bits(rng.standard_normal((64, 128)) * rng.uniform(0.01, 10, (64, 1)))
    x[5] = 0
    codes, scale = Qo.int8_quantize(x)
    assert scale[5] == 0 and not codes[5].any()
    rows = np.delete(np.arange(64), 5)
    assert np.all(np.abs(codes[rows]).max(axis=1) == 127)           # the row maximum maps to +-127
    xf = Qo.bf16_bits_to_f32(x)
    assert np.array_equal(np.sign(codes[np.abs(codes) > 0]), np.sign(xf[np.abs(codes) > 0]))


def test_int8_round_trip_error_bound():
    rng = np.random.default_rng(2)
    x = _bits(rng.standard_normal((256, 128)) * 3)
    codes, scale = Qo.int8_quantize(x)
    back = Qo.bf16_bits_to_f32(Qo.int8_dequantize(codes, scale)).astype(np.float64)
    xf = Qo.bf16_bits_to_f32(x).astype(np.float64)
    # half a quantisation step, plus the bf16 rounding of the decoded value (2^-9 relative)
    bound = scale[:, None] / 2 * (1 + 1e-6) + np.abs(back) * 2.0 ** -8
    assert np.all(np.abs(back - xf) <= bound)


def test_int8_dequantize_is_code_times_scale():
    codes = np.array([[1, -2, 127, 0]], np.int8)
    scale = np.float32([0.5])
    assert Qo.bf16_bits_to_f32(Qo.int8_dequantize(codes, scale))[0].tolist() == [0.5, -1.0, 63.5, 0.0]


# ----------------------------------------------------------------------------- FP8 rows
def test_fp8_row_maximum_maps_to_448_and_relative_error():
    rng = np.random.default_rng(3)
    x = _bits(rng.standard_normal((128, 128)) * rng.uniform(0.01, 10, (128, 1)))
    codes, scale = Qo.fp8_quantize(x)
    assert np.all(np.max(codes & 0x7F, axis=1) == 0x7E)
    xf = Qo.bf16_bits_to_f32(x).astype(np.float64)
    back = Qo.bf16_bits_to_f32(Qo.fp8_dequantize(codes, scale)).astype(np.float64)
    # E4M3 normal range: relative error <= 2^-4; subnormal part: absolute <= 2^-10 * scale
    err = np.abs(back - xf)
    bound = np.maximum(np.abs(xf) * (2.0 ** -4 + 2.0 ** -8), scale[:, None] * 2.0 ** -10 * 1.01)
    assert np.all(err <= bound * 1.0001)


def test_fp8_zero_row_and_unit_scale():
    x = _bits([[0.0] * 8, [448.0, -1.0, 0.3, 2.0 ** -9, 3.3, -448.0, 17.0, 0.0]])
    codes, scale = Qo.fp8_quantize(x)
    assert scale[0] == 0 and not codes[0].any()
    assert scale[1] == 1.0
    want = Qo.e4m3_encode(Qo.bf16_bits_to_f32(x[1]))
    assert np.array_equal(codes[1], want)
    assert codes[1][0] == 0x7E and codes[1][5] == 0xFE and codes[1][1] == 0xB8


def test_size_ratio_is_51_6_percent_at_d128():
    d = 128
    assert abs((d + 4) / (2 * d) - 0.516) < 5e-4


# ----------------------------------------------------------------------------- GPU parity
def _gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    from block_sparse_attention_attn_amd import sol_attn
    sol_attn.load_library()
    return sol_attn


def _dev_bf16(bits):
    return torch.from_numpy(np.ascontiguousarray(bits).view(np.int16)).view(torch.bfloat16).cuda()


def _every_bf16_up_to(limit, d):
    """Rows [n, d] holding every bf16 value in [-limit, limit] (both zeros included), each
    row also holding +limit so that its scale makes x * (qmax / amax) == x exactly."""
    allbits = np.arange(1 << 16, dtype=np.uint32).astype(np.uint16)
    vals = Qo.bf16_bits_to_f32(allbits)
    keep = allbits[np.isfinite(vals) & (np.abs(vals) <= limit)]
    per = d - 1
    n = -(-keep.size // per)
    body = np.resize(keep, n * per).reshape(n, per)
    lim = Qo.bf16_bits_round(np.float32([limit]))[0]
    return np.concatenate([np.full((n, 1), lim, np.uint16), body], axis=1)


@pytest.mark.gpu
@pytest.mark.parametrize("fmt", [0, 1])
def test_codes_exhaustive_over_bf16_values(fmt):
    """Unit scale (row maximum 127 or 448): every bf16 value in range is coded exactly as
    the oracle codes it -- ties, subnormal E4M3 steps, signed zeros."""
    S = _gpu()
    limit = 127.0 if fmt == 0 else 448.0
    rows = _every_bf16_up_to(limit, 128)
    x = rows.reshape(1, 1, *rows.shape)
    codes, scales = S.sol_attn_quantize(_dev_bf16(x), fmt)
    torch.cuda.synchronize()
    want_codes, want_scales = (Qo.int8_quantize if fmt == 0 else Qo.fp8_quantize)(x)
    assert np.all(want_scales == 1.0)
    assert np.array_equal(codes.cpu().numpy().view(np.uint8), want_codes.view(np.uint8))
    assert np.array_equal(scales.cpu().numpy(), want_scales)


@pytest.mark.gpu
@pytest.mark.parametrize("d", [8, 64, 128, 136, 512])
@pytest.mark.parametrize("fmt", [0, 1])
def test_quantize_dequantize_match_oracle(fmt, d):
    S = _gpu()
    rng = np.random.default_rng(d + fmt)
    B, H, L = 2, 3, 37                                  # 222 rows: a ragged last workgroup
    x = rng.standard_normal((B, H, L, d)) * rng.uniform(1e-3, 50, (B, H, L, 1))
    x[0, 0, 3] = 0.0                                    # a row of zeros
    x[1, 2, 5, : d // 2] = -0.0
    x[1, 2, 5, d // 2:] = 0.0                           # a row of signed zeros
    x[0, 1, 7, 0] = -0.0                                # a negative zero in an ordinary row
    bits = Qo.bf16_bits_round(x.astype(np.float32))
    codes, scales = S.sol_attn_quantize(_dev_bf16(bits), fmt)
    torch.cuda.synchronize()
    q, dq = (Qo.int8_quantize, Qo.int8_dequantize) if fmt == 0 else (Qo.fp8_quantize, Qo.fp8_dequantize)
    want_codes, want_scales = q(bits)
    got_codes = codes.cpu().numpy()
    assert np.array_equal(got_codes.view(np.uint8), want_codes.view(np.uint8))
    assert np.array_equal(scales.cpu().numpy(), want_scales)
    out = S.sol_attn_dequantize(codes, scales, fmt)
    torch.cuda.synchronize()
    assert np.array_equal(out.cpu().view(torch.int16).numpy().view(np.uint16),
                          dq(want_codes, want_scales))


@pytest.mark.gpu
@pytest.mark.parametrize("fmt", [0, 1])
def test_dequantize_every_code(fmt):
    """Every code byte (E4M3 without its two NaN codes) decodes as the oracle decodes it."""
    S = _gpu()
    codes = np.array([c for c in range(256) if fmt == 0 or (c & 0x7F) != 0x7F], np.uint8)
    codes = np.resize(codes, 8 * 256).reshape(1, 1, 8, 256)
    scales = np.float32([[[1.0, 0.5, 3.0, 1e-3, 7.25, 0.0, 2.0 ** -20, 1234.5]]])
    out = S.sol_attn_dequantize(torch.from_numpy(codes).cuda(), torch.from_numpy(scales).cuda(), fmt)
    torch.cuda.synchronize()
    c = codes.view(np.int8) if fmt == 0 else codes
    want = (Qo.int8_dequantize if fmt == 0 else Qo.fp8_dequantize)(c, scales)
    assert np.array_equal(out.cpu().view(torch.int16).numpy().view(np.uint16), want)


@pytest.mark.gpu
@pytest.mark.timeout(600)
def test_quantize_full_size_sampled_rows():
    """1344x768 workload Q (40 heads x 64,512 tokens): INT8 and FP8 codes and scales of
    sampled rows equal the oracle's, and decoding matches on those rows."""
    from block_sparse_attention_attn_amd import workloads as W
    S = _gpu()
    wl = W.get("refine_1344x768")
    q, _, _ = W.make_qkv(wl)
    X = _dev_bf16(q)
    rows = np.random.default_rng(11).choice(wl.B * wl.H * wl.L, 4096, replace=False)
    flat = q.reshape(-1, wl.d)[rows]
    for fmt, (qf, dqf) in enumerate(((Qo.int8_quantize, Qo.int8_dequantize), (Qo.fp8_quantize, Qo.fp8_dequantize))):
        codes, scales = S.sol_attn_quantize(X, fmt)
        out = S.sol_attn_dequantize(codes, scales, fmt)
        torch.cuda.synchronize()
        wc, ws = qf(flat)
        idx = torch.from_numpy(rows)
        assert np.array_equal(codes.view(-1, wl.d)[idx.cuda()].cpu().numpy().view(np.uint8), wc.view(np.uint8))
        assert np.array_equal(scales.view(-1)[idx.cuda()].cpu().numpy(), ws)
        assert np.array_equal(out.view(-1, wl.d)[idx.cuda()].cpu().view(torch.int16).numpy().view(np.uint16),
                              dqf(wc, ws))
