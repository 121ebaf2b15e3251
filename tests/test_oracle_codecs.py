"""Pins of the oracle's storage codecs against the format definitions and
against independent library conversions (NumPy bit reinterpretation for
bfloat16, PyTorch's float8_e4m3fn for E4M3)."""

import numpy as np
import pytest
import torch

from oracle import bf16_decode, e4m3_decode, e4m3_encode, quantize_fp8_rows


def test_bf16_decode_all_codes_match_bit_reinterpretation():
    codes = np.arange(1 << 16, dtype=np.uint32)
    ref = (codes << 16).astype(np.uint32).view(np.float32)
    with np.errstate(invalid="ignore"):
        ref = ref.astype(np.float64)
    got = bf16_decode(codes.astype(np.uint16))
    nan = np.isnan(ref)
    assert np.array_equal(np.isnan(got), nan)
    assert np.array_equal(got[~nan], ref[~nan])
    # sign of zero is kept
    assert np.signbit(got[0x8000]) and not np.signbit(got[0])


def test_e4m3_decode_all_codes_match_torch():
    codes = torch.arange(256, dtype=torch.int16).to(torch.uint8)
    ref = codes.view(torch.float8_e4m3fn).to(torch.float64).numpy()
    got = e4m3_decode(np.arange(256))
    nan = np.isnan(ref)
    assert nan.sum() == 2 and np.array_equal(np.isnan(got), nan)
    assert np.array_equal(got[~nan], ref[~nan])


def test_e4m3_encode_matches_torch_rounding():
    rng = np.random.default_rng(7)
    # random magnitudes over the whole range, including subnormals, and all
    # exact midpoints between neighbouring finite codes (the tie rule)
    vals = e4m3_decode(np.arange(0x7F))
    mids = (vals[:-1] + vals[1:]) / 2
    x = np.concatenate([
        rng.uniform(-460, 460, 20000),
        rng.uniform(-0.02, 0.02, 5000),
        mids, -mids, vals, -vals,
        np.exp(rng.uniform(np.log(1e-4), np.log(460), 5000)),
    ]).astype(np.float32)
    ref = torch.from_numpy(x).to(torch.float8_e4m3fn).view(torch.uint8).numpy()
    got = e4m3_encode(x.astype(np.float64))
    assert np.array_equal(got, ref)


def test_e4m3_encode_saturates_and_keeps_sign():
    got = e4m3_encode(np.array([465.0, 1e6, -1e6, -0.0, -1e-9]))
    assert list(got) == [0x7E, 0x7E, 0xFE, 0x80, 0x80]
    with pytest.raises(ValueError):
        e4m3_encode(np.array([np.nan]))


def test_codec_golden(load_golden):
    g = load_golden("codecs.json")
    for code, val in g["bf16"]:
        assert bf16_decode(np.array([code]))[0] == val
    for code, val in g["e4m3_decode"]:
        assert e4m3_decode(np.array([code]))[0] == val
    assert np.isnan(e4m3_decode(np.array([g["e4m3_nan_code"]]))[0])
    for val, code in g["e4m3_encode"]:
        assert e4m3_encode(np.array([val]))[0] == code
    codes, scale = quantize_fp8_rows(np.array([g["quant_row"]], dtype=np.float32))
    assert list(codes[0]) == g["quant_codes"]
    assert scale[0] == np.float32(2.0) / np.float32(448.0)


def test_quantizer_is_idempotent_on_representable_rows():
    """A row whose values are e4m3 values times a power of two, with the
    largest magnitude exactly 448 * 2^e, quantizes back to the same codes
    and scale 2^e (every division involved is exact)."""
    rng = np.random.default_rng(3)
    for e in (-10, -3, 0, 4):
        codes = rng.integers(0, 0x7F, size=(50, 128)).astype(np.uint8)
        codes[:, 5] = 0x7E  # make 448 the row maximum
        codes |= (rng.integers(0, 2, size=codes.shape) * 0x80).astype(np.uint8)
        x = (e4m3_decode(codes) * 2.0 ** e).astype(np.float32)
        got_codes, got_scale = quantize_fp8_rows(x)
        assert np.all(got_scale == np.float32(2.0 ** e))
        # -0 codes quantize to -0: compare decoded values and sign bits
        assert np.array_equal(got_codes, codes)


def test_quantizer_zero_row_and_error_bound():
    codes, scale = quantize_fp8_rows(np.zeros((1, 16), dtype=np.float32))
    assert scale[0] == 1.0 and not codes.any()
    rng = np.random.default_rng(11)
    x = rng.standard_normal((200, 128)).astype(np.float32)
    codes, scale = quantize_fp8_rows(x)
    deq = e4m3_decode(codes) * scale[:, None].astype(np.float64)
    # e4m3 keeps 3 fraction bits: relative rounding error <= 2^-4 for normal
    # values, absolute error <= half the subnormal step (2^-10) * scale
    err = np.abs(deq - x)
    bound = np.maximum(np.abs(x) * 2.0 ** -4, 2.0 ** -10 * scale[:, None]) * (1 + 1e-6)
    assert np.all(err <= bound)
    assert np.all(np.abs(e4m3_decode(codes)).max(axis=1) == 448.0)


# ------------------------------------------------------------------ MXFP4
#
# torch has no FP4 arithmetic, so the E2M1 codec is pinned through a generic
# minifloat definition (sign, biased exponent, fraction, subnormals at
# exponent 0) that is itself checked against torch's E4M3 and E5M2 on every
# finite code; E2M1 is that definition with 2 exponent bits, 1 fraction bit
# and bias 1.  E8M0 decoding is checked against torch directly.

from oracle import (e2m1_decode, e2m1_encode, e8m0_decode, mxfp4_decode_rows,
                    quantize_mxfp4_rows)


def _minifloat_values(e_bits, m_bits, bias):
    """Every non-negative value of a minifloat without specials, by code."""
    out = []
    for code in range(1 << (e_bits + m_bits)):
        e, f = code >> m_bits, code & ((1 << m_bits) - 1)
        if e == 0:
            out.append(2.0 ** (1 - bias) * f / (1 << m_bits))
        else:
            out.append(2.0 ** (e - bias) * (1 + f / (1 << m_bits)))
    return np.array(out)


def _minifloat_round(x, values):
    """Nearest of the ascending ``values``, ties to the even code, saturating."""
    a = np.minimum(np.abs(x), values[-1])
    codes = np.empty(a.shape, np.int64)
    for i, v in enumerate(a):
        d = np.abs(values - v)
        best = np.flatnonzero(d == d.min())
        codes[i] = best[0] if len(best) == 1 else best[best % 2 == 0][0]
    return codes


def test_generic_minifloat_matches_torch_fp8_formats():
    for dt, e_bits, m_bits, bias in ((torch.float8_e4m3fn, 4, 3, 7), (torch.float8_e5m2, 5, 2, 15)):
        vals = _minifloat_values(e_bits, m_bits, bias)
        ref = torch.arange(1 << (e_bits + m_bits), dtype=torch.int16).to(torch.uint8).view(dt)
        ref = ref.to(torch.float64).numpy()
        finite = np.isfinite(ref)
        assert np.array_equal(vals[finite], ref[finite]), dt


def test_e2m1_decode_is_the_minifloat_definition():
    vals = _minifloat_values(2, 1, 1)
    assert np.array_equal(e2m1_decode(np.arange(8)), vals)
    assert np.array_equal(e2m1_decode(np.arange(8, 16)), -vals)
    assert vals.max() == 6.0


def test_e2m1_encode_nearest_even_and_saturating():
    vals = _minifloat_values(2, 1, 1)
    rng = np.random.default_rng(11)
    mids = (vals[:-1] + vals[1:]) / 2
    x = np.concatenate([rng.uniform(-7, 7, 4000), mids, -mids, vals, -vals,
                        [6.5, 100.0, -1e9, 0.0]])
    got = e2m1_encode(x)
    want = _minifloat_round(x, vals) | np.where(np.signbit(x), 8, 0)
    assert np.array_equal(got, want)
    assert list(e2m1_encode(np.array([-0.0, -0.1, 0.25, 0.75, 5.0]))) == [8, 8, 0, 2, 6]


def test_e8m0_decode_all_codes_match_torch():
    ref = torch.arange(256, dtype=torch.int16).to(torch.uint8).view(torch.float8_e8m0fnu)
    ref = ref.to(torch.float64).numpy()
    got = e8m0_decode(np.arange(256))
    assert np.isnan(got[255]) and np.isnan(ref[255])
    assert np.array_equal(got[:255], ref[:255])


def test_fp4_to_fp8_is_lossless():
    # the pages: FP4 (E2M1) dequantizes to FP8 (E4M3) without loss -- every
    # E2M1 value is an E4M3 value, so an E2M1 code survives the round trip
    vals = e2m1_decode(np.arange(16))
    assert np.array_equal(e4m3_decode(e4m3_encode(vals)), vals)


def test_mxfp4_quantizer_hand_worked_block():
    # amax 6 -> floor(log2 6) - 2 = 0 -> scale code 127 (X = 1); codes
    # 1.0 -> 2, -0.5 -> 9, 6.0 -> 7, 3.0 -> 5, 0 -> 0; packed low nibble first
    row = np.zeros(32)
    row[:4] = [1.0, -0.5, 6.0, 3.0]
    codes, scales = quantize_mxfp4_rows(row[None])
    assert list(codes[0, :3]) == [0x92, 0x57, 0x00] and list(scales[0]) == [127]
    # amax 0.3 -> floor(log2 0.3) - 2 = -4 (X = 1/16): 0.3 * 16 = 4.8 -> 4.0
    row = np.zeros(32)
    row[5] = -0.3
    codes, scales = quantize_mxfp4_rows(row[None])
    assert scales[0, 0] == 123 and codes[0, 2] == 0xE0 and mxfp4_decode_rows(codes, scales)[0, 5] == -0.25


def test_mxfp4_quantizer_scale_rule_error_bound_and_idempotence():
    rng = np.random.default_rng(12)
    x = (rng.standard_normal((64, 128)) * np.exp(rng.uniform(-20, 20, (64, 1)))).astype(np.float32)
    x[0, :32] = 0.0                      # an all-zero block
    codes, scales = quantize_mxfp4_rows(x)
    assert codes.shape == (64, 64) and scales.shape == (64, 4)
    blocks = x.astype(np.float64).reshape(64, 4, 32)
    amax = np.abs(blocks).max(-1)
    X = e8m0_decode(scales)
    nz = amax > 0
    assert np.all((amax[nz] / X[nz] >= 4) & (amax[nz] / X[nz] < 8))
    assert scales[0, 0] == 0 and np.all(codes[0, :16] == 0)
    deq = mxfp4_decode_rows(codes, scales).reshape(64, 4, 32)
    # half the local E2M1 spacing: 0.5 X below 4 X, X up to 6 X; past 6 X
    # the value saturates to 6 X, and x < 8 X bounds that error by 2 X
    err = np.abs(deq - blocks)
    Xb = X[..., None].repeat(32, -1)
    a = np.abs(blocks)
    assert np.all(err <= 2 * Xb)
    assert np.all(err[a <= 6 * Xb] <= Xb[a <= 6 * Xb])
    assert np.all(err[a < 4 * Xb] <= 0.5 * Xb[a < 4 * Xb])
    # dequantized blocks are representable: quantizing them again is exact
    codes2, scales2 = quantize_mxfp4_rows(deq.reshape(64, 128))
    assert np.array_equal(mxfp4_decode_rows(codes2, scales2), deq.reshape(64, 128))
