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
