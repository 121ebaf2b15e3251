"""Storage formats used by the oracle: bfloat16, OCP FP8 E4M3FN and the OCP
microscaling FP4 format MXFP4 (E2M1 elements with an E8M0 scale per 32).

TEST INFRASTRUCTURE ONLY (see the package docstring).

Values are decoded from the bit fields of each format's definition by plain
arithmetic (sign, biased exponent, fraction), not by reinterpreting memory,
so that these decoders are independent of how the HIP library handles the
same bytes.  The fp8 encoder is a nearest-value search over the decoded code
table, again independent of any bit-manipulation encoder.

The FP8 row quantizer follows the low-precision indexer path: the pages
state that the Lightning Indexer's query-key path is quantized (FP4 QAT,
dequantized losslessly through FP8 E4M3) -- "DeepSeek V4 technical review"
(takeshell.com) section 5 "FP4 Quantization-Aware Training", and
dataforcee.us "Muon Optimizer and FP4 QAT".  The workload this build targets
stores indexer keys as E4M3 codes with one fp32 scale per row; the scale rule
(amax / 448, correctly rounded fp32 division, scale 1 for an all-zero row)
is this build's reading, since the pages give none.

MXFP4 is the pages' own precision for that path (the two sections above:
MXFP4 quantization-aware training of the indexer's query-key path, FP4
E2M1 dequantizing losslessly to FP8 E4M3).  The pages give no rules for the
format; these functions follow the public OCP Microscaling Formats (MX)
v1.0 definition: a block of 32 consecutive elements shares one E8M0 scale
X = 2^(floor(log2(amax)) - 2) (2 being the largest exponent of E2M1), and
each element is the E2M1 rounding (nearest, ties to even, saturating at 6)
of value / X.  An all-zero block gets scale code 0.  Storage: two codes per
byte, element 2i in the low nibble.
"""

from __future__ import annotations

import numpy as np

E4M3_MAX = 448.0


def bf16_decode(codes) -> np.ndarray:
    """Decode uint16 bfloat16 codes to float64.

    bfloat16: 1 sign bit, 8 exponent bits (bias 127), 7 fraction bits.
    Exponent 0 is subnormal (2^-126 * f/128); exponent 255 is inf/NaN.
    """
    c = np.asarray(codes).astype(np.int64)
    sign = np.where((c >> 15) & 1, -1.0, 1.0)
    e = (c >> 7) & 0xFF
    f = (c & 0x7F).astype(np.float64)
    normal = sign * np.ldexp(1.0 + f / 128.0, (e - 127).astype(np.int64))
    sub = sign * np.ldexp(f / 128.0, -126)
    out = np.where(e == 0, sub, normal)
    special = np.where(f == 0, sign * np.inf, np.nan)
    return np.where(e == 255, special, out)


def e4m3_decode(codes) -> np.ndarray:
    """Decode uint8 OCP FP8 E4M3FN codes to float64.

    E4M3FN: 1 sign bit, 4 exponent bits (bias 7), 3 fraction bits, no
    infinities; exponent 15 with fraction 7 is NaN, so the largest finite
    magnitude is 2^8 * 1.75 = 448.  Exponent 0 is subnormal: 2^-6 * f/8.
    """
    c = np.asarray(codes).astype(np.int64)
    sign = np.where((c >> 7) & 1, -1.0, 1.0)
    e = (c >> 3) & 0xF
    f = (c & 0x7).astype(np.float64)
    normal = sign * np.ldexp(1.0 + f / 8.0, (e - 7).astype(np.int64))
    sub = sign * np.ldexp(f / 8.0, -6)
    out = np.where(e == 0, sub, normal)
    return np.where((e == 15) & (f == 7), np.nan, out)


# Non-negative finite code table, ascending in value (codes 0x00..0x7E).
_POS_CODES = np.arange(0x7F, dtype=np.int64)
_POS_VALUES = e4m3_decode(_POS_CODES)
assert np.all(np.diff(_POS_VALUES) > 0)


def e4m3_encode(x) -> np.ndarray:
    """Round float values to E4M3FN codes: nearest value, ties to the code
    with an even fraction (the even code), magnitudes beyond 448 saturate to
    448.  The sign bit follows the sign of x, including -0.0 and negative
    values that round to zero.  NaN input is rejected.
    """
    v = np.asarray(x, dtype=np.float64)
    if np.isnan(v).any():
        raise ValueError("e4m3_encode: NaN input")
    neg = np.signbit(v)
    a = np.minimum(np.abs(v), E4M3_MAX)
    # index of the first table value >= a
    hi = np.searchsorted(_POS_VALUES, a, side="left")
    hi = np.minimum(hi, len(_POS_VALUES) - 1)
    lo = np.maximum(hi - 1, 0)
    d_hi = _POS_VALUES[hi] - a
    d_lo = a - _POS_VALUES[lo]
    pick_hi = (d_hi < d_lo) | ((d_hi == d_lo) & (_POS_CODES[hi] % 2 == 0))
    mag = np.where(pick_hi, _POS_CODES[hi], _POS_CODES[lo])
    mag = np.where(a == _POS_VALUES[hi], _POS_CODES[hi], mag)
    return (mag | np.where(neg, 0x80, 0)).astype(np.uint8)


def quantize_fp8_rows(x) -> tuple[np.ndarray, np.ndarray]:
    """Quantize each row of ``x`` (last axis) to E4M3 codes plus one fp32 scale.

    scale = amax(|row|) / 448 as a correctly rounded fp32 division (1.0 when
    the row is all zero); code = E4M3 rounding of the correctly rounded fp32
    quotient x / scale.  Both divisions are done in fp32 because the result
    is an integer code and the HIP library takes the same decision in fp32.
    Dequantized value = e4m3_decode(code) * scale.
    """
    xf = np.asarray(x, dtype=np.float32)
    amax = np.max(np.abs(xf), axis=-1)
    scale = np.where(amax > 0, amax / np.float32(E4M3_MAX), np.float32(1.0))
    scale = scale.astype(np.float32)
    q = (xf / scale[..., None]).astype(np.float32)
    return e4m3_encode(q.astype(np.float64)), scale


# ------------------------------------------------------------------ MXFP4

MX_BLOCK = 32
E2M1_MAX = 6.0


def e2m1_decode(codes) -> np.ndarray:
    """Decode 4-bit E2M1 codes (0..15) to float64.

    E2M1: 1 sign bit, 2 exponent bits (bias 1), 1 fraction bit, no
    infinities or NaN.  Exponent 0 is subnormal: 2^0 * f/2.
    """
    c = np.asarray(codes).astype(np.int64)
    sign = np.where((c >> 3) & 1, -1.0, 1.0)
    e = (c >> 1) & 0x3
    f = (c & 0x1).astype(np.float64)
    normal = sign * np.ldexp(1.0 + f / 2.0, (e - 1).astype(np.int64))
    sub = sign * (f / 2.0)
    return np.where(e == 0, sub, normal)


def e8m0_decode(codes) -> np.ndarray:
    """Decode E8M0 scale bytes to float64: 2^(code - 127); 255 is NaN."""
    c = np.asarray(codes).astype(np.int64)
    return np.where(c == 255, np.nan, np.ldexp(1.0, (np.minimum(c, 254) - 127).astype(np.int64)))


_E2M1_POS_CODES = np.arange(8, dtype=np.int64)
_E2M1_POS_VALUES = e2m1_decode(_E2M1_POS_CODES)
assert np.all(np.diff(_E2M1_POS_VALUES) > 0)


def e2m1_encode(x) -> np.ndarray:
    """Round float values to E2M1 codes: nearest value, ties to the even
    code, magnitudes beyond 6 saturate to 6; the sign bit follows the sign
    of x (also for -0.0 and negative values that round to zero)."""
    v = np.asarray(x, dtype=np.float64)
    if np.isnan(v).any():
        raise ValueError("e2m1_encode: NaN input")
    neg = np.signbit(v)
    a = np.minimum(np.abs(v), E2M1_MAX)
    hi = np.minimum(np.searchsorted(_E2M1_POS_VALUES, a, side="left"), 7)
    lo = np.maximum(hi - 1, 0)
    d_hi = _E2M1_POS_VALUES[hi] - a
    d_lo = a - _E2M1_POS_VALUES[lo]
    pick_hi = (d_hi < d_lo) | ((d_hi == d_lo) & (_E2M1_POS_CODES[hi] % 2 == 0))
    mag = np.where(pick_hi, _E2M1_POS_CODES[hi], _E2M1_POS_CODES[lo])
    mag = np.where(a == _E2M1_POS_VALUES[hi], _E2M1_POS_CODES[hi], mag)
    return (mag | np.where(neg, 8, 0)).astype(np.uint8)


def quantize_mxfp4_rows(x) -> tuple[np.ndarray, np.ndarray]:
    """Quantize each row of ``x`` (last axis, a multiple of 32 long) to MXFP4.

    Returns (codes, scales): codes uint8 [..., d/2] with element 2i in the
    low nibble of byte i and 2i+1 in the high nibble; scales uint8
    [..., d/32], E8M0 codes.  Per block of 32: amax = max |x|; scale
    exponent s = floor(log2(amax)) - 2 clamped to [-127, 127] (code s + 127),
    code 0 for an all-zero block; element code = e2m1_encode(x / 2^s), the
    quotient exact in float64.  Inputs are taken as float32 values.
    """
    xf = np.asarray(x, dtype=np.float32).astype(np.float64)
    d = xf.shape[-1]
    if d % MX_BLOCK:
        raise ValueError("row length must be a multiple of 32")
    blocks = xf.reshape(xf.shape[:-1] + (d // MX_BLOCK, MX_BLOCK))
    amax = np.max(np.abs(blocks), axis=-1)
    with np.errstate(divide="ignore"):
        s = np.floor(np.log2(np.where(amax > 0, amax, 1.0))) - 2
    s = np.clip(s, -127, 127).astype(np.int64)
    scale_codes = np.where(amax > 0, s + 127, 0)
    s_used = np.where(amax > 0, s, -127)
    q = np.ldexp(blocks, -s_used[..., None])
    codes = e2m1_encode(q).reshape(xf.shape).astype(np.int64)
    packed = (codes[..., 0::2] | (codes[..., 1::2] << 4)).astype(np.uint8)
    return packed, scale_codes.astype(np.uint8)


def mxfp4_decode_rows(codes, scales) -> np.ndarray:
    """Dequantize MXFP4 rows: codes uint8 [..., d/2] (low nibble first),
    scales uint8 [..., d/32] -> float64 [..., d]."""
    c = np.asarray(codes).astype(np.int64)
    nib = np.stack([c & 0xF, c >> 4], axis=-1).reshape(c.shape[:-1] + (2 * c.shape[-1],))
    vals = e2m1_decode(nib)
    sc = e8m0_decode(np.asarray(scales))
    d = vals.shape[-1]
    return (vals.reshape(vals.shape[:-1] + (d // MX_BLOCK, MX_BLOCK)) * sc[..., None]).reshape(vals.shape)
