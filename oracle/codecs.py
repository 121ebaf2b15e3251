"""Storage formats used by the oracle: bfloat16 and OCP FP8 E4M3FN.

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
