"""OCP FP8 E4M3FN codec, written from the format's definition.

The pages fix only that an FP8 KV element takes one byte, half of fp16
(youngju.dev "KV cache and paged attention", section "KV 양자화: FP8과 INT8").
The concrete format is E4M3 in its "FN" variant (no infinities, a single NaN
mantissa pattern), which is the FP8 format gfx950 computes in natively:

* bit 7 sign, bits 6..3 exponent (bias 7), bits 2..0 mantissa;
* exponent 0: subnormal, value m/8 * 2**-6;
* exponent 15 with mantissa 7: NaN; every other code is finite;
* largest finite magnitude (1 + 6/8) * 2**8 = 448.

Encoding saturates: magnitudes above 448 become 448 (not NaN), then rounds
to the nearest representable value, ties to an even mantissa code.  NaN input
maps to code 0x7F.
"""
from __future__ import annotations

import numpy as np

E4M3_MAX = 448.0
E4M3_NAN_CODE = 0x7F


def decode(codes) -> np.ndarray:
    """Value of each uint8 code as float64 (NaN for 0x7F / 0xFF)."""
    c = np.asarray(codes, dtype=np.uint8).astype(np.int64)
    sign = np.where((c >> 7) & 1, -1.0, 1.0)
    e = (c >> 3) & 0xF
    m = c & 0x7
    sub = (m / 8.0) * 2.0 ** -6
    nor = (1.0 + m / 8.0) * np.exp2(e.astype(np.float64) - 7.0)
    val = np.where(e == 0, sub, nor)
    val = np.where((e == 15) & (m == 7), np.nan, val)
    return sign * val


def encode(x) -> np.ndarray:
    """Saturating round-to-nearest-even encode of float values to E4M3FN codes.

    ``x`` is taken exactly as given (float32 inputs are exact in float64).
    """
    v = np.asarray(x, dtype=np.float64)
    nan = np.isnan(v)
    neg = np.signbit(v)
    a = np.minimum(np.abs(np.where(nan, 0.0, v)), E4M3_MAX)
    codes = np.zeros(v.shape, dtype=np.int64)

    # Subnormal range: spacing 2**-9 below the smallest normal 2**-6.  A
    # quotient that rounds up to 8 is exactly the smallest normal, whose code
    # (exponent 1, mantissa 0) is also 8, so the formula stays valid.
    small = a < 2.0 ** -6
    q_sub = np.rint(a / 2.0 ** -9)  # numpy rint: ties to even
    codes = np.where(small, q_sub.astype(np.int64), codes)

    # Normal range: a = 2**e * (q / 8) with q in [8, 16).
    safe = np.where(small, 1.0, a)
    e = np.floor(np.log2(safe)).astype(np.int64)
    # log2 can be off by one ulp near powers of two; correct e so 2**e <= a < 2**(e+1).
    e = np.where(np.exp2(e.astype(np.float64)) > safe, e - 1, e)
    e = np.where(np.exp2((e + 1).astype(np.float64)) <= safe, e + 1, e)
    q = np.rint(safe / np.exp2((e - 3).astype(np.float64))).astype(np.int64)
    carry = q == 16
    e = np.where(carry, e + 1, e)
    q = np.where(carry, 8, q)
    nor_code = ((e + 7) << 3) | (q - 8)
    codes = np.where(small, codes, nor_code)

    codes = np.where(neg, codes | 0x80, codes)
    codes = np.where(nan, E4M3_NAN_CODE, codes)
    return codes.astype(np.uint8)


def quantize(x_fp16, inv_scale) -> np.ndarray:
    """Codes of ``f32(x) * f32(inv_scale)`` (one float32 multiply, then encode).

    ``inv_scale`` broadcasts against ``x``.  The product is formed in float32
    so that any implementation doing the same single multiply rounds alike.
    """
    x32 = np.asarray(x_fp16, dtype=np.float16).astype(np.float32)
    y = x32 * np.asarray(inv_scale, dtype=np.float32)
    return encode(y.astype(np.float32))


def inverse_scale(scale) -> np.ndarray:
    """float32 reciprocal ``f32(1) / f32(scale)`` (IEEE division, RNE)."""
    s = np.asarray(scale, dtype=np.float32)
    return (np.float32(1.0) / s).astype(np.float32)
