"""INT8 KV codec with a scale and a zero point, written from its definition.

The pages fix that an INT8 KV element takes one byte, half of fp16, and that
it needs a scale and a zero point (youngju.dev "KV cache and paged
attention", section "KV 양자화: FP8과 INT8").  They give no formula or
granularity; the plainest reading, affine quantisation, is taken here:

* a code is a signed 8-bit integer c in [-128, 127];
* its value is (c - z) * s, with one fp32 scale s > 0 and one integer zero
  point z in [-128, 127] per (layer, KV head), for K and for V separately
  (the granularity of the fp8 path);
* encoding forms y = f32(x) * f32(1 / s) with one float32 multiply, rounds y
  to the nearest integer with ties to even, adds z and saturates to
  [-128, 127]; NaN encodes as z (the value 0), infinities saturate.

Both sides take the rounding decision on the same float32 product, so the
codes agree bit for bit.
"""
from __future__ import annotations

import numpy as np

INT8_MIN, INT8_MAX = -128, 127


def inverse_scale(scale) -> np.ndarray:
    """float32 reciprocal ``f32(1) / f32(scale)`` (IEEE division, RNE)."""
    s = np.asarray(scale, dtype=np.float32)
    return (np.float32(1.0) / s).astype(np.float32)


def encode(y, zero) -> np.ndarray:
    """int8 codes of already-scaled values ``y`` (float32): RNE, + zero, saturate."""
    y = np.asarray(y, dtype=np.float32).astype(np.float64)  # exact
    z = np.asarray(zero, dtype=np.int64)
    nan = np.isnan(y)
    r = np.rint(np.where(nan, 0.0, y))  # numpy rint: ties to even; inf stays inf
    c = np.clip(r + z, INT8_MIN, INT8_MAX)
    return c.astype(np.int8)


def quantize(x_fp16, inv_scale, zero) -> np.ndarray:
    """Codes of ``f32(x) * f32(inv_scale)``, rounded, shifted by ``zero`` and
    saturated.  ``inv_scale`` and ``zero`` broadcast against ``x``."""
    x32 = np.asarray(x_fp16, dtype=np.float16).astype(np.float32)
    y = x32 * np.asarray(inv_scale, dtype=np.float32)
    return encode(y.astype(np.float32), zero)


def decode(codes, scale, zero) -> np.ndarray:
    """float64 values ``(c - z) * s``; ``scale`` and ``zero`` broadcast."""
    c = np.asarray(codes, dtype=np.int8).astype(np.float64)
    z = np.asarray(zero, dtype=np.int64).astype(np.float64)
    s = np.asarray(scale, dtype=np.float32).astype(np.float64)
    return (c - z) * s
