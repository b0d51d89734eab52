"""Pins of the oracle's E4M3FN codec against torch's float8_e4m3fn (CPU)."""
import numpy as np
import pytest
import torch

from oracle import fp8


def _torch_decode_all():
    return torch.arange(256, dtype=torch.uint8).view(torch.float8_e4m3fn).to(torch.float64).numpy()


def test_decode_matches_torch_for_all_codes():
    ref = _torch_decode_all()
    got = fp8.decode(np.arange(256, dtype=np.uint8))
    nan_ref, nan_got = np.isnan(ref), np.isnan(got)
    assert (nan_ref == nan_got).all()
    assert nan_got.sum() == 2  # 0x7F and 0xFF only
    np.testing.assert_array_equal(got[~nan_got], ref[~nan_ref])
    assert fp8.decode(np.uint8(0x7E)) == 448.0
    assert fp8.decode(np.uint8(0x01)) == 2.0 ** -9


def _torch_encode(x32):
    t = torch.from_numpy(np.asarray(x32, dtype=np.float32)).clamp(-448.0, 448.0)
    return t.to(torch.float8_e4m3fn).view(torch.uint8).numpy()


def test_encode_matches_torch_on_all_fp16_values():
    x = np.arange(65536, dtype=np.uint16).view(np.float16).astype(np.float32)
    x = x[np.isfinite(x)]
    np.testing.assert_array_equal(fp8.encode(x), _torch_encode(x))


@pytest.mark.parametrize("seed", [0, 1, 2])
def test_encode_matches_torch_on_random_fp32(seed):
    rng = np.random.default_rng(seed)
    x = (rng.standard_normal(200_000) * np.exp2(rng.uniform(-14, 12, 200_000))).astype(np.float32)
    np.testing.assert_array_equal(fp8.encode(x), _torch_encode(x))


def test_encode_ties_and_saturation():
    cases = {
        464.0: 0x7E,            # midpoint 448/480 -> saturate and round to 448
        1e9: 0x7E,              # saturation, not NaN
        -1e9: 0xFE,
        2.0 ** -10: 0x00,       # tie between 0 and 2^-9 -> even (0)
        3 * 2.0 ** -10: 0x02,   # tie between 2^-9 and 2^-8 -> even code 2
        1.5 * 2.0 ** -10: 0x01,
        1.0 + 1 / 16: 0x38,     # tie 1.0 / 1.125 -> mantissa 0
        1.0 + 3 / 16: 0x3A,     # tie 1.125 / 1.25 -> mantissa 2
        -0.0: 0x80,
    }
    x = np.array(list(cases), dtype=np.float32)
    np.testing.assert_array_equal(fp8.encode(x), np.array(list(cases.values()), dtype=np.uint8))
    assert fp8.encode(np.array([np.nan], dtype=np.float32))[0] == 0x7F


def test_round_trip_all_finite_codes():
    codes = np.array([c for c in range(256) if c not in (0x7F, 0xFF)], dtype=np.uint8)
    vals = fp8.decode(codes).astype(np.float32)
    back = fp8.encode(vals)
    # +0 and -0 both decode to zero but keep their sign bit
    np.testing.assert_array_equal(back, codes)


def test_quantize_is_single_fp32_multiply():
    x = np.array([1.0, -3.5, 0.1], dtype=np.float16)
    inv = fp8.inverse_scale(np.float32(0.0123))
    expect = fp8.encode(x.astype(np.float32) * inv)
    np.testing.assert_array_equal(fp8.quantize(x, inv), expect)
    assert inv.dtype == np.float32 and inv == np.float32(1) / np.float32(0.0123)
