"""Pins of the oracle's int8 (scale + zero point) codec: torch's per-tensor
qint8 quantiser (CPU), exact grid points, ties, saturation, the half-step
error bound, and the store's round trip; plus paged decode over an int8 store
against torch SDPA on the dense dequantised K/V."""
import numpy as np
import pytest
import torch

from oracle import attention, int8
from oracle.kvstore import OracleKVStore
from tests.oracle_helpers import build_paged, tables_of
from tests.test_oracle_attention import _case, _sdpa_reference


def _torch_qint8(x32, scale, zero):
    """Codes of torch.quantize_per_tensor(x, scale, zero, qint8)."""
    t = torch.from_numpy(np.asarray(x32, dtype=np.float32))
    return torch.quantize_per_tensor(t, float(scale), int(zero), torch.qint8).int_repr().numpy()


@pytest.mark.parametrize("scale,zero", [(0.02, 0), (0.0371, -17), (1.5, 90), (2.0 ** -7, -128), (0.3, 127)])
def test_encode_matches_torch_qint8_away_from_ties(scale, zero):
    rng = np.random.default_rng(int(scale * 1e4) + zero + 500)
    x = (rng.standard_normal(100_000) * 60 * scale).astype(np.float32)
    y = x * int8.inverse_scale(scale)
    # torch may form x / s where the oracle forms x * f32(1/s); away from the
    # rounding ties both products round to the same integer.
    far = np.abs(np.abs(y) - np.floor(np.abs(y)) - 0.5) > 1e-3
    got = int8.quantize(x.astype(np.float16), int8.inverse_scale(scale), zero)
    ref = _torch_qint8(x.astype(np.float16).astype(np.float32), scale, zero)
    assert far.mean() > 0.99
    np.testing.assert_array_equal(got[far], ref[far])
    assert got.dtype == np.int8 and ((got == 127) | (got == -128)).any()  # saturation exercised


def test_grid_points_are_exact_and_round_trip():
    s = np.float32(2.0 ** -5)
    for z in (-128, -3, 0, 77, 127):
        c = np.arange(-128, 128)
        x = ((c - z) * float(s)).astype(np.float16)  # exact: |c - z| <= 255, power-of-two step
        np.testing.assert_array_equal(x.astype(np.float64), (c - z) * float(s))
        codes = int8.quantize(x, int8.inverse_scale(s), z)
        np.testing.assert_array_equal(codes, c.astype(np.int8))
        np.testing.assert_array_equal(int8.decode(codes, s, z), x.astype(np.float64))


def test_ties_to_even_saturation_and_nan():
    y = np.array([0.5, 1.5, 2.5, -0.5, -1.5, -2.5, 126.5, 1e9, -1e9, np.inf, -np.inf, np.nan],
                 dtype=np.float32)
    np.testing.assert_array_equal(int8.encode(y, 0), [0, 2, 2, 0, -2, -2, 126, 127, -128, 127, -128, 0])
    np.testing.assert_array_equal(int8.encode(y, 3), [3, 5, 5, 3, 1, 1, 127, 127, -128, 127, -128, 3])
    # the zero point shifts before saturation: -130 + 5 stays in range
    np.testing.assert_array_equal(int8.encode(np.float32([-130.0, 125.0]), 5), [-125, 127])


@pytest.mark.parametrize("seed", [0, 1, 2])
def test_half_step_error_bound_inside_the_range(seed):
    rng = np.random.default_rng(seed)
    s = np.float32(rng.uniform(0.005, 0.1))
    z = int(rng.integers(-100, 100))
    lo, hi = (-128 - z) * float(s), (127 - z) * float(s)
    x = rng.uniform(lo, hi, 50_000).astype(np.float16)
    x = x[(x.astype(np.float64) >= lo) & (x.astype(np.float64) <= hi)]
    err = np.abs(int8.decode(int8.quantize(x, int8.inverse_scale(s), z), s, z) - x.astype(np.float64))
    assert err.max() <= float(s) * (0.5 + 1e-5)
    assert err.max() > float(s) * 0.45  # the bound is reached, not loose


def test_store_round_trip_mask_and_copy():
    st = OracleKVStore(2, 6, 2, 4, 128, "int8", k_scales=[0.01, 0.02, 0.03, 0.04],
                       v_scales=[0.05, 0.06, 0.07, 0.08], k_zeros=[0, -5, 7, 127], v_zeros=[-128, 1, 2, 3])
    rng = np.random.default_rng(4)
    k = (rng.standard_normal((3, 2, 128)) * 0.5).astype(np.float16)
    v = (rng.standard_normal((3, 2, 128)) * 2).astype(np.float16)
    st.write(1, k, v, [5, 6, -1])  # block 1 offsets 1, 2; the third token is skipped
    kc, vc = st.read_slots(1, [5, 6])
    assert kc.dtype == np.int8
    np.testing.assert_array_equal(kc[0, 1], int8.quantize(k[0, 1], int8.inverse_scale(0.04), 127))
    kb, vb = st.block_values(1, 1)
    np.testing.assert_array_equal(kb[1, 1], int8.decode(kc[0, 1], np.float32(0.04), 127))
    assert np.isnan(kb[:, 0]).all() and np.isnan(vb[:, 3]).all()  # never written
    assert np.isnan(st.block_values(0, 1)[0]).all()  # other layer untouched
    st.copy_block(1, 4)
    k4, v4 = st.block_values(1, 4)
    np.testing.assert_array_equal(np.isnan(k4), np.isnan(kb))
    np.testing.assert_array_equal(k4[~np.isnan(k4)], kb[~np.isnan(kb)])
    with pytest.raises(ValueError):
        OracleKVStore(1, 2, 1, 4, 128, "int8", [1.0], [1.0], [128], [0])


@pytest.mark.parametrize("hq,hkv,bs", [(32, 8, 16), (32, 1, 8), (8, 2, 32)])
def test_decode_matches_sdpa_int8(hq, hkv, bs):
    d = 128
    lens, k, v, q, n_blocks, order = _case(41 + bs, 3, hq, hkv, d, bs, 60)
    kall, vall = np.concatenate(k).astype(np.float64), np.concatenate(v).astype(np.float64)
    shift = np.linspace(-1.0, 1.5, hkv)[None, :, None]
    k = [(x.astype(np.float64) + shift).astype(np.float16) for x in k]  # per-head offsets
    kall = kall + shift
    kmin, kmax = kall.min(axis=(0, 2)), kall.max(axis=(0, 2))
    vmin, vmax = vall.min(axis=(0, 2)), vall.max(axis=(0, 2))
    ks = ((kmax - kmin) / 255).astype(np.float32)
    vs = ((vmax - vmin) / 255).astype(np.float32)
    kz = np.clip(np.rint(-128 - kmin / ks), -128, 127).astype(np.int64)
    vz = np.clip(np.rint(-128 - vmin / vs), -128, 127).astype(np.int64)
    alloc, store, seqs, _ = build_paged(k, v, lens, bs, n_blocks, order, "int8", ks, vs, kz, vz)
    tables, _ = tables_of(alloc, seqs)
    got = attention.decode(store, 0, q, tables, lens)
    # Dense K/V from the codes, dequantised per token by hand: (c - z) * s.
    kd, vd = [], []
    for x, y in zip(k, v):
        ck = int8.quantize(x, int8.inverse_scale(ks)[:, None], kz[:, None]).astype(np.float64)
        cv = int8.quantize(y, int8.inverse_scale(vs)[:, None], vz[:, None]).astype(np.float64)
        kd.append((ck - kz[:, None]) * ks[:, None].astype(np.float64))
        vd.append((cv - vz[:, None]) * vs[:, None].astype(np.float64))
    np.testing.assert_allclose(got, _sdpa_reference(q, kd, vd, lens, hq // hkv), rtol=0, atol=1e-12)
    # and the quantised attention stays close to the fp16 one (step <= range / 255)
    ref16 = _sdpa_reference(q, k, v, lens, hq // hkv)
    assert np.abs(got - ref16).max() < 0.1
