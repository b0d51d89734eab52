"""Planted mistakes in the oracle (CPU only) must be caught by its pins.

Each test patches one plausible slip into an oracle function (a dropped
scale, a wrong index, a swapped operand, a wrong exponent bias, truncation
instead of round-to-nearest-even) and checks that at least one pin fails.
"""
import numpy as np
import pytest

from oracle import allocator as alloc_mod
from oracle import attention, fp8
from tests import test_oracle_allocator as ta
from tests import test_oracle_attention as tt
from tests import test_oracle_fp8 as tf


def _fails(fn, *args):
    with pytest.raises(AssertionError):
        fn(*args)


def test_dropped_softmax_scale_is_caught(monkeypatch):
    orig = attention._attend
    monkeypatch.setattr(attention, "_attend", lambda q, k, v, scale: orig(q, k, v, 1.0))
    _fails(tt.test_decode_matches_sdpa_fp16, 8, 2, 16)


def test_wrong_kv_head_is_caught(monkeypatch):
    orig = attention.gather_context
    monkeypatch.setattr(attention, "gather_context",
                        lambda s, l, t, n, h: orig(s, l, t, n, (h + 1) % s.kv_heads))
    _fails(tt.test_decode_matches_sdpa_fp16, 8, 2, 16)


def test_reversed_block_order_is_caught(monkeypatch):
    orig = attention.gather_context

    def bad(s, l, table, n, h):
        nb = -(-int(n) // s.block_size)
        return orig(s, l, list(table[:nb])[::-1], n, h)

    monkeypatch.setattr(attention, "gather_context", bad)
    _fails(tt.test_decode_matches_sdpa_fp16, 32, 8, 8)


def test_off_by_one_context_is_caught(monkeypatch):
    orig = attention.gather_context
    monkeypatch.setattr(attention, "gather_context", lambda s, l, t, n, h: orig(s, l, t, max(1, n - 1), h))
    _fails(tt.test_decode_matches_sdpa_fp16, 4, 4, 32)


def test_transposed_pv_is_caught(monkeypatch):
    def bad(q, k, v, scale):
        s = (k @ q) * scale
        p = np.exp(s - s.max())
        return (v.T @ p)[::-1] / p.sum()  # dims reversed
    monkeypatch.setattr(attention, "_attend", bad)
    _fails(tt.test_decode_matches_sdpa_fp16, 8, 2, 16)


def test_wrong_fp8_bias_is_caught(monkeypatch):
    orig = fp8.decode
    monkeypatch.setattr(fp8, "decode", lambda c: orig(c) * 2.0)
    _fails(tf.test_decode_matches_torch_for_all_codes)


def test_truncating_fp8_encode_is_caught(monkeypatch):
    monkeypatch.setattr(np, "rint", np.trunc)
    _fails(tf.test_encode_matches_torch_on_all_fp16_values)


def test_unsaturated_fp8_encode_is_caught(monkeypatch):
    monkeypatch.setattr(fp8, "E4M3_MAX", 480.0)
    _fails(tf.test_encode_ties_and_saturation)


def test_wrong_slot_offset_is_caught(monkeypatch):
    class Bad(alloc_mod.OracleAllocator):
        def alloc(self, sid, n):
            start = self.lens[sid]
            slots, cow = super().alloc(sid, n)
            bs = self.block_size
            # offset taken from the wrong end of the block
            return [s - (start + j) % bs + (bs - 1 - (start + j) % bs) for j, s in enumerate(slots)], cow
    monkeypatch.setattr(ta, "OracleAllocator", Bad)
    _fails(ta.test_page_block_table_example)


def test_cow_without_copy_is_caught(monkeypatch):
    class Bad(alloc_mod.OracleAllocator):
        def alloc(self, sid, n):
            slots, cow = super().alloc(sid, n)
            return slots, None  # forgets to report (so nobody copies) the shared block
    monkeypatch.setattr(ta, "OracleAllocator", Bad)
    _fails(ta.test_slot_mapping_content_round_trip_through_fork_and_cow)


def test_int8_zero_point_with_wrong_sign_is_caught(monkeypatch):
    from oracle import int8
    from tests import test_oracle_int8 as ti
    monkeypatch.setattr(int8, "decode", lambda c, s, z: (np.asarray(c, dtype=np.int8).astype(np.float64)
                                                         + np.asarray(z, dtype=np.float64))
                        * np.asarray(s, dtype=np.float32).astype(np.float64))
    _fails(ti.test_grid_points_are_exact_and_round_trip)


def test_truncating_int8_encode_is_caught(monkeypatch):
    from oracle import int8
    from tests import test_oracle_int8 as ti

    def bad(y, zero):
        y = np.nan_to_num(np.asarray(y, dtype=np.float64), nan=0.0, posinf=1e9, neginf=-1e9)
        return np.clip(np.trunc(y) + np.asarray(zero), -128, 127).astype(np.int8)
    monkeypatch.setattr(int8, "encode", bad)
    _fails(ti.test_ties_to_even_saturation_and_nan)
    _fails(ti.test_encode_matches_torch_qint8_away_from_ties, 0.02, 0)


def test_int8_zero_point_after_saturation_is_caught(monkeypatch):
    from oracle import int8
    from tests import test_oracle_int8 as ti

    def bad(y, zero):
        y = np.nan_to_num(np.asarray(y, dtype=np.float64), nan=0.0, posinf=1e9, neginf=-1e9)
        return np.clip(np.clip(np.rint(y), -128, 127) + np.asarray(zero), -128, 127).astype(np.int8)
    monkeypatch.setattr(int8, "encode", bad)
    _fails(ti.test_ties_to_even_saturation_and_nan)


def _multi_token_with(visible_of):
    """A copy of the oracle's multi-token attention with the causal limit replaced."""
    import math

    def bad(store, layer, q, query_start, block_tables, context_lens, scale=None):
        q = np.asarray(q, dtype=np.float64)
        n_rows, hq, d = q.shape
        g = hq // store.kv_heads
        scale = 1.0 / math.sqrt(d) if scale is None else scale
        qs = [int(x) for x in query_start]
        out = np.zeros((n_rows, hq, d))
        for i in range(len(qs) - 1):
            n_i, length = qs[i + 1] - qs[i], int(context_lens[i])
            for kvh in range(store.kv_heads):
                k, v = attention.gather_context(store, layer, block_tables[i], length, kvh)
                for j in range(n_i):
                    vis = max(1, min(length, visible_of(length, n_i, j)))
                    for h in range(kvh * g, (kvh + 1) * g):
                        out[qs[i] + j, h] = attention._attend(q[qs[i] + j, h], k[:vis], v[:vis], scale)
        return out
    return bad


def test_causal_limit_off_by_one_is_caught(monkeypatch):
    from tests import test_oracle_multi_token as tm
    monkeypatch.setattr(attention, "multi_token", _multi_token_with(lambda t, n, j: t - n + j))
    _fails(tm.test_full_prefill_is_causal_sdpa, 8, 2, 16)


def test_chunk_positions_from_the_start_are_caught(monkeypatch):
    from tests import test_oracle_multi_token as tm
    monkeypatch.setattr(attention, "multi_token", _multi_token_with(lambda t, n, j: j + 1))
    _fails(tm.test_chunk_after_cached_context_matches_masked_sdpa)
