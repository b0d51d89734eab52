"""Pins of the oracle's paged decode against contiguous attention computed
independently (torch scaled_dot_product_attention in float64 on the dense
K/V straight from the generator, never through a block table), closed-form
special cases, placement/sharing invariants and the LSE merge identity."""
import math

import numpy as np
import pytest
import torch

from oracle import attention, fp8
from oracle.allocator import OracleAllocator
from oracle.kvstore import OracleKVStore
from tests.oracle_helpers import build_paged, tables_of
from workloads import free_order, normal_fp16, uniform_ints


def _sdpa_reference(q, k_list, v_list, lens, group):
    """softmax(q K^T / sqrt(d)) V per (seq, head) via torch SDPA in float64, GQA by
    repeating each KV head for its consecutive group of query heads."""
    out = []
    for i, t in enumerate(lens):
        k = torch.from_numpy(np.asarray(k_list[i][:t], dtype=np.float64)).permute(1, 0, 2)  # [Hkv][T][d]
        v = torch.from_numpy(np.asarray(v_list[i][:t], dtype=np.float64)).permute(1, 0, 2)
        k = k.repeat_interleave(group, dim=0).contiguous()
        v = v.repeat_interleave(group, dim=0).contiguous()
        qi = torch.from_numpy(np.asarray(q[i], dtype=np.float64))[:, None, :]  # [Hq][1][d]
        o = torch.nn.functional.scaled_dot_product_attention(qi, k, v)
        out.append(o[:, 0, :].numpy())
    return np.stack(out)


def _case(seed, n_seqs, hq, hkv, d, bs, max_t, dtype="fp16"):
    lens = uniform_ints(seed, 5, 1, max_t, n_seqs)
    lens[0] = 1  # always include the single-token edge case
    k = [normal_fp16((int(t), hkv, d), seed, 100 + i).numpy() for i, t in enumerate(lens)]
    v = [normal_fp16((int(t), hkv, d), seed, 200 + i).numpy() for i, t in enumerate(lens)]
    q = normal_fp16((n_seqs, hq, d), seed, 300).numpy()
    n_blocks = int(sum(-(-int(t) // bs) for t in lens)) + 3
    order = free_order(seed, n_blocks)
    return lens, k, v, q, n_blocks, order


@pytest.mark.parametrize("hq,hkv", [(8, 2), (4, 4), (32, 8), (32, 1), (16, 2)])
@pytest.mark.parametrize("bs", [8, 16, 32])
def test_decode_matches_sdpa_fp16(hq, hkv, bs):
    seed = 7 + hq * 31 + hkv * 7 + bs
    d = 128
    lens, k, v, q, n_blocks, order = _case(seed, 4, hq, hkv, d, bs, 75)
    alloc, store, seqs, _ = build_paged(k, v, lens, bs, n_blocks, order)
    tables, tl = tables_of(alloc, seqs)
    np.testing.assert_array_equal(tl, lens)
    got = attention.decode(store, 0, q, tables, lens)
    ref = _sdpa_reference(q, k, v, lens, hq // hkv)
    np.testing.assert_allclose(got, ref, rtol=0, atol=1e-12)


def test_decode_matches_sdpa_head_dim_64():
    lens, k, v, q, n_blocks, order = _case(11, 3, 8, 2, 64, 16, 50)
    alloc, store, seqs, _ = build_paged(k, v, lens, 16, n_blocks, order)
    tables, _ = tables_of(alloc, seqs)
    got = attention.decode(store, 0, q, tables, lens)
    np.testing.assert_allclose(got, _sdpa_reference(q, k, v, lens, 4), rtol=0, atol=1e-12)


@pytest.mark.parametrize("hq,hkv,bs", [(32, 8, 16), (32, 1, 8), (32, 1, 32)])
def test_decode_matches_sdpa_fp8(hq, hkv, bs):
    d = 128
    lens, k, v, q, n_blocks, order = _case(23 + bs, 3, hq, hkv, d, bs, 60)
    ks = (np.abs(np.concatenate(k)).max(axis=(0, 2)) / 448).astype(np.float32)
    vs = (np.abs(np.concatenate(v)).max(axis=(0, 2)) / 448).astype(np.float32)
    alloc, store, seqs, _ = build_paged(k, v, lens, bs, n_blocks, order, "fp8", ks, vs)
    tables, _ = tables_of(alloc, seqs)
    got = attention.decode(store, 0, q, tables, lens)
    # Dense dequantised K/V computed per token without any block table.
    kd = [fp8.decode(fp8.quantize(x, fp8.inverse_scale(ks)[:, None])) * ks[:, None].astype(np.float64) for x in k]
    vd = [fp8.decode(fp8.quantize(x, fp8.inverse_scale(vs)[:, None])) * vs[:, None].astype(np.float64) for x in v]
    np.testing.assert_allclose(got, _sdpa_reference(q, kd, vd, lens, hq // hkv), rtol=0, atol=1e-12)


def test_single_token_returns_its_value_exactly():
    k = [normal_fp16((1, 2, 128), 1, 1).numpy()]
    v = [normal_fp16((1, 2, 128), 1, 2).numpy()]
    q = normal_fp16((1, 8, 128), 1, 3).numpy()
    alloc, store, seqs, _ = build_paged(k, v, [1], 16, 4)
    out = attention.decode(store, 0, q, *tables_of(alloc, seqs))
    for h in range(8):
        np.testing.assert_array_equal(out[0, h], v[0][0, h // 4].astype(np.float64))


def test_equal_keys_give_mean_value():
    t = 37
    kk = np.repeat(normal_fp16((1, 2, 128), 2, 1).numpy(), t, axis=0)
    v = [normal_fp16((t, 2, 128), 2, 2).numpy()]
    q = normal_fp16((1, 8, 128), 2, 3).numpy()
    alloc, store, seqs, _ = build_paged([kk], v, [t], 16, 4, [3, 1, 0, 2])
    out = attention.decode(store, 0, q, *tables_of(alloc, seqs))
    mean = v[0].astype(np.float64).mean(axis=0)  # [Hkv][d]
    for h in range(8):
        np.testing.assert_allclose(out[0, h], mean[h // 4], rtol=0, atol=1e-14)


def test_dominant_key_selects_its_value():
    t, d = 29, 128
    k = normal_fp16((t, 1, d), 3, 1).numpy() * np.float16(0.01)
    q = np.zeros((1, 1, d), dtype=np.float16)
    q[0, 0, :] = 4.0
    k[17, 0, :] = 4.0  # score 4*4*128/sqrt(128) ~ 181 above the rest
    v = [normal_fp16((t, 1, d), 3, 2).numpy()]
    alloc, store, seqs, _ = build_paged([k], v, [t], 8, 8, list(range(8))[::-1])
    out = attention.decode(store, 0, q, *tables_of(alloc, seqs))
    np.testing.assert_allclose(out[0, 0], v[0][17, 0].astype(np.float64), rtol=0, atol=1e-30)


def test_kv_head_grouping_is_consecutive():
    """Distinct data per KV head: query head h must read KV head h // G."""
    lens, k, v, q, n_blocks, order = _case(5, 2, 8, 2, 128, 16, 30)
    alloc, store, seqs, _ = build_paged(k, v, lens, 16, n_blocks, order)
    out = attention.decode(store, 0, q, *tables_of(alloc, seqs))
    for h in range(8):
        solo = _sdpa_reference(q[:, h:h + 1], [x[:, h // 4:h // 4 + 1] for x in k],
                               [x[:, h // 4:h // 4 + 1] for x in v], lens, 1)
        np.testing.assert_allclose(out[:, h], solo[:, 0], rtol=0, atol=1e-12)
    # An interleaved map (h % Hkv) would differ for these inputs.
    wrong = _sdpa_reference(q[:, 1:2], [x[:, 1:2] for x in k], [x[:, 1:2] for x in v], lens, 1)
    assert np.abs(out[:, 1] - wrong[:, 0]).max() > 1e-3


def test_output_invariant_under_physical_placement():
    lens, k, v, q, n_blocks, _ = _case(9, 5, 32, 8, 128, 16, 90)
    outs = []
    for s in range(3):
        order = free_order(1000 + s, n_blocks)
        alloc, store, seqs, _ = build_paged(k, v, lens, 16, n_blocks, order)
        outs.append(attention.decode(store, 0, q, *tables_of(alloc, seqs)))
    np.testing.assert_array_equal(outs[0], outs[1])
    np.testing.assert_array_equal(outs[0], outs[2])


def test_shared_prefix_equals_unshared_clone():
    bs, hkv, d, prefix, suffix = 16, 2, 128, 40, 13
    kp = normal_fp16((prefix + suffix, hkv, d), 4, 1).numpy()
    vp = normal_fp16((prefix + suffix, hkv, d), 4, 2).numpy()
    q = normal_fp16((1, 8, d), 4, 3).numpy()
    alloc = OracleAllocator(32, bs, free_order(4, 32))
    store = OracleKVStore(1, 32, hkv, bs, d)
    parent = alloc.seq_create()
    slots, _ = alloc.alloc(parent, prefix)
    store.write(0, kp[:prefix], vp[:prefix], slots)
    child = alloc.fork(parent)
    # Sharers read the same physical blocks.
    assert alloc.tables[child] == alloc.tables[parent]
    slots, cow = alloc.alloc(child, suffix)
    assert cow is not None  # partial shared last block copied for the writer
    store.copy_block(*cow)
    store.write(0, kp[prefix:], vp[prefix:], slots)
    clone = alloc.seq_create()
    slots, _ = alloc.alloc(clone, prefix + suffix)
    store.write(0, kp, vp, slots)
    # The full shared blocks are still shared, the copied one is not.
    assert alloc.tables[child][:2] == alloc.tables[parent][:2]
    assert alloc.tables[child][2] != alloc.tables[parent][2]
    tables, lens = tables_of(alloc, [child, clone])
    out = attention.decode(store, 0, np.concatenate([q, q]), tables, lens)
    np.testing.assert_array_equal(out[0], out[1])
    # The parent still sees only its own 40 tokens.
    tp, lp = tables_of(alloc, [parent])
    ref = _sdpa_reference(q, [kp[:prefix]], [vp[:prefix]], [prefix], 4)
    np.testing.assert_allclose(attention.decode(store, 0, q, tp, lp), ref, rtol=0, atol=1e-12)


@pytest.mark.parametrize("partition", [16, 32, 512, None])
def test_split_then_lse_merge_equals_decode(partition):
    lens, k, v, q, n_blocks, order = _case(13, 4, 16, 2, 128, 16, 700)
    alloc, store, seqs, _ = build_paged(k, v, lens, 16, n_blocks, order)
    tables, tl = tables_of(alloc, seqs)
    full = attention.decode(store, 0, q, tables, tl)
    p = partition or int(max(lens))
    parts = attention.split_partials(store, 0, q, tables, tl, p)
    for i in range(len(lens)):
        m, lsum, o = parts[i]
        assert m.shape[1] == -(-int(lens[i]) // p)
        for h in range(q.shape[1]):
            merged = attention.lse_merge(m[h], lsum[h], o[h])
            np.testing.assert_allclose(merged, full[i, h], rtol=1e-13, atol=1e-15)


def test_split_chunk_outputs_are_chunk_attention():
    lens = np.array([200, 77])
    k = [normal_fp16((int(t), 2, 128), 17, 100 + i).numpy() for i, t in enumerate(lens)]
    v = [normal_fp16((int(t), 2, 128), 17, 200 + i).numpy() for i, t in enumerate(lens)]
    q = normal_fp16((2, 8, 128), 17, 300).numpy()
    alloc, store, seqs, _ = build_paged(k, v, lens, 16, 20, free_order(17, 20))
    tables, tl = tables_of(alloc, seqs)
    parts = attention.split_partials(store, 0, q, tables, tl, 64)
    for i, t in enumerate(lens):
        _, _, o = parts[i]
        for c in range(-(-int(t) // 64)):
            lo, hi = 64 * c, min(64 * (c + 1), int(t))
            ref = _sdpa_reference(q[i:i + 1], [k[i][lo:hi]], [v[i][lo:hi]], [hi - lo], 4)
            np.testing.assert_allclose(o[:, c], ref[0], rtol=0, atol=1e-12)


def test_unwritten_slots_never_read():
    """Unused slots of the last block hold NaN in the oracle store; outputs stay finite."""
    lens, k, v, q, n_blocks, order = _case(19, 3, 8, 2, 128, 16, 45)
    alloc, store, seqs, _ = build_paged(k, v, lens, 16, n_blocks, order)
    out = attention.decode(store, 0, q, *tables_of(alloc, seqs))
    assert np.isfinite(out).all()


def test_scale_argument_is_softmax_temperature():
    lens, k, v, q, n_blocks, order = _case(21, 2, 8, 2, 128, 16, 40)
    alloc, store, seqs, _ = build_paged(k, v, lens, 16, n_blocks, order)
    tables, tl = tables_of(alloc, seqs)
    a = attention.decode(store, 0, q, tables, tl, scale=1.0 / math.sqrt(128))
    b = attention.decode(store, 0, q, tables, tl)
    np.testing.assert_array_equal(a, b)
    c = attention.decode(store, 0, q, tables, tl, scale=0.0)  # uniform weights -> mean
    np.testing.assert_allclose(c[1, 0], np.asarray(v[1][:lens[1], 0], np.float64).mean(0), atol=1e-14)
