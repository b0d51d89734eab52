"""Pins of the oracle's multi-token (chunked prefill / mixed batch) paged
attention: torch SDPA in float64 with its own causal masks on the dense K/V
straight from the generator, the decode special case, and prefix invariance."""
import numpy as np
import pytest
import torch

from oracle import attention
from tests.oracle_helpers import build_paged, tables_of
from workloads import free_order, normal_fp16


def _dense_case(seed, lens, hq, hkv, bs):
    k = [normal_fp16((t, hkv, 128), seed, 100 + i).numpy() for i, t in enumerate(lens)]
    v = [normal_fp16((t, hkv, 128), seed, 200 + i).numpy() for i, t in enumerate(lens)]
    nb = sum(-(-t // bs) for t in lens) + 3
    alloc, store, seqs, _ = build_paged(k, v, lens, bs, nb, free_order(seed, nb))
    tables, tl = tables_of(alloc, seqs)
    return k, v, store, tables, tl


def _sdpa_rows(q_rows, k, v, group, positions):
    """SDPA over dense K/V [T][Hkv][d] for query rows at the given positions,
    masking key t > position with torch's boolean attn_mask."""
    kk = torch.from_numpy(k.astype(np.float64)).permute(1, 0, 2).repeat_interleave(group, 0).contiguous()
    vv = torch.from_numpy(v.astype(np.float64)).permute(1, 0, 2).repeat_interleave(group, 0).contiguous()
    qq = torch.from_numpy(q_rows.astype(np.float64)).permute(1, 0, 2).contiguous()  # [Hq][n][d]
    mask = torch.arange(k.shape[0])[None, :] <= torch.as_tensor(positions)[:, None]
    o = torch.nn.functional.scaled_dot_product_attention(qq, kk, vv, attn_mask=mask)
    return o.permute(1, 0, 2).numpy()


@pytest.mark.parametrize("hq,hkv,bs", [(8, 2, 16), (32, 8, 8), (32, 1, 32), (4, 4, 16)])
def test_full_prefill_is_causal_sdpa(hq, hkv, bs):
    """n_i = T_i: the whole prompt attends causally (torch's is_causal)."""
    lens = [1, 37, 70]
    k, v, store, tables, tl = _dense_case(11 + bs, lens, hq, hkv, bs)
    qs = np.concatenate([[0], np.cumsum(lens)])
    q = normal_fp16((int(qs[-1]), hq, 128), 11 + bs, 300).numpy()
    got = attention.multi_token(store, 0, q, qs, tables, tl)
    for i, t in enumerate(lens):
        qq = torch.from_numpy(q[qs[i]:qs[i + 1]].astype(np.float64)).permute(1, 0, 2).contiguous()
        kk = torch.from_numpy(k[i].astype(np.float64)).permute(1, 0, 2).repeat_interleave(hq // hkv, 0).contiguous()
        vv = torch.from_numpy(v[i].astype(np.float64)).permute(1, 0, 2).repeat_interleave(hq // hkv, 0).contiguous()
        ref = torch.nn.functional.scaled_dot_product_attention(qq, kk, vv, is_causal=True).permute(1, 0, 2).numpy()
        np.testing.assert_allclose(got[qs[i]:qs[i + 1]], ref, rtol=0, atol=1e-12)


def test_chunk_after_cached_context_matches_masked_sdpa():
    """A chunk of n_i < T_i tokens at the end of the context (earlier tokens
    cached), mixed with decode rows and an empty sequence."""
    lens = [50, 1, 33, 20, 9]
    n = [12, 1, 33, 0, 1]
    k, v, store, tables, tl = _dense_case(21, lens, 16, 2, 8)
    qs = np.concatenate([[0], np.cumsum(n)])
    q = normal_fp16((int(qs[-1]), 16, 128), 21, 300).numpy()
    got = attention.multi_token(store, 0, q, qs, tables, tl)
    for i, t in enumerate(lens):
        if n[i] == 0:
            continue
        pos = np.arange(t - n[i], t)
        ref = _sdpa_rows(q[qs[i]:qs[i + 1]], k[i], v[i], 8, pos)
        np.testing.assert_allclose(got[qs[i]:qs[i + 1]], ref, rtol=0, atol=1e-12)


def test_one_token_per_sequence_is_decode():
    lens = [5, 64, 17]
    k, v, store, tables, tl = _dense_case(31, lens, 8, 2, 16)
    q = normal_fp16((3, 8, 128), 31, 300).numpy()
    got = attention.multi_token(store, 0, q, [0, 1, 2, 3], tables, tl)
    np.testing.assert_array_equal(got, attention.decode(store, 0, q, tables, tl))


def test_row_equals_decode_of_its_prefix_and_bad_inputs_raise():
    lens = [40]
    k, v, store, tables, tl = _dense_case(41, lens, 8, 8, 16)
    q = normal_fp16((10, 8, 128), 41, 300).numpy()
    got = attention.multi_token(store, 0, q, [0, 10], tables, tl)
    for j in range(10):
        ref = attention.decode(store, 0, q[j:j + 1], tables, [30 + j + 1])
        np.testing.assert_allclose(got[j], ref[0], rtol=0, atol=1e-12)
    with pytest.raises(ValueError):
        attention.multi_token(store, 0, q, [0, 10], tables, [9])  # more queries than context
    with pytest.raises(ValueError):
        attention.multi_token(store, 0, q, [0, 11], tables, tl)
