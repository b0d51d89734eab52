"""The parity criteria of tests/parity.py see the mistakes that matter at long
context, and pass the rounding the kernel's arithmetic makes.

Inputs are the long-context and GQA workloads' shapes on one KV head: K, V, q
~ N(0, 1) in fp16, 512-token chunks (131072 tokens, 8 query heads per KV
head) and 16-token blocks (4096 tokens, 4 query heads per KV head).  The
mistakes are made on the oracle's own output: its chunk partials merged with
one chunk left out, and attention with one block of keys left out.
"""
import numpy as np
import pytest

from oracle import attention
from oracle.kvstore import OracleKVStore
from tests import parity
from workloads import normal_fp16


def _store(t, g, seed):
    """One-layer, one-KV-head store holding t tokens in blocks 0, 1, 2, ...
    and the query of g heads."""
    bs = 16
    k = normal_fp16((t, 1, 128), seed, 1).numpy()
    v = normal_fp16((t, 1, 128), seed, 2).numpy()
    q = normal_fp16((1, g, 128), seed, 3).numpy()
    st = OracleKVStore(1, -(-t // bs), 1, bs, 128)
    st.write(0, k, v, np.arange(t))
    table = np.arange(-(-t // bs))[None, :]
    return st, q, table


@pytest.fixture(scope="module")
def long_ctx_parts():
    t, g, p = 131072, 8, 512
    st, q, table = _store(t, g, 464_004)
    (m, lsum, o), = attention.split_partials(st, 0, q, table, [t], p)
    ref = np.stack([attention.lse_merge(m[h], lsum[h], o[h]) for h in range(g)])[None]
    return m, lsum, o, ref


@pytest.mark.parametrize("chunk", [0, 101, 255])
def test_a_lost_512_token_chunk_at_131072_tokens_is_rejected(long_ctx_parts, chunk):
    m, lsum, o, ref = long_ctx_parts
    keep = np.ones(m.shape[1], dtype=bool)
    keep[chunk] = False
    lost = np.stack([attention.lse_merge(m[h][keep], lsum[h][keep], o[h][keep])
                     for h in range(m.shape[0])])[None]
    bad, max_abs, row_rel = parity.failures(lost, ref, "fp16")
    # The stated max-abs bound alone would accept this mistake ...
    assert max_abs <= parity.FP16_ATOL
    # ... the derived row-relative bound does not.
    assert bad and row_rel > 2 * parity.ROW_RTOL, (max_abs, row_rel)


@pytest.mark.parametrize("block", [0, 128, 255])
def test_a_lost_16_token_block_at_4096_tokens_is_rejected(block):
    t, g = 4096, 4
    st, q, table = _store(t, g, 464_002)
    ref = attention.decode(st, 0, q, table, [t])
    # Attention with one block of keys left out (the table without it).
    short = np.delete(table[0], block)[None, :]
    lost = attention.decode(st, 0, q, short, [t - 16])
    bad, max_abs, row_rel = parity.failures(lost, ref, "fp16")
    assert bad and row_rel > 2 * parity.ROW_RTOL, (max_abs, row_rel)


def _kernel_precision(k, v, q, scale):
    """The kernel's rounding steps in numpy: fp32 scores of exact fp16
    operands, fp32 exponentials, probabilities rounded to fp16 for the P.V
    product, fp32 sums, fp16 output."""
    s = (k.astype(np.float32) @ q.astype(np.float32)) * np.float32(scale)
    p = np.exp(s - s.max()).astype(np.float32)
    num = p.astype(np.float16).astype(np.float32) @ v.astype(np.float32)
    return (num / p.sum(dtype=np.float32)).astype(np.float16)


@pytest.mark.parametrize("t", [1, 20, 40, 4096, 131072])
def test_the_kernels_rounding_passes_with_margin(t):
    g = 8
    st, q, table = _store(t, g, 464_100 + t)
    ref = attention.decode(st, 0, q, table, [t])
    kc, vc = attention.gather_context(st, 0, table[0], t, 0)
    got = np.stack([_kernel_precision(kc, vc, q[0, h], 1 / np.sqrt(128)) for h in range(g)])[None]
    bad, max_abs, row_rel = parity.failures(got.astype(np.float64), ref, "fp16")
    assert not bad
    # The fp16 output rounding bounds it: at most 2^-11 of the row's largest
    # value per element, plus far smaller probability and sum rounding.
    assert row_rel <= 2.0 ** -11 * 1.5, row_rel
    assert row_rel * 4 <= parity.ROW_RTOL


def test_stated_fp8_bound_is_kept_beside_the_derived_one():
    ref = np.ones((1, 1, 128))
    got = ref.copy()
    got[0, 0, 0] += 3e-2
    bad, _, _ = parity.failures(got, ref, "fp8")
    assert any("2e-02" in b or "0.02" in b for b in bad) and len(bad) == 2
    got[0, 0, 0] = 1 + 1e-2  # inside the stated 2e-2, outside the derived 4e-3
    bad, _, _ = parity.failures(got, ref, "fp8")
    assert len(bad) == 1 and str(parity.ROW_RTOL) in bad[0]


def test_non_finite_output_fails():
    ref = np.zeros((1, 2, 128))
    got = ref.copy()
    got[0, 1, 5] = np.nan
    assert parity.failures(got, ref, "int8")[0] == ["non-finite output"]
