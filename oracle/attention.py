"""Reference paged decode attention (float64).

Attention is softmax(Q K^T / sqrt(d_k)) V (youngju.dev "KV cache and paged
attention", section "핵심 원리: KV 캐시란 무엇인가").  In decode there is one
new query token per sequence; its K/V for all earlier tokens come from the
cache.  The paged kernel follows the sequence's block table to the physical
blocks and gathers non-contiguous K/V (iq-blog ch.4 "Why PagedAttention cuts
GPU memory waste", section "PagedAttention 알고리즘"); the result is the same
as attention over the contiguous sequence, which is what this module computes
by first rebuilding the contiguous K/V from the table.

Query head h reads KV head ``h // G`` with ``G = Hq / Hkv``: the query heads
are split into consecutive groups, one KV head per group (youngju.dev page,
section "GQA와 MQA").

Split-context decode (chunks of P tokens, each producing max / sum / normalised
partial output, merged by log-sum-exp) is not on the pages; it is the standard
decomposition softmax over a union of disjoint chunks, written out in
``split_partials`` and ``lse_merge``.
"""
from __future__ import annotations

import math

import numpy as np


def gather_context(store, layer, table, length, kv_head):
    """Contiguous ``(K[T][d], V[T][d])`` in float64 of one sequence and KV head.

    Logical token t lives in physical block ``table[t // B]`` at offset ``t % B``.
    """
    bs = store.block_size
    n_blocks = -(-int(length) // bs)
    ks, vs = [], []
    for j in range(n_blocks):
        kb, vb = store.block_values(layer, int(table[j]))
        ks.append(kb[kv_head])
        vs.append(vb[kv_head])
    k = np.concatenate(ks, axis=0)[:length]
    v = np.concatenate(vs, axis=0)[:length]
    return k, v


def _attend(q, k, v, scale):
    """softmax(k @ q * scale) @ v for one query vector, max-subtracted."""
    s = (k @ q) * scale
    m = np.max(s)
    p = np.exp(s - m)
    return (p @ v) / np.sum(p)


def decode(store, layer, q, block_tables, context_lens, scale=None):
    """Decode attention output ``[S][Hq][d]`` float64.

    ``q``: ``[S][Hq][d]`` (any float dtype; used exactly); ``block_tables[i]``
    lists sequence i's physical blocks; ``context_lens[i] >= 1`` tokens are
    attended (the newly written token included).
    """
    q = np.asarray(q, dtype=np.float64)
    n_seqs, n_q_heads, d = q.shape
    g = n_q_heads // store.kv_heads
    if scale is None:
        scale = 1.0 / math.sqrt(d)
    out = np.zeros((n_seqs, n_q_heads, d), dtype=np.float64)
    for i in range(n_seqs):
        length = int(context_lens[i])
        for kvh in range(store.kv_heads):
            k, v = gather_context(store, layer, block_tables[i], length, kvh)
            for h in range(kvh * g, (kvh + 1) * g):
                out[i, h] = _attend(q[i, h], k, v, scale)
    return out


def split_partials(store, layer, q, block_tables, context_lens, partition, scale=None):
    """Per chunk c of ``partition`` tokens: (m_c, l_c, o_c) for every (seq, q head).

    m_c = max of the chunk's scores, l_c = sum exp(s - m_c),
    o_c = sum exp(s - m_c) v / l_c.  Returns a list over sequences of
    ``(m[Hq][C], l[Hq][C], o[Hq][C][d])`` with C = ceil(T / partition).
    """
    q = np.asarray(q, dtype=np.float64)
    n_seqs, n_q_heads, d = q.shape
    g = n_q_heads // store.kv_heads
    if scale is None:
        scale = 1.0 / math.sqrt(d)
    result = []
    for i in range(n_seqs):
        length = int(context_lens[i])
        n_chunks = -(-length // partition)
        m = np.zeros((n_q_heads, n_chunks))
        lsum = np.zeros((n_q_heads, n_chunks))
        o = np.zeros((n_q_heads, n_chunks, d))
        for kvh in range(store.kv_heads):
            k, v = gather_context(store, layer, block_tables[i], length, kvh)
            for h in range(kvh * g, (kvh + 1) * g):
                s = (k @ q[i, h]) * scale
                for c in range(n_chunks):
                    lo, hi = c * partition, min((c + 1) * partition, length)
                    sc = s[lo:hi]
                    mc = np.max(sc)
                    pc = np.exp(sc - mc)
                    m[h, c] = mc
                    lsum[h, c] = np.sum(pc)
                    o[h, c] = (pc @ v[lo:hi]) / lsum[h, c]
        result.append((m, lsum, o))
    return result


def lse_merge(m, lsum, o):
    """Merge chunk partials of one (seq, head): out = sum_c w_c o_c / sum_c w_c,
    w_c = l_c * exp(m_c - max_c m_c)."""
    m = np.asarray(m, dtype=np.float64)
    w = np.asarray(lsum, dtype=np.float64) * np.exp(m - np.max(m))
    return (w[:, None] * np.asarray(o, dtype=np.float64)).sum(axis=0) / w.sum()


def multi_token(store, layer, q, query_start, block_tables, context_lens, scale=None):
    """Paged attention for several new query tokens per sequence (a prefill
    chunk, or one decode token), output ``[N][Hq][d]`` float64.

    Attention is causal: a token attends to itself and the tokens before it
    (youngju.dev page, section "핵심 원리: KV 캐시란 무엇인가"); batches may mix
    prefill chunks and decode tokens (iq-blog ch.4, the scheduler described
    in its vLLM architecture section).  Sequence i owns query rows
    ``query_start[i] .. query_start[i+1] - 1``: its last n_i tokens, whose K/V
    are already in the cache, so that row j (0-based within the sequence)
    sits at position ``T_i - n_i + j`` and attends to the first
    ``T_i - n_i + j + 1`` tokens through the block table.
    """
    q = np.asarray(q, dtype=np.float64)
    n_rows, n_q_heads, d = q.shape
    g = n_q_heads // store.kv_heads
    if scale is None:
        scale = 1.0 / math.sqrt(d)
    qs = [int(x) for x in query_start]
    if qs[0] != 0 or qs[-1] != n_rows or any(b < a for a, b in zip(qs, qs[1:])):
        raise ValueError("query_start must rise from 0 to the number of query rows")
    out = np.zeros((n_rows, n_q_heads, d), dtype=np.float64)
    for i in range(len(qs) - 1):
        n_i = qs[i + 1] - qs[i]
        if n_i == 0:
            continue
        length = int(context_lens[i])
        if length < n_i:
            raise ValueError(f"sequence {i}: {n_i} query tokens but a context of {length}")
        for kvh in range(store.kv_heads):
            k, v = gather_context(store, layer, block_tables[i], length, kvh)
            for j in range(n_i):
                visible = length - n_i + j + 1
                for h in range(kvh * g, (kvh + 1) * g):
                    out[qs[i] + j, h] = _attend(q[qs[i] + j, h], k[:visible], v[:visible], scale)
    return out
