"""Closed forms the pages print, written out.

Each function is pinned in tests against the numbers the pages print for
their worked examples (tests/golden/*.json).
"""
from __future__ import annotations


def kv_bytes(layers, kv_heads, head_dim, dtype_bytes, tokens):
    """KV bytes = 2 (K and V) x layers x KV heads x head_dim x bytes x tokens.

    openakashic KV-cache failure-modes note, Key Points (capacity estimate);
    youngju.dev "KV cache and paged attention", sections "KV 캐시는 왜 메모리를
    먹는가" and "메모리 산수 예시".
    """
    return 2 * layers * kv_heads * head_dim * dtype_bytes * tokens


def internal_fragmentation(tokens, max_tokens):
    """Contiguous pre-allocation waste 1 - T / T_max (iq-blog ch.4, "낭비의 구조")."""
    return 1.0 - tokens / max_tokens


def reservation_waste(used, reserved):
    """Fraction of a reservation never used (iq-blog ch.4, "낭비의 구조")."""
    return 1.0 - used / reserved


def paged_waste_bound(block_size, min_tokens):
    """Theorem 1 bound: wasted / allocated <= B_s / T (iq-blog ch.4, Theorem 1)."""
    return block_size / min_tokens


def tail_waste_tokens(tokens, block_size):
    """Empty slots in a request's last block: ceil(T / B) * B - T (<= B - 1)."""
    return -(-tokens // block_size) * block_size - tokens


def prefix_savings(requests, prefix, mean_suffix):
    """(R - 1) p / (R (p + s)) (iq-blog ch.4, "Prefix Caching")."""
    return (requests - 1) * prefix / (requests * (prefix + mean_suffix))


def shared_copy_savings(requests):
    """1 - 1/R when R requests share one copy (iq-blog ch.4, "OS Paging에서 가져온 해법")."""
    return 1.0 - 1.0 / requests


def kv_head_ratio(kv_heads, reference_heads):
    """KV size relative to a layout with ``reference_heads`` KV heads (youngju.dev, "GQA와 MQA")."""
    return kv_heads / reference_heads


def block_table_bytes(requests, blocks_per_request, entry_bytes=4):
    """Block-table metadata size (iq-blog ch.4, "vLLM의 4-Layer 통합 아키텍처")."""
    return requests * blocks_per_request * entry_bytes
