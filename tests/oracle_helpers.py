"""Helpers that drive the oracle on synthetic data (test-side only)."""
from __future__ import annotations

import numpy as np

from oracle.allocator import OracleAllocator
from oracle.kvstore import OracleKVStore


def build_paged(k_dense, v_dense, lens, block_size, num_blocks, free_order=None,
                dtype="fp16", k_scales=None, v_scales=None, k_zeros=None, v_zeros=None):
    """Allocate each sequence's tokens through the oracle allocator and write them.

    ``k_dense[i]``: ``[T_i][Hkv][d]`` fp16 for sequence i (one layer).
    Returns (allocator, store, seq ids, slots per seq).
    """
    hkv, d = k_dense[0].shape[1], k_dense[0].shape[2]
    alloc = OracleAllocator(num_blocks, block_size, free_order)
    store = OracleKVStore(1, num_blocks, hkv, block_size, d, dtype, k_scales, v_scales,
                          k_zeros, v_zeros)
    seqs, all_slots = [], []
    for i, t in enumerate(lens):
        s = alloc.seq_create()
        slots, _ = alloc.alloc(s, int(t))
        store.write(0, k_dense[i][:t], v_dense[i][:t], slots)
        seqs.append(s)
        all_slots.append(slots)
    return alloc, store, seqs, all_slots


def tables_of(alloc, seqs):
    width = max(len(alloc.tables[s]) for s in seqs)
    rows, lens = alloc.block_tables(seqs, width)
    return np.asarray(rows, dtype=np.int64), np.asarray(lens, dtype=np.int64)
