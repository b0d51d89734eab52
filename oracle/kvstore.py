"""Reference block-pooled K/V store and the reshape-and-cache write.

Logical layout (the oracle's own; it need not match the GPU's byte layout):
per layer, per physical block, arrays ``K[Hkv][B][d]`` and ``V[Hkv][B][d]``.
A token's K/V go to block ``slot // B`` at offset ``slot % B`` (the block table
maps a logical block to a physical one and keeps the in-block offset;
youngju.dev "KV cache and paged attention", section "PagedAttention: OS 가상
메모리식 관리").  Blocks are materialised lazily and start as NaN (fp16) or
the NaN code 0x7F (fp8) so that any read of a never-written slot shows up.

fp8 storage (same page, section "KV 양자화: FP8과 INT8": one byte per element)
uses E4M3FN codes with one fp32 scale per (layer, KV head) for K and one for
V: ``code = encode(f32(x) * f32(1 / scale))`` and ``value = decode(code) * scale``.
"""
from __future__ import annotations

import numpy as np

from . import fp8 as _fp8


class OracleKVStore:
    def __init__(self, layers, num_blocks, kv_heads, block_size, head_dim, dtype="fp16",
                 k_scales=None, v_scales=None):
        self.layers = int(layers)
        self.num_blocks = int(num_blocks)
        self.kv_heads = int(kv_heads)
        self.block_size = int(block_size)
        self.head_dim = int(head_dim)
        if dtype not in ("fp16", "fp8"):
            raise ValueError(dtype)
        self.dtype = dtype
        if dtype == "fp8":
            ks = np.asarray(k_scales, dtype=np.float32).reshape(self.layers, self.kv_heads)
            vs = np.asarray(v_scales, dtype=np.float32).reshape(self.layers, self.kv_heads)
            self.k_scales, self.v_scales = ks, vs
        else:
            self.k_scales = self.v_scales = None
        self._blocks = [dict() for _ in range(self.layers)]  # block id -> [2][Hkv][B][d]

    def _new_block(self):
        shape = (2, self.kv_heads, self.block_size, self.head_dim)
        if self.dtype == "fp16":
            return np.full(shape, np.nan, dtype=np.float16)
        return np.full(shape, _fp8.E4M3_NAN_CODE, dtype=np.uint8)

    def _block(self, layer, b):
        if not 0 <= b < self.num_blocks:
            raise IndexError(f"block {b} outside pool of {self.num_blocks}")
        blk = self._blocks[layer].get(b)
        if blk is None:
            blk = self._new_block()
            self._blocks[layer][b] = blk
        return blk

    def write(self, layer, k_new, v_new, slots):
        """Store token t's K/V (``[n][Hkv][d]`` fp16) at ``slots[t]``; slots < 0 are skipped."""
        k_new = np.asarray(k_new, dtype=np.float16)
        v_new = np.asarray(v_new, dtype=np.float16)
        slots = np.asarray(slots, dtype=np.int64)
        if self.dtype == "fp8":
            k_inv = _fp8.inverse_scale(self.k_scales[layer])[:, None]  # [Hkv][1]
            v_inv = _fp8.inverse_scale(self.v_scales[layer])[:, None]
        for t, slot in enumerate(slots):
            if slot < 0:
                continue
            blk = self._block(layer, int(slot) // self.block_size)
            off = int(slot) % self.block_size
            if self.dtype == "fp16":
                blk[0, :, off, :] = k_new[t]
                blk[1, :, off, :] = v_new[t]
            else:
                blk[0, :, off, :] = _fp8.quantize(k_new[t], k_inv)
                blk[1, :, off, :] = _fp8.quantize(v_new[t], v_inv)

    def copy_block(self, src, dst):
        """Copy-on-write duplicate: every layer, K and V, all slots of the block."""
        for layer in range(self.layers):
            self._block(layer, dst)[...] = self._block(layer, src)

    def read_slots(self, layer, slots):
        """Raw stored K and V of each slot: ``[n][Hkv][d]`` fp16 values or uint8 codes."""
        slots = np.asarray(slots, dtype=np.int64)
        dt = np.float16 if self.dtype == "fp16" else np.uint8
        k = np.empty((len(slots), self.kv_heads, self.head_dim), dtype=dt)
        v = np.empty_like(k)
        for t, slot in enumerate(slots):
            blk = self._block(layer, int(slot) // self.block_size)
            off = int(slot) % self.block_size
            k[t] = blk[0, :, off, :]
            v[t] = blk[1, :, off, :]
        return k, v

    def block_values(self, layer, b):
        """Dequantised float64 ``(K[Hkv][B][d], V[Hkv][B][d])`` of physical block ``b``."""
        blk = self._block(layer, b)
        if self.dtype == "fp16":
            return blk[0].astype(np.float64), blk[1].astype(np.float64)
        ks = self.k_scales[layer].astype(np.float64)[:, None, None]
        vs = self.v_scales[layer].astype(np.float64)[:, None, None]
        return _fp8.decode(blk[0]) * ks, _fp8.decode(blk[1]) * vs
