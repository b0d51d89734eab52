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

int8 storage (same section: one byte per element, with a scale and a zero
point) keeps signed codes with one fp32 scale and one integer zero point per
(layer, KV head) for K and for V: ``value = (code - zero) * scale`` (see
``int8``).  Every int8 code is a number, so int8 blocks carry a written-mask
instead, and never-written slots read as NaN.
"""
from __future__ import annotations

import numpy as np

from . import fp8 as _fp8
from . import int8 as _int8


class OracleKVStore:
    def __init__(self, layers, num_blocks, kv_heads, block_size, head_dim, dtype="fp16",
                 k_scales=None, v_scales=None, k_zeros=None, v_zeros=None):
        self.layers = int(layers)
        self.num_blocks = int(num_blocks)
        self.kv_heads = int(kv_heads)
        self.block_size = int(block_size)
        self.head_dim = int(head_dim)
        if dtype not in ("fp16", "fp8", "int8"):
            raise ValueError(dtype)
        self.dtype = dtype
        lh = (self.layers, self.kv_heads)
        self.k_scales = self.v_scales = self.k_zeros = self.v_zeros = None
        if dtype in ("fp8", "int8"):
            self.k_scales = np.asarray(k_scales, dtype=np.float32).reshape(lh)
            self.v_scales = np.asarray(v_scales, dtype=np.float32).reshape(lh)
        if dtype == "int8":
            self.k_zeros = np.asarray(k_zeros, dtype=np.int64).reshape(lh)
            self.v_zeros = np.asarray(v_zeros, dtype=np.int64).reshape(lh)
            if (np.abs(self.k_zeros + 0.5) > 128).any() or (np.abs(self.v_zeros + 0.5) > 128).any():
                raise ValueError("int8 zero points must lie in [-128, 127]")
        self._blocks = [dict() for _ in range(self.layers)]  # block id -> [2][Hkv][B][d]
        self._written = [dict() for _ in range(self.layers)]  # int8: block id -> bool mask

    def _new_block(self):
        shape = (2, self.kv_heads, self.block_size, self.head_dim)
        if self.dtype == "fp16":
            return np.full(shape, np.nan, dtype=np.float16)
        if self.dtype == "int8":
            return np.zeros(shape, dtype=np.int8)
        return np.full(shape, _fp8.E4M3_NAN_CODE, dtype=np.uint8)

    def _block(self, layer, b):
        if not 0 <= b < self.num_blocks:
            raise IndexError(f"block {b} outside pool of {self.num_blocks}")
        blk = self._blocks[layer].get(b)
        if blk is None:
            blk = self._new_block()
            self._blocks[layer][b] = blk
            if self.dtype == "int8":
                self._written[layer][b] = np.zeros(blk.shape, dtype=bool)
        return blk

    def write(self, layer, k_new, v_new, slots):
        """Store token t's K/V (``[n][Hkv][d]`` fp16) at ``slots[t]``; slots < 0 are skipped."""
        k_new = np.asarray(k_new, dtype=np.float16)
        v_new = np.asarray(v_new, dtype=np.float16)
        slots = np.asarray(slots, dtype=np.int64)
        if self.dtype == "fp8":
            k_inv = _fp8.inverse_scale(self.k_scales[layer])[:, None]  # [Hkv][1]
            v_inv = _fp8.inverse_scale(self.v_scales[layer])[:, None]
        if self.dtype == "int8":
            k_inv = _int8.inverse_scale(self.k_scales[layer])[:, None]  # [Hkv][1]
            v_inv = _int8.inverse_scale(self.v_scales[layer])[:, None]
            k_z = self.k_zeros[layer][:, None]
            v_z = self.v_zeros[layer][:, None]
        for t, slot in enumerate(slots):
            if slot < 0:
                continue
            blk = self._block(layer, int(slot) // self.block_size)
            off = int(slot) % self.block_size
            if self.dtype == "fp16":
                blk[0, :, off, :] = k_new[t]
                blk[1, :, off, :] = v_new[t]
            elif self.dtype == "int8":
                blk[0, :, off, :] = _int8.quantize(k_new[t], k_inv, k_z)
                blk[1, :, off, :] = _int8.quantize(v_new[t], v_inv, v_z)
                self._written[layer][int(slot) // self.block_size][:, :, off, :] = True
            else:
                blk[0, :, off, :] = _fp8.quantize(k_new[t], k_inv)
                blk[1, :, off, :] = _fp8.quantize(v_new[t], v_inv)

    def copy_block(self, src, dst):
        """Copy-on-write duplicate: every layer, K and V, all slots of the block."""
        for layer in range(self.layers):
            self._block(layer, dst)[...] = self._block(layer, src)
            if self.dtype == "int8":
                self._written[layer][dst][...] = self._written[layer][src]

    def read_slots(self, layer, slots):
        """Raw stored K and V of each slot: ``[n][Hkv][d]`` fp16 values or uint8 codes."""
        slots = np.asarray(slots, dtype=np.int64)
        dt = {"fp16": np.float16, "fp8": np.uint8, "int8": np.int8}[self.dtype]
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
        if self.dtype == "int8":
            k = _int8.decode(blk[0], ks, self.k_zeros[layer][:, None, None])
            v = _int8.decode(blk[1], vs, self.v_zeros[layer][:, None, None])
            w = self._written[layer][b]
            return np.where(w[0], k, np.nan), np.where(w[1], v, np.nan)
        return _fp8.decode(blk[0]) * ks, _fp8.decode(blk[1]) * vs
