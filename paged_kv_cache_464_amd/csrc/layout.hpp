// Byte layout of the KV block pool in HBM.
//
// Pool: [layer][K|V][block][kv_head][tile].  A tile is one (block, KV head):
// B tokens x D dims (D = head_dim, 64 or 128), stored in the order the decode
// kernel's 64-lane loads consume it, so that every 16-byte lane load of one
// wave lands in a contiguous 1 KiB run (512 B for block_size 8) and the
// registers it fills are already the MFMA operand fragments:
//
//  K tile: 16-byte chunks of X consecutive dims (X = 8 fp16 / 16 fp8) of one
//    token; for a run of TR = min(B, 16) tokens the chunk index is the outer
//    loop and the token the inner one:
//        k_index(t, dim) = (((t / TR) * (D / X) + dim / X) * TR + t % TR) * X + dim % X
//    Lane (g, n) of a 16-token step, load j, reads chunk j*4+g of token n.
//
//  V tile: 4-token x 16-dim sub-tiles.  With r = dim / 16, n = dim % 16,
//    tg = t / 4, tt = t % 4 and R = X / 4 dim sub-tiles per 16 bytes:
//        v_index(t, dim) = (((r / R) * (B / 4) + tg) * 16 + n) * X + (r % R) * 4 + tt
//    Lane (g, n), load j, reads the 4 tokens 4g..4g+3 for dims r*16 + n of
//    R consecutive r: exactly the A-operand fragment of a 16x16x16 MFMA with
//    V^T as the left matrix.
#pragma once

#include <cstdint>

namespace pa {

// head_dim values the kernels are built for (a template parameter of every
// kernel that touches a tile).
constexpr int kHeadDimSmall = 64, kHeadDimLarge = 128;

// Element kinds of a pool (the values of PA_DTYPE_*): fp16, fp8 E4M3FN codes,
// and int8 codes with a scale and a zero point.  The pool keeps an int8 code
// c as the byte c + 128 (offset binary), which the decode kernel widens to
// fp16 without a sign step; the gather returns c itself.
constexpr int kF16 = 0, kF8 = 1, kI8 = 2;
__host__ __device__ constexpr int kind_bytes(int kind) { return kind == kF16 ? 2 : 1; }

__host__ __device__ constexpr int chunk_elems(int elem_bytes) { return 16 / elem_bytes; }

__host__ __device__ inline int k_index(int t, int dim, int block_size, int x, int head_dim) {
  const int tr = block_size < 16 ? block_size : 16;
  return (((t / tr) * (head_dim / x) + dim / x) * tr + t % tr) * x + dim % x;
}

__host__ __device__ inline int v_index(int t, int dim, int block_size, int x) {
  const int rr = x / 4;
  const int r = dim / 16, n = dim % 16, tg = t / 4, tt = t % 4;
  return (((r / rr) * (block_size / 4) + tg) * 16 + n) * x + (r % rr) * 4 + tt;
}

// Geometry of one bound pool, passed by value to every kernel.
struct PoolGeom {
  uint8_t* base;           // device base of the pool
  int32_t layers, kv_heads, head_dim, block_size, num_blocks, elem_bytes;
  int32_t kind;            // kF16, kF8 or kI8
  uint64_t tile_bytes;     // block_size * head_dim * elem_bytes
  uint64_t block_stride;   // kv_heads * tile_bytes (one block of one layer's K or V)
  uint64_t half_stride;    // num_blocks * block_stride (one layer's K pool)
  float* scales;           // [6][layers][kv_heads]: k_scale, v_scale, k_inv, v_inv,
                           // k_zero, v_zero (int8 zero points, exact in fp32)
  uint32_t* status;        // PA_DEV_* bits

  __host__ __device__ uint8_t* k_layer(int layer) const {
    return base + static_cast<uint64_t>(layer) * 2u * half_stride;
  }
  __host__ __device__ uint8_t* v_layer(int layer) const { return k_layer(layer) + half_stride; }
};

}  // namespace pa
