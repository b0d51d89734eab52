// Device helpers shared by the cache kernels and the decode kernel: the fp8
// E4M3FN and int8 encoders and the store of one new token's K/V (one KV head)
// into its slot, i.e. the reshape-and-cache scatter (youngju.dev "KV cache and
// paged attention", section "PagedAttention: OS 가상 메모리식 관리" for slots;
// section "KV 양자화: FP8과 INT8" for the one-byte elements, int8 with a scale
// and a zero point).
#pragma once

#include <hip/hip_runtime.h>

#include <cstdint>

#include "layout.hpp"

namespace pa {

// OCP E4M3FN encode of an fp32 value: NaN -> 0x7F, |y| >= 448 -> +-448
// (saturation), otherwise round to nearest, ties to even mantissa code.
// Integer arithmetic on the fp32 bit pattern, so the result is exact.
__device__ inline uint32_t e4m3_encode(float y) {
  const uint32_t u = __float_as_uint(y);
  const uint32_t sign = (u >> 24) & 0x80u;
  const uint32_t a = u & 0x7FFFFFFFu;
  if (a > 0x7F800000u) return 0x7Fu;                // NaN
  if (a >= 0x43E00000u) return sign | 0x7Eu;        // >= 448.0f: saturate
  if (a < 0x3C800000u) {                            // < 2^-6: spacing 2^-9
    const float q = rintf(__uint_as_float(a) * 512.0f);  // exact scale, then RNE
    return sign | static_cast<uint32_t>(q);         // q in [0, 8]; 8 is 2^-6 (code 8)
  }
  const uint32_t e = (a >> 23) - 127u + 7u;         // biased e4m3 exponent, 1..15
  uint32_t keep = ((a >> 20) & 0x7u) | (e << 3);    // code before rounding
  const uint32_t rem = a & 0xFFFFFu;
  if (rem > 0x80000u || (rem == 0x80000u && (keep & 1u))) ++keep;  // carry into exponent is correct
  return sign | keep;
}

// int8 code of y = x * inv_scale: y rounded to the nearest integer (ties to
// even), plus the zero point, saturated to [-128, 127]; NaN gives the zero
// point and infinities saturate.  Returned as the stored byte c + 128.
__device__ inline uint32_t i8_encode_stored(float y, float zero) {
  float r = rintf(y);
  // NaN test on the bit pattern: it must hold where the compiler may assume
  // that no value is NaN (the decode kernels are built so).
  r = (__float_as_uint(r) & 0x7FFFFFFFu) > 0x7F800000u ? 0.0f : r;
  const float c = fminf(fmaxf(r + zero, -128.0f), 127.0f);
  return static_cast<uint32_t>(static_cast<int>(c) + 128);
}

// The stored byte of y = x * inv_scale in a pool of the given one-byte kind.
template <int KIND>
__device__ inline uint32_t encode_byte(float y, float zero) {
  if constexpr (KIND == kI8) return i8_encode_stored(y, zero);
  (void)zero;
  return e4m3_encode(y);
}

__device__ inline float half_bits_to_float(uint32_t bits) {
  return static_cast<float>(__builtin_bit_cast(_Float16, static_cast<uint16_t>(bits)));
}

// One wave stores token `slot` of KV head h of `layer`: lane l takes dims 2l
// and 2l+1 of k_src / v_src (fp16 [head_dim] each).  fp8 and int8 pools
// quantise with the (layer, head) inverse scales (and int8 zero points).  The
// slot must be inside the pool.
template <int KIND>
__device__ inline void store_token(const PoolGeom& g, int layer, int h, int slot,
                                   const _Float16* k_src, const _Float16* v_src, int lane) {
  constexpr int ELEM = kind_bytes(KIND);
  constexpr int X = 16 / ELEM;
  const int blk = slot / g.block_size, t = slot % g.block_size;
  uint8_t* kt = g.k_layer(layer) + static_cast<uint64_t>(blk) * g.block_stride +
                static_cast<uint64_t>(h) * g.tile_bytes;
  uint8_t* vt = g.v_layer(layer) + static_cast<uint64_t>(blk) * g.block_stride +
                static_cast<uint64_t>(h) * g.tile_bytes;
  const int d0 = 2 * lane;  // this lane's two dims
  const uint32_t kk = *reinterpret_cast<const uint32_t*>(k_src + d0);
  const uint32_t vv = *reinterpret_cast<const uint32_t*>(v_src + d0);
  const int bs = g.block_size;
  if constexpr (ELEM == 2) {
    // d0, d0+1 are adjacent inside one K chunk.
    *reinterpret_cast<uint32_t*>(kt + 2 * k_index(t, d0, bs, X, kHeadDim)) = kk;
    *reinterpret_cast<uint16_t*>(vt + 2 * v_index(t, d0, bs, X)) = static_cast<uint16_t>(vv);
    *reinterpret_cast<uint16_t*>(vt + 2 * v_index(t, d0 + 1, bs, X)) = static_cast<uint16_t>(vv >> 16);
  } else {
    const int lh = layer * g.kv_heads + h;
    const int lhs = g.layers * g.kv_heads;
    const float k_inv = g.scales[2 * lhs + lh];
    const float v_inv = g.scales[3 * lhs + lh];
    const float k_z = g.scales[4 * lhs + lh];
    const float v_z = g.scales[5 * lhs + lh];
    const uint32_t k0 = encode_byte<KIND>(half_bits_to_float(kk) * k_inv, k_z);
    const uint32_t k1 = encode_byte<KIND>(half_bits_to_float(kk >> 16) * k_inv, k_z);
    const uint32_t v0 = encode_byte<KIND>(half_bits_to_float(vv) * v_inv, v_z);
    const uint32_t v1 = encode_byte<KIND>(half_bits_to_float(vv >> 16) * v_inv, v_z);
    *reinterpret_cast<uint16_t*>(kt + k_index(t, d0, bs, X, kHeadDim)) = static_cast<uint16_t>(k0 | (k1 << 8));
    vt[v_index(t, d0, bs, X)] = static_cast<uint8_t>(v0);
    vt[v_index(t, d0 + 1, bs, X)] = static_cast<uint8_t>(v1);
  }
}

}  // namespace pa
