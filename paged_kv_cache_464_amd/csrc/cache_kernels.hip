// Cache-side kernels: the reshape-and-cache scatter of new tokens' K/V into
// their slots (fp16 copy or fp8 E4M3FN quantise), its inverse gather, and the
// whole-block copy used by copy-on-write.
//
// A slot is block * block_size + offset: the block table maps a sequence's
// logical block to a physical block and the offset inside the block is kept
// (youngju.dev "KV cache and paged attention", section "PagedAttention: OS
// 가상 메모리식 관리").  A shared block is duplicated before one sharer writes
// into it (same page, section "prefix 공유와 copy-on-write").
#include <hip/hip_runtime.h>

#include <cstdint>

#include "kernels.hpp"

namespace pa {
namespace {

constexpr int kWaves = 4;  // waves per 256-thread workgroup

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

template <int ELEM>
__global__ __launch_bounds__(256) void write_kv_kernel(PoolGeom g, int layer,
                                                       const _Float16* __restrict__ k_new,
                                                       const _Float16* __restrict__ v_new,
                                                       const int32_t* __restrict__ slots,
                                                       int n_tokens) {
  constexpr int X = 16 / ELEM;
  const int64_t wave = static_cast<int64_t>(blockIdx.x) * kWaves + (threadIdx.x >> 6);
  const int lane = threadIdx.x & 63;
  if (wave >= static_cast<int64_t>(n_tokens) * g.kv_heads) return;
  const int tok = static_cast<int>(wave / g.kv_heads);
  const int h = static_cast<int>(wave % g.kv_heads);
  const int slot = slots[tok];
  if (slot < 0) return;
  if (slot >= g.num_blocks * g.block_size) {
    if (lane == 0) atomicOr(g.status, kDevBadSlot);
    return;
  }
  const int blk = slot / g.block_size, t = slot % g.block_size;
  uint8_t* kt = g.k_layer(layer) + static_cast<uint64_t>(blk) * g.block_stride +
                static_cast<uint64_t>(h) * g.tile_bytes;
  uint8_t* vt = g.v_layer(layer) + static_cast<uint64_t>(blk) * g.block_stride +
                static_cast<uint64_t>(h) * g.tile_bytes;
  const int64_t src = (static_cast<int64_t>(tok) * g.kv_heads + h) * kHeadDim;
  const int d0 = 2 * lane;  // this lane's two dims
  const uint32_t kk = *reinterpret_cast<const uint32_t*>(k_new + src + d0);
  const uint32_t vv = *reinterpret_cast<const uint32_t*>(v_new + src + d0);
  const int bs = g.block_size;
  if constexpr (ELEM == 2) {
    // d0, d0+1 are adjacent inside one K chunk.
    *reinterpret_cast<uint32_t*>(kt + 2 * k_index(t, d0, bs, X, kHeadDim)) = kk;
    *reinterpret_cast<uint16_t*>(vt + 2 * v_index(t, d0, bs, X)) = static_cast<uint16_t>(vv);
    *reinterpret_cast<uint16_t*>(vt + 2 * v_index(t, d0 + 1, bs, X)) =
        static_cast<uint16_t>(vv >> 16);
  } else {
    const int lh = layer * g.kv_heads + h;
    const int lhs = g.layers * g.kv_heads;
    const float k_inv = g.scales[2 * lhs + lh];
    const float v_inv = g.scales[3 * lhs + lh];
    auto h2f = [](uint32_t bits) {
      return static_cast<float>(__builtin_bit_cast(_Float16, static_cast<uint16_t>(bits)));
    };
    const uint32_t k0 = e4m3_encode(h2f(kk) * k_inv), k1 = e4m3_encode(h2f(kk >> 16) * k_inv);
    const uint32_t v0 = e4m3_encode(h2f(vv) * v_inv), v1 = e4m3_encode(h2f(vv >> 16) * v_inv);
    *reinterpret_cast<uint16_t*>(kt + k_index(t, d0, bs, X, kHeadDim)) =
        static_cast<uint16_t>(k0 | (k1 << 8));
    vt[v_index(t, d0, bs, X)] = static_cast<uint8_t>(v0);
    vt[v_index(t, d0 + 1, bs, X)] = static_cast<uint8_t>(v1);
  }
}

template <int ELEM>
__global__ __launch_bounds__(256) void gather_kv_kernel(PoolGeom g, int layer,
                                                        const int32_t* __restrict__ slots,
                                                        int n_tokens, uint8_t* __restrict__ k_out,
                                                        uint8_t* __restrict__ v_out) {
  constexpr int X = 16 / ELEM;
  const int64_t wave = static_cast<int64_t>(blockIdx.x) * kWaves + (threadIdx.x >> 6);
  const int lane = threadIdx.x & 63;
  if (wave >= static_cast<int64_t>(n_tokens) * g.kv_heads) return;
  const int tok = static_cast<int>(wave / g.kv_heads);
  const int h = static_cast<int>(wave % g.kv_heads);
  const int slot = slots[tok];
  if (slot < 0) return;
  if (slot >= g.num_blocks * g.block_size) {
    if (lane == 0) atomicOr(g.status, kDevBadSlot);
    return;
  }
  const int blk = slot / g.block_size, t = slot % g.block_size;
  const uint8_t* kt = g.k_layer(layer) + static_cast<uint64_t>(blk) * g.block_stride +
                      static_cast<uint64_t>(h) * g.tile_bytes;
  const uint8_t* vt = g.v_layer(layer) + static_cast<uint64_t>(blk) * g.block_stride +
                      static_cast<uint64_t>(h) * g.tile_bytes;
  const int64_t dst = (static_cast<int64_t>(tok) * g.kv_heads + h) * kHeadDim * ELEM;
  const int d0 = 2 * lane;
  const int bs = g.block_size;
  if constexpr (ELEM == 2) {
    const uint32_t kk = *reinterpret_cast<const uint32_t*>(kt + 2 * k_index(t, d0, bs, X, kHeadDim));
    const uint32_t v0 = *reinterpret_cast<const uint16_t*>(vt + 2 * v_index(t, d0, bs, X));
    const uint32_t v1 = *reinterpret_cast<const uint16_t*>(vt + 2 * v_index(t, d0 + 1, bs, X));
    *reinterpret_cast<uint32_t*>(k_out + dst + 2 * d0) = kk;
    *reinterpret_cast<uint32_t*>(v_out + dst + 2 * d0) = v0 | (v1 << 16);
  } else {
    const uint16_t kk = *reinterpret_cast<const uint16_t*>(kt + k_index(t, d0, bs, X, kHeadDim));
    const uint32_t v0 = vt[v_index(t, d0, bs, X)];
    const uint32_t v1 = vt[v_index(t, d0 + 1, bs, X)];
    *reinterpret_cast<uint16_t*>(k_out + dst + d0) = kk;
    *reinterpret_cast<uint16_t*>(v_out + dst + d0) = static_cast<uint16_t>(v0 | (v1 << 8));
  }
}

constexpr int kMaxCopyPairs = 64;
struct CopyPairs {
  int32_t src[kMaxCopyPairs];
  int32_t dst[kMaxCopyPairs];
};

// One workgroup per (pair, layer, K|V): copies kv_heads tiles (contiguous).
__global__ __launch_bounds__(256) void copy_blocks_kernel(PoolGeom g, CopyPairs pairs) {
  const int pair = blockIdx.x / (2 * g.layers);
  const int lk = blockIdx.x % (2 * g.layers);  // layer * 2 + (0: K, 1: V)
  const int32_t s = pairs.src[pair], d = pairs.dst[pair];
  if (s < 0 || s >= g.num_blocks || d < 0 || d >= g.num_blocks) {
    if (threadIdx.x == 0) atomicOr(g.status, kDevBadBlock);
    return;
  }
  const uint8_t* from = g.base + static_cast<uint64_t>(lk) * g.half_stride +
                        static_cast<uint64_t>(s) * g.block_stride;
  uint8_t* to = g.base + static_cast<uint64_t>(lk) * g.half_stride +
                static_cast<uint64_t>(d) * g.block_stride;
  const uint64_t units = g.block_stride / 16;
  for (uint64_t i = threadIdx.x; i < units; i += blockDim.x) {
    reinterpret_cast<uint4*>(to)[i] = reinterpret_cast<const uint4*>(from)[i];
  }
}

}  // namespace

hipError_t launch_write_kv(const PoolGeom& g, int layer, const void* k_new, const void* v_new,
                           const int32_t* slots, int n_tokens, hipStream_t stream) {
  if (n_tokens <= 0) return hipSuccess;
  const int64_t waves = static_cast<int64_t>(n_tokens) * g.kv_heads;
  const dim3 grid(static_cast<unsigned>((waves + kWaves - 1) / kWaves));
  const auto* k = static_cast<const _Float16*>(k_new);
  const auto* v = static_cast<const _Float16*>(v_new);
  if (g.elem_bytes == 2)
    return launch_kernel(write_kv_kernel<2>, grid, dim3(256), stream, nullptr, nullptr, g, layer, k, v, slots, n_tokens);
  return launch_kernel(write_kv_kernel<1>, grid, dim3(256), stream, nullptr, nullptr, g, layer, k, v, slots, n_tokens);
}

hipError_t launch_gather_kv(const PoolGeom& g, int layer, const int32_t* slots, int n_tokens,
                            void* k_out, void* v_out, hipStream_t stream) {
  if (n_tokens <= 0) return hipSuccess;
  const int64_t waves = static_cast<int64_t>(n_tokens) * g.kv_heads;
  const dim3 grid(static_cast<unsigned>((waves + kWaves - 1) / kWaves));
  auto* ko = static_cast<uint8_t*>(k_out);
  auto* vo = static_cast<uint8_t*>(v_out);
  if (g.elem_bytes == 2)
    return launch_kernel(gather_kv_kernel<2>, grid, dim3(256), stream, nullptr, nullptr, g, layer, slots, n_tokens, ko, vo);
  return launch_kernel(gather_kv_kernel<1>, grid, dim3(256), stream, nullptr, nullptr, g, layer, slots, n_tokens, ko, vo);
}

hipError_t launch_copy_blocks(const PoolGeom& g, const int32_t* src, const int32_t* dst, int n,
                              hipStream_t stream) {
  for (int base = 0; base < n; base += kMaxCopyPairs) {
    CopyPairs p;
    const int m = (n - base) < kMaxCopyPairs ? (n - base) : kMaxCopyPairs;
    for (int i = 0; i < kMaxCopyPairs; ++i) {
      p.src[i] = i < m ? src[base + i] : -1;
      p.dst[i] = i < m ? dst[base + i] : -1;
    }
    const hipError_t e = launch_kernel(copy_blocks_kernel, dim3(m * 2 * g.layers), dim3(256), stream, nullptr,
                                       nullptr, g, p);
    if (e != hipSuccess) return e;
  }
  return hipSuccess;
}

}  // namespace pa
