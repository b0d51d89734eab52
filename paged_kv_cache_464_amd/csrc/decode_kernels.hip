// Paged decode attention on gfx950.
//
// For every sequence i and query head h: out = softmax(q K^T * scale) V over
// the sequence's T_i cached tokens (youngju.dev "KV cache and paged
// attention", section "핵심 원리: KV 캐시란 무엇인가"), where the K/V of
// logical token t sit in physical block table[t / B] at offset t % B and the
// kernel follows the block table to gather them (iq-blog ch.4, section
// "PagedAttention 알고리즘").  Query head h reads KV head h / G (youngju.dev
// page, section "GQA와 MQA").
//
// Mapping to CDNA4:
//  * one workgroup of four waves per (sequence, KV head, context chunk); its
//    waves take interleaved 16-token steps of the chunk;
//  * K/V are read with nontemporal 16-byte loads: each byte is used once per
//    launch, and on MI355X such loads sustain about 11% more bandwidth over
//    randomly placed 4 KiB tiles than ordinary ones;
//  * each step loads the K and V tiles of 16 tokens with 16-byte lane loads
//    (one contiguous 1 KiB run per load instruction), directly in the
//    register layout of the MFMA operands -- no LDS round trip;
//  * S^T[token][head] = K * Q^T with v_mfma_f32_16x16x32_f16 (rows = 16 tokens,
//    columns = the G query heads of the KV head, padded to 16), so the K tile
//    is read once for all G heads of the group;
//  * online softmax in fp32 (base-2 exponent), with the per-head maximum
//    exchanged across the four 16-lane groups by two xor shuffles;
//  * O^T[dim][head] += V^T * P^T with v_mfma_f32_16x16x16_f16, P in fp16;
//  * the waves merge their (max, sum, O) through LDS at the end, and the
//    workgroup writes either the final fp16 output or one chunk's partials.
// fp8 (E4M3FN) tiles are widened to fp16 in registers (exactly: every E4M3
// value times 2^-8 is an fp16 value); the 2^8 and the per-(layer, KV head)
// scales are folded into the score and output multipliers.
#include <hip/hip_ext.h>
#include <hip/hip_runtime.h>

#include <cstdint>

#include "kernels.hpp"

namespace pa {
namespace {

typedef _Float16 f16x8 __attribute__((ext_vector_type(8)));
typedef _Float16 f16x4 __attribute__((ext_vector_type(4)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));

constexpr float kLog2e = 1.4426950408889634f;
constexpr int kD = kHeadDim;
constexpr int kSmoStride = kD + 4;  // padded LDS row of the merge buffer
constexpr int kDecodeWaves = 4;     // waves per decode workgroup

// Two E4M3FN bytes (bits 8..15 and 24..31 of x) -> two fp16 equal to value * 2^-8:
// sign to bit 15, exponent+mantissa bits shifted into place.  Exact for every
// finite code, normal and subnormal.
__device__ inline uint32_t e4m3x2_to_f16x2_scaled(uint32_t x) {
  return (x & 0x80008000u) | ((x >> 1) & 0x3F803F80u);
}
// Bytes b0..b3 of w -> 4 fp16 (x 2^-8) in two dwords.
__device__ inline u32x2 e4m3x4_to_f16x4(uint32_t w) {
  const uint32_t lo = ((w & 0x000000FFu) << 8) | ((w & 0x0000FF00u) << 16);  // [0, b0, 0, b1]
  const uint32_t hi = ((w & 0x00FF0000u) >> 8) | (w & 0xFF000000u);          // [0, b2, 0, b3]
  return u32x2{e4m3x2_to_f16x2_scaled(lo), e4m3x2_to_f16x2_scaled(hi)};
}

template <int ELEM>
struct StepRegs {
  static constexpr int kLoads = 2 * ELEM;  // 16-byte loads per lane for K (and for V)
  u32x4 k[kLoads];
  u32x4 v[kLoads];
};

template <int ELEM, int BS, int NT, bool PARTIAL, int NW>
__global__ __launch_bounds__(NW * 64) void decode_kernel(PoolGeom g, DecodeLaunch p) {
  constexpr int X = 16 / ELEM;             // elements per 16-byte chunk
  constexpr int NLD = StepRegs<ELEM>::kLoads;
  constexpr int R = X / 4;                 // V dim sub-tiles per 16-byte load
  constexpr int NCOL = NT * 16;

  const int lane = threadIdx.x & 63;
  const int w = threadIdx.x >> 6;
  const int gq = lane >> 4;  // 16-lane group
  const int n = lane & 15;

  int wg = blockIdx.x;
  const int part = wg % p.num_partitions;
  wg /= p.num_partitions;
  const int kvh = wg % g.kv_heads;
  const int seq = wg / g.kv_heads;
  const int group = p.num_q_heads / g.kv_heads;

  const int32_t* trow = p.tables + static_cast<int64_t>(seq) * p.max_blocks;
  const int start = part * p.partition_tokens;
  // Block ids of this wave's steps, one per lane (lane L: wave-step c0 + L),
  // refilled every 64 steps.  Entries are clamped to the table width only, so
  // the first load is issued together with the context length instead of
  // after it; ids of steps past the end are never used.
  int tl_lo = 0, tl_hi = 0;
  auto load_ids = [&](int c0) {
    const int64_t b = (start + 16ll * (w + NW * (c0 + lane))) / BS;
    const int64_t last = p.max_blocks - 1;
    tl_lo = trow[b < last ? b : last];
    if constexpr (BS == 8) tl_hi = trow[b + 1 < last ? b + 1 : last];
  };
  load_ids(0);

  int T = p.lens[seq];
  const int t_cap = p.max_blocks * BS;
  if (T < 1 || T > t_cap) {
    if (threadIdx.x == 0) atomicOr(g.status, kDevBadLen);
    T = T < 0 ? 0 : (T > t_cap ? t_cap : T);
  }
  if (T == 0) {
    if constexpr (!PARTIAL) {
      // Nothing to attend to: defined output of zeros.
      for (int i = threadIdx.x; i < group * kD; i += NW * 64) {
        reinterpret_cast<_Float16*>(p.out)[(static_cast<int64_t>(seq) * p.num_q_heads +
                                            kvh * group) * kD + i] = 0;
      }
    }
    return;
  }
  if (start >= T) return;
  const int end = (start + p.partition_tokens < T) ? start + p.partition_tokens : T;
  const int nsteps = (end - start + 15) >> 4;
  const int my_steps = (w < nsteps) ? (nsteps - w + NW - 1) / NW : 0;

  // ---- scales ----------------------------------------------------------------
  float qk_mul = p.scale * kLog2e;
  float out_mul = 1.0f;
  if constexpr (ELEM == 1) {
    const int lhs = g.layers * g.kv_heads;
    const int lh = p.layer * g.kv_heads + kvh;
    qk_mul *= g.scales[lh] * 256.0f;
    out_mul = g.scales[lhs + lh] * 256.0f;
  }

  // ---- Q^T operands: lane (gq, n) holds head column n, 8 dims per MFMA -------
  f16x8 qop[NT][4];
  const _Float16* qs = static_cast<const _Float16*>(p.q) +
                       static_cast<int64_t>(seq) * p.num_q_heads * kD;
#pragma unroll
  for (int nt = 0; nt < NT; ++nt) {
    const int col = nt * 16 + n;
    const bool valid = col < group;
    const _Float16* qh = qs + static_cast<int64_t>(kvh * group + (valid ? col : 0)) * kD;
#pragma unroll
    for (int u = 0; u < 4; ++u) {
      const int dim0 = (ELEM == 2) ? (u * 4 + gq) * 8 : ((u >> 1) * 4 + gq) * 16 + (u & 1) * 8;
      f16x8 v = *reinterpret_cast<const f16x8*>(qh + dim0);
      qop[nt][u] = valid ? v : f16x8{0, 0, 0, 0, 0, 0, 0, 0};
    }
  }

  // ---- per-lane byte offsets inside the tiles --------------------------------
  uint32_t koff[NLD], voff[NLD];
#pragma unroll
  for (int j = 0; j < NLD; ++j) {
    const int c = j * 4 + gq;  // K chunk of this lane for load j
    if constexpr (BS == 8) {
      koff[j] = ((c * 8 + (n & 7)) * X) * ELEM;
      voff[j] = (((j * 2 + (gq & 1)) * 16 + n) * X) * ELEM;
    } else {
      koff[j] = ((c * 16 + n) * X) * ELEM;
      voff[j] = (((j * (BS / 4) + gq) * 16 + n) * X) * ELEM;
    }
  }

  const uint8_t* kbase = g.k_layer(p.layer) + static_cast<uint64_t>(kvh) * g.tile_bytes;
  const uint8_t* vbase = g.v_layer(p.layer) + static_cast<uint64_t>(kvh) * g.tile_bytes;

  f32x4 oacc[NT][8];
  float m_run[NT], l_part[NT];
#pragma unroll
  for (int nt = 0; nt < NT; ++nt) {
    m_run[nt] = -__builtin_inff();
    l_part[nt] = 0.0f;
#pragma unroll
    for (int r = 0; r < 8; ++r) oacc[nt][r] = f32x4{0, 0, 0, 0};
  }

  uint32_t bad = 0;

  auto phys_ok = [&](int b) -> int {
    if (static_cast<uint32_t>(b) >= static_cast<uint32_t>(g.num_blocks)) {
      bad |= kDevBadBlock;
      return 0;
    }
    return b;
  };

  // K/V are streamed once per launch: nontemporal loads keep them from
  // displacing anything in the caches.
  auto ld16 = [](const uint8_t* a) {
    return __builtin_nontemporal_load(reinterpret_cast<const u32x4*>(a));
  };
  auto issue = [&](StepRegs<ELEM>& r, int i_in_chunk, int tb) {
    if constexpr (BS == 8) {
      const int b0 = phys_ok(__builtin_amdgcn_readlane(tl_lo, i_in_chunk));
      // The second block of the step exists only if its first token does.
      const int b1 = (tb + 8 < T) ? phys_ok(__builtin_amdgcn_readlane(tl_hi, i_in_chunk)) : b0;
      const uint8_t* kp = kbase + static_cast<uint64_t>(n < 8 ? b0 : b1) * g.block_stride;
      const uint8_t* vp = vbase + static_cast<uint64_t>(gq < 2 ? b0 : b1) * g.block_stride;
#pragma unroll
      for (int j = 0; j < NLD; ++j) {
        r.k[j] = ld16(kp + koff[j]);
        r.v[j] = ld16(vp + voff[j]);
      }
    } else {
      const int b = phys_ok(__builtin_amdgcn_readlane(tl_lo, i_in_chunk));
      uint64_t koff_sub = 0, voff_sub = 0;
      if constexpr (BS == 32) {
        const int sub = (tb >> 4) & 1;
        koff_sub = static_cast<uint64_t>(sub) * 16 * kD * ELEM;
        voff_sub = static_cast<uint64_t>(sub) * 4 * 16 * X * ELEM;
      }
      const uint8_t* kp = kbase + static_cast<uint64_t>(b) * g.block_stride + koff_sub;
      const uint8_t* vp = vbase + static_cast<uint64_t>(b) * g.block_stride + voff_sub;
#pragma unroll
      for (int j = 0; j < NLD; ++j) {
        r.k[j] = ld16(kp + koff[j]);
        r.v[j] = ld16(vp + voff[j]);
      }
    }
  };

  auto compute = [&](StepRegs<ELEM>& r, int tb) {
    // S^T = K Q^T
    f32x4 s[NT];
#pragma unroll
    for (int nt = 0; nt < NT; ++nt) s[nt] = f32x4{0, 0, 0, 0};
#pragma unroll
    for (int u = 0; u < 4; ++u) {
      f16x8 kop;
      if constexpr (ELEM == 2) {
        kop = __builtin_bit_cast(f16x8, r.k[u]);
      } else {
        const u32x4 raw = r.k[u >> 1];
        const u32x2 a = e4m3x4_to_f16x4((u & 1) ? raw[2] : raw[0]);
        const u32x2 b = e4m3x4_to_f16x4((u & 1) ? raw[3] : raw[1]);
        kop = __builtin_bit_cast(f16x8, u32x4{a[0], a[1], b[0], b[1]});
      }
#pragma unroll
      for (int nt = 0; nt < NT; ++nt)
        s[nt] = __builtin_amdgcn_mfma_f32_16x16x32_f16(kop, qop[nt][u], s[nt], 0, 0, 0);
    }
    // Scores of tokens tb + 4*gq + e for head column n; mask the tail.
    const bool tail = tb + 16 > T;
    const int valid_here = T - (tb + 4 * gq);  // tokens of this lane's 4 that exist
    float mx[NT], mnew[NT];
    bool grow = false;
#pragma unroll
    for (int nt = 0; nt < NT; ++nt) {
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        float x = s[nt][e] * qk_mul;
        if (tail && e >= valid_here) x = -__builtin_inff();
        s[nt][e] = x;
      }
      float m = fmaxf(fmaxf(s[nt][0], s[nt][1]), fmaxf(s[nt][2], s[nt][3]));
      m = fmaxf(m, __shfl_xor(m, 16));
      m = fmaxf(m, __shfl_xor(m, 32));
      mx[nt] = m;
      mnew[nt] = fmaxf(m_run[nt], m);
      grow |= mnew[nt] > m_run[nt];
    }
    if (__any(grow)) {
#pragma unroll
      for (int nt = 0; nt < NT; ++nt) {
        const float alpha = exp2f(m_run[nt] - mnew[nt]);
        l_part[nt] *= alpha;
#pragma unroll
        for (int rr = 0; rr < 8; ++rr) oacc[nt][rr] *= alpha;
        m_run[nt] = mnew[nt];
      }
    }
    f16x4 pop[NT];
#pragma unroll
    for (int nt = 0; nt < NT; ++nt) {
      float pe[4];
#pragma unroll
      for (int e = 0; e < 4; ++e) pe[e] = exp2f(s[nt][e] - m_run[nt]);
      l_part[nt] += (pe[0] + pe[1]) + (pe[2] + pe[3]);
      pop[nt] = f16x4{(_Float16)pe[0], (_Float16)pe[1], (_Float16)pe[2], (_Float16)pe[3]};
    }
    // Unused slots of the last block may hold anything (NaN included): zero them,
    // since 0 * NaN would poison the product.
    if (tail) {
      const int vc = valid_here < 0 ? 0 : (valid_here > 4 ? 4 : valid_here);
#pragma unroll
      for (int j = 0; j < NLD; ++j) {
        if constexpr (ELEM == 2) {
          const uint32_t m01 = (vc > 0 ? 0x0000FFFFu : 0u) | (vc > 1 ? 0xFFFF0000u : 0u);
          const uint32_t m23 = (vc > 2 ? 0x0000FFFFu : 0u) | (vc > 3 ? 0xFFFF0000u : 0u);
          r.v[j] &= u32x4{m01, m23, m01, m23};
        } else {
          const uint32_t mb = vc >= 4 ? 0xFFFFFFFFu : ((1u << (8 * vc)) - 1u);
          r.v[j] &= u32x4{mb, mb, mb, mb};
        }
      }
    }
    // O^T += V^T P^T, one 16-dim sub-tile at a time.
#pragma unroll
    for (int rr = 0; rr < 8; ++rr) {
      f16x4 vop;
      if constexpr (ELEM == 2) {
        const u32x4 raw = r.v[rr >> 1];
        vop = __builtin_bit_cast(f16x4, (rr & 1) ? u32x2{raw[2], raw[3]} : u32x2{raw[0], raw[1]});
      } else {
        const u32x4 raw = r.v[rr >> 2];
        vop = __builtin_bit_cast(f16x4, e4m3x4_to_f16x4(raw[rr & 3]));
      }
#pragma unroll
      for (int nt = 0; nt < NT; ++nt)
        oacc[nt][rr] = __builtin_amdgcn_mfma_f32_16x16x16f16(vop, pop[nt], oacc[nt][rr], 0, 0, 0);
    }
  };

  // ---- main loop: chunks of up to 64 wave-steps, two-deep register pipeline ----
  constexpr int kStepTok = 16 * NW;  // tokens between a wave's consecutive steps
  for (int c0 = 0; c0 < my_steps; c0 += 64) {
    const int cn = (my_steps - c0) < 64 ? (my_steps - c0) : 64;
    if (c0 > 0) load_ids(c0);
    StepRegs<ELEM> ra, rb;
    issue(ra, 0, start + 16 * (w + NW * c0));
    for (int i = 0; i < cn; i += 2) {
      const int tb_a = start + 16 * (w + NW * (c0 + i));
      if (i + 1 < cn) issue(rb, i + 1, tb_a + kStepTok);
      compute(ra, tb_a);
      if (i + 1 >= cn) break;
      if (i + 2 < cn) issue(ra, i + 2, tb_a + 2 * kStepTok);
      compute(rb, tb_a + kStepTok);
    }
  }
  if (bad && lane == 0) atomicOr(g.status, bad);

  // ---- merge the four waves ---------------------------------------------------
  __shared__ float sm_m[NW][NCOL];
  __shared__ float sm_l[NW][NCOL];
  __shared__ float sm_o[NW - 1][NCOL][kSmoStride];
  float l_head[NT];
#pragma unroll
  for (int nt = 0; nt < NT; ++nt) {
    float l = l_part[nt];
    l += __shfl_xor(l, 16);
    l += __shfl_xor(l, 32);
    l_head[nt] = l;
    if (gq == 0) {
      sm_m[w][nt * 16 + n] = m_run[nt];
      sm_l[w][nt * 16 + n] = l;
    }
  }
  __syncthreads();
  float big_m[NT], big_l[NT], f[NT];
#pragma unroll
  for (int nt = 0; nt < NT; ++nt) {
    const int col = nt * 16 + n;
    float M = sm_m[0][col];
#pragma unroll
    for (int ww = 1; ww < NW; ++ww) M = fmaxf(M, sm_m[ww][col]);
    float L = 0.0f;
#pragma unroll
    for (int ww = 0; ww < NW; ++ww) {
      const float mw = sm_m[ww][col];
      L += (mw == -__builtin_inff()) ? 0.0f : sm_l[ww][col] * exp2f(mw - M);
    }
    big_m[nt] = M;
    big_l[nt] = L;
    f[nt] = (m_run[nt] == -__builtin_inff()) ? 0.0f : exp2f(m_run[nt] - M);
    (void)l_head[nt];
    if (w > 0 && col < group) {
#pragma unroll
      for (int rr = 0; rr < 8; ++rr) {
        *reinterpret_cast<f32x4*>(&sm_o[w - 1][col][rr * 16 + 4 * gq]) = oacc[nt][rr] * f[nt];
      }
    }
  }
  __syncthreads();
  if (w != 0) return;
#pragma unroll
  for (int nt = 0; nt < NT; ++nt) {
    const int col = nt * 16 + n;
    if (col >= group) continue;
    const int head = kvh * group + col;
    const float inv_l = out_mul / big_l[nt];
    const int64_t row = static_cast<int64_t>(seq) * p.num_q_heads + head;
#pragma unroll
    for (int rr = 0; rr < 8; ++rr) {
      const int dim = rr * 16 + 4 * gq;
      f32x4 acc = oacc[nt][rr] * f[nt];
#pragma unroll
      for (int ww = 0; ww < NW - 1; ++ww) acc += *reinterpret_cast<const f32x4*>(&sm_o[ww][col][dim]);
      acc *= inv_l;
      if constexpr (PARTIAL) {
        float* po = p.part_o + (row * p.num_partitions + part) * kD + dim;
        *reinterpret_cast<f32x4*>(po) = acc;
      } else {
        _Float16* po = static_cast<_Float16*>(p.out) + row * kD + dim;
        *reinterpret_cast<f16x4*>(po) =
            f16x4{(_Float16)acc[0], (_Float16)acc[1], (_Float16)acc[2], (_Float16)acc[3]};
      }
    }
    if constexpr (PARTIAL) {
      if (gq == 0) {
        p.part_m[row * p.num_partitions + part] = big_m[nt];
        p.part_l[row * p.num_partitions + part] = big_l[nt];
      }
    }
  }
}

// Log-sum-exp merge of the chunk partials of one (sequence, query head):
// out = sum_c w_c o_c / sum_c w_c with w_c = l_c * 2^(m_c - max_c m_c).
template <int BS>
__global__ __launch_bounds__(128) void lse_reduce_kernel(PoolGeom g, DecodeLaunch p) {
  const int row = blockIdx.x;  // seq * Hq + head
  const int seq = row / p.num_q_heads;
  const int dim = threadIdx.x;
  int T = p.lens[seq];
  const int t_cap = p.max_blocks * BS;
  T = T < 0 ? 0 : (T > t_cap ? t_cap : T);
  const int cv = (T + p.partition_tokens - 1) / p.partition_tokens;
  const float* m = p.part_m + static_cast<int64_t>(row) * p.num_partitions;
  const float* l = p.part_l + static_cast<int64_t>(row) * p.num_partitions;
  const float* o = p.part_o + static_cast<int64_t>(row) * p.num_partitions * kD + dim;
  float M = -__builtin_inff();
  for (int c = 0; c < cv; ++c) M = fmaxf(M, m[c]);
  float num = 0.0f, den = 0.0f;
  for (int c = 0; c < cv; ++c) {
    const float wgt = l[c] * exp2f(m[c] - M);
    den += wgt;
    num += wgt * o[static_cast<int64_t>(c) * kD];
  }
  _Float16* out = static_cast<_Float16*>(p.out) + static_cast<int64_t>(row) * kD + dim;
  *out = (_Float16)(cv > 0 ? num / den : 0.0f);
  (void)g;
}

// Kernels are launched with hipExtLaunchKernelGGL: its start/stop events (null
// when not timing) are stamped by the dispatch itself, so timing a launch adds
// no barrier packets to the stream.
template <int ELEM, int BS>
hipError_t launch_decode_bs(const PoolGeom& g, const DecodeLaunch& d, bool partial, int nt,
                            dim3 grid, hipStream_t s, hipEvent_t t0, hipEvent_t t1) {
  constexpr int NW = kDecodeWaves;
  const dim3 block(NW * 64);
  if (nt == 1) {
    if (partial) hipExtLaunchKernelGGL((decode_kernel<ELEM, BS, 1, true, NW>), grid, block, 0, s, t0, t1, 0, g, d);
    else hipExtLaunchKernelGGL((decode_kernel<ELEM, BS, 1, false, NW>), grid, block, 0, s, t0, t1, 0, g, d);
  } else {
    if (partial) hipExtLaunchKernelGGL((decode_kernel<ELEM, BS, 2, true, NW>), grid, block, 0, s, t0, t1, 0, g, d);
    else hipExtLaunchKernelGGL((decode_kernel<ELEM, BS, 2, false, NW>), grid, block, 0, s, t0, t1, 0, g, d);
  }
  return hipGetLastError();
}

template <int ELEM>
hipError_t launch_decode_elem(const PoolGeom& g, const DecodeLaunch& d, bool partial, int nt,
                              dim3 grid, hipStream_t s, hipEvent_t t0, hipEvent_t t1) {
  switch (g.block_size) {
    case 8: return launch_decode_bs<ELEM, 8>(g, d, partial, nt, grid, s, t0, t1);
    case 16: return launch_decode_bs<ELEM, 16>(g, d, partial, nt, grid, s, t0, t1);
    case 32: return launch_decode_bs<ELEM, 32>(g, d, partial, nt, grid, s, t0, t1);
    default: return hipErrorInvalidValue;
  }
}

}  // namespace

hipError_t launch_decode(const PoolGeom& g, const DecodeLaunch& d, bool partial, hipStream_t s,
                         hipEvent_t t0, hipEvent_t t1) {
  const int group = d.num_q_heads / g.kv_heads;
  const int nt = group > 16 ? 2 : 1;
  const int64_t wgs = static_cast<int64_t>(d.num_partitions) * g.kv_heads * d.num_seqs;
  if (wgs <= 0) return hipSuccess;
  const dim3 grid(static_cast<unsigned>(wgs));
  if (g.elem_bytes == 2) return launch_decode_elem<2>(g, d, partial, nt, grid, s, t0, t1);
  return launch_decode_elem<1>(g, d, partial, nt, grid, s, t0, t1);
}

hipError_t launch_lse_reduce(const PoolGeom& g, const DecodeLaunch& d, hipStream_t s,
                             hipEvent_t t0, hipEvent_t t1) {
  const int64_t rows = static_cast<int64_t>(d.num_seqs) * d.num_q_heads;
  if (rows <= 0) return hipSuccess;
  const dim3 grid(static_cast<unsigned>(rows));
  switch (g.block_size) {
    case 8: hipExtLaunchKernelGGL(lse_reduce_kernel<8>, grid, dim3(kD), 0, s, t0, t1, 0, g, d); break;
    case 16: hipExtLaunchKernelGGL(lse_reduce_kernel<16>, grid, dim3(kD), 0, s, t0, t1, 0, g, d); break;
    case 32: hipExtLaunchKernelGGL(lse_reduce_kernel<32>, grid, dim3(kD), 0, s, t0, t1, 0, g, d); break;
    default: return hipErrorInvalidValue;
  }
  return hipGetLastError();
}

}  // namespace pa
