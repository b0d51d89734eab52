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
// Mapping to CDNA4.  A wave works on 16-token steps of one (sequence, KV
// head):
//  * each step loads the K and V tiles of 16 tokens with 16-byte lane loads
//    (one contiguous 1 KiB run per load instruction) directly in the register
//    layout of the MFMA operands -- no LDS round trip.  Where every tile is
//    read once per launch the loads are nontemporal (on MI355X they sustain
//    about 11% more bandwidth over randomly placed 4 KiB tiles than ordinary
//    ones); where many sequences share blocks (beams, common prompts) they are
//    ordinary loads, so that the sharers' reads of a tile hit in L2 (CACHED);
//  * S^T[token][head] = K * Q^T with v_mfma_f32_16x16x32_f16 (rows = 16 tokens,
//    columns = the G query heads of the KV head, padded to 16), so the K tile
//    is read once for all G heads of the group;
//  * online softmax in fp32 (base-2 exponent), with the per-head maximum
//    exchanged across the four 16-lane rows by two VALU row swaps;
//  * O^T[dim][head] += V^T * P^T with v_mfma_f32_16x16x16_f16, P in fp16;
//  * block ids are wave-uniform and read with scalar loads one pipeline block
//    ahead; K/V loads run a two-step register pipeline with no data-dependent
//    branch around any vector load.
// decode_kernel runs this per-wave engine in one of three schedules:
//  * single pass: one workgroup of four waves per (sequence, KV head); the
//    waves take interleaved steps and merge (max, sum, O) through LDS;
//  * split, four waves per chunk: a workgroup streams a run of P-token chunks
//    of one (sequence, KV head), the waves interleaving within each chunk and
//    merging at its end into that chunk's partials (max, sum, normalised O);
//  * split, one wave per run: each wave streams its own run of chunks and
//    writes each chunk's partials without any merge;
// lse_reduce_kernel merges the partials.
// fp8 (E4M3FN) tiles are widened to fp16 in registers with the hardware
// packed converter (exact: every E4M3 value is an fp16 value); int8 tiles
// become the fp16 integers c - z (exact, |c - z| <= 255) with a byte
// shuffle and a packed fp16 subtraction.  The per-(layer, KV head) scales are
// folded into the score and output multipliers.
#pragma once

#include <hip/hip_ext.h>
#include <hip/hip_runtime.h>

#include <cstdint>
#include <type_traits>

#include "kernels.hpp"
#include "token_store.hpp"

namespace pa {
// Kernel templates of the decode and multi-token paths, instantiated per
// (element kind, head_dim) in decode_inst.hip and launched from
// decode_kernels.hip.
namespace dk {

typedef _Float16 f16x8 __attribute__((ext_vector_type(8)));
typedef _Float16 f16x4 __attribute__((ext_vector_type(4)));
typedef _Float16 f16x2 __attribute__((ext_vector_type(2)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));

// Read-only view of a block-table row: loads with wave-uniform indices become
// scalar loads (the table is not written while a kernel runs).
typedef const int32_t __attribute__((address_space(4))) ConstI32;

constexpr float kLog2e = 1.4426950408889634f;
constexpr int kWaves = 4;  // waves per decode workgroup

// Steps of K/V loads each wave keeps in flight beyond the one it computes on.
// One step is 16 tokens of one KV head (8 KiB fp16, 4 KiB fp8 at head_dim
// 128; half that at 64).  Measured on
// MI355X over depths 1-6: 2 is best or within noise of the best for fp16 and
// fp8, GQA and MQA; deeper pipelines only cost registers and occupancy.
constexpr int kDepth = 2;

// How far (base 2) a score may exceed the softmax reference before the
// accumulators are rescaled, where rescaling is lazy (two or more column
// tiles): probabilities then stay below 2^8, exact as fp16 operands.  Lazy
// rescaling saves the wide rescale on most steps of MQA-sized groups; with
// one column tile the eager form schedules better (measured on MI355X).
constexpr float kRescaleSlack = 8.0f;

// 2^x with the bare v_exp_f32: results below 2^-126 flush to zero instead of
// going through exp2f's denormal rescaling (four more VALU instructions per
// call).  Used for probabilities and rescale factors, which are at most 2^8
// and where a value below 2^-126 is zero after the fp16 conversion anyway.
__device__ inline float fast_exp2(float x) { return __builtin_amdgcn_exp2f(x); }

// Four E4M3FN codes (bytes 0..3 of w) -> four fp16 in byte order, with the
// gfx950 packed converter at scale 1: every E4M3FN value is an fp16 value, so
// the conversion is exact (checked for all byte pairs on MI355X).
__device__ inline f16x4 e4m3x4_to_f16x4(uint32_t w) {
  const f16x2 lo = __builtin_amdgcn_cvt_scalef32_pk_f16_fp8(w, 1.0f, false);
  const f16x2 hi = __builtin_amdgcn_cvt_scalef32_pk_f16_fp8(w, 1.0f, true);
  return f16x4{lo[0], lo[1], hi[0], hi[1]};
}

// Four stored int8 bytes (c + 128 each, bytes 0..3 of w) -> four fp16 c - z
// in byte order.  Each byte becomes the low byte of the fp16 bit pattern
// 0x64XX, i.e. the value 1024 + c + 128 exactly; subtracting bias = 1152 + z
// (an integer in [1024, 1279]) leaves c - z exactly.
__device__ inline f16x4 i8x4_to_f16x4(uint32_t w, f16x2 bias) {
  const uint32_t lo = (w & 0xFFu) | ((w & 0xFF00u) << 8) | 0x64006400u;
  const uint32_t hi = ((w >> 16) & 0xFFu) | ((w >> 8) & 0xFF0000u) | 0x64006400u;
  const f16x2 a = __builtin_bit_cast(f16x2, lo) - bias;
  const f16x2 b = __builtin_bit_cast(f16x2, hi) - bias;
  return f16x4{a[0], a[1], b[0], b[1]};
}

// Maximum / sum of x over the four 16-lane rows of the wave (lanes n, n+16,
// n+32, n+48 end up with the same value), with two VALU row swaps:
// permlane16_swap pairs rows 0-1 and 2-3, permlane32_swap the two halves.
__device__ inline float max_across_rows(float x) {
  const auto a = __builtin_amdgcn_permlane16_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  const float y = fmaxf(__uint_as_float(a[0]), __uint_as_float(a[1]));
  const auto b = __builtin_amdgcn_permlane32_swap(__float_as_uint(y), __float_as_uint(y), false, false);
  return fmaxf(__uint_as_float(b[0]), __uint_as_float(b[1]));
}
__device__ inline float sum_across_rows(float x) {
  const auto a = __builtin_amdgcn_permlane16_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  const float y = __uint_as_float(a[0]) + __uint_as_float(a[1]);
  const auto b = __builtin_amdgcn_permlane32_swap(__float_as_uint(y), __float_as_uint(y), false, false);
  return __uint_as_float(b[0]) + __uint_as_float(b[1]);
}

// K and V registers of one 16-token step: a tile of 16 tokens x D dims x
// ELEM bytes is D * ELEM / 64 16-byte loads per lane.
template <int ELEM, int D>
struct StepRegs {
  static constexpr int kLoads = D * ELEM / 64;  // 16-byte loads per lane for K (and for V)
  u32x4 k[kLoads];
  u32x4 v[kLoads];
};

// Device-memory (global address space) bytes.
using GlobalBytes = const __attribute__((address_space(1))) uint8_t*;

// A wave-uniform device-memory pointer, moved to scalar registers.
__device__ inline GlobalBytes uniform_ptr(const uint8_t* p) {
  const uint64_t v = reinterpret_cast<uint64_t>(p);
  const uint32_t lo = __builtin_amdgcn_readfirstlane(static_cast<uint32_t>(v));
  const uint32_t hi = __builtin_amdgcn_readfirstlane(static_cast<uint32_t>(v >> 32));
  return reinterpret_cast<GlobalBytes>((static_cast<uint64_t>(hi) << 32) | lo);
}

// The per-wave engine: operands, softmax state and the load / compute of one
// 16-token step of one (sequence, KV head).  Lane (gq, n): gq = lane / 16 is
// its row group, n = lane % 16 its head column.  FUSE: the launch also
// stores each unit's new token (the fused scatter).  MULTI: the columns are
// (query token, head) pairs of several new tokens of one sequence, each with
// its own causal limit (multi-token attention).
template <int D, int KIND, int BS, int NT, bool FUSE, bool MULTI = false, bool CACHED = false>
struct WaveDecoder {
  static constexpr int ELEM = kind_bytes(KIND);
  static constexpr int kElem = ELEM;
  static constexpr bool kFuse = FUSE;
  static constexpr int kNT = NT;
  static constexpr int kD = D;        // head_dim
  static constexpr int NDT = D / 16;  // 16-dim tiles of O: P.V MFMAs per column tile
  static constexpr int NKU = D / 32;  // 32-dim slices of the dot product: Q.K MFMAs per column tile
  static constexpr int X = 16 / ELEM;  // elements per 16-byte chunk
  using Regs = StepRegs<ELEM, D>;
  static constexpr int NLD = Regs::kLoads;

  int gq, n, T, max_blocks, num_blocks;
  // MULTI: keys visible to this lane's column of each tile (its position + 1)
  // and the smallest limit of the wave's columns; the query rows of the
  // columns start at mt_row0 (column c: token c / group, head c % group), or
  // are mt_rowmap[c / group] when that is set (columns of several
  // sequences), and columns at or past mt_ncols are padding.
  int lim[NT], lim_min, mt_row0, mt_ncols;
  const int32_t* mt_rowmap;
  uint64_t block_stride;
  const ConstI32* trow;
  const uint8_t* kbase;
  const uint8_t* vbase;
  uint32_t koff[NLD], voff[NLD];
  float qk_mul, out_mul;
  // Fused scatter: this unit's new token (K and V of token T - 1, fp16), or
  // null; owns_new marks the wave whose step holds that token.
  const _Float16* knew;
  const _Float16* vnew;
  float new_kinv, new_vinv;  // fp8 / int8: inverse scales of this (layer, KV head)
  float new_kz, new_vz;      // int8: its zero points
  f16x2 kbias, vbias;        // int8: 1152 + zero point, twice (see i8x4_to_f16x4)
  int new_slot, new_blk;     // slot given for the new token; table entry of token T - 1
  bool owns_new;
  int new_tr;
  u32x4 newk[NLD][1];         // fp16: the new token's K chunks
  _Float16 newv[NLD][X / 4];  // fp16: its V elements
  uint32_t new_kh, new_vh;    // fp8: its K and V dims 2*lane, 2*lane+1 (fp16)
  uint8_t* lds_new;           // fp8 / int8: this wave's 256-byte LDS scratch for its codes
  f16x8 qop[NT][NKU];
  f32x4 oacc[NT][NDT];
  // Online-softmax state per head column: accumulators relative to the
  // reference m_run (base 2).  With kLazy the reference may trail the true
  // running maximum m_true by less than kRescaleSlack and fresh marks a state
  // with nothing accumulated; otherwise m_run is the running maximum itself.
  static constexpr bool kLazy = NT > 1;
  float m_run[NT], m_true[NT], l_part[NT];
  // MULTI: the softmax denominators accumulate on the matrix cores (one
  // 16x16x32 MFMA of an all-ones operand with P per pair and column tile),
  // so every lane holds its column's whole sum; finish_l turns them into
  // l_part for the merges.
  f32x4 lacc[NT];
  bool fresh;
  uint32_t bad;

  // Largest score seen since the last reset.
  __device__ float top(int nt) const {
    if constexpr (kLazy) return m_true[nt];
    return m_run[nt];
  }

  // Geometry and the block-table row; needs no context length.
  __device__ void bind(const PoolGeom& g, const DecodeLaunch& p, int seq, int kvh, int lane) {
    gq = lane >> 4;
    n = lane & 15;
    T = 0;
    max_blocks = p.max_blocks;
    num_blocks = g.num_blocks;
    block_stride = g.block_stride;
    trow = (const ConstI32*)(p.tables + static_cast<int64_t>(seq) * p.max_blocks);
    kbase = g.k_layer(p.layer) + static_cast<uint64_t>(kvh) * g.tile_bytes;
    vbase = g.v_layer(p.layer) + static_cast<uint64_t>(kvh) * g.tile_bytes;
    bad = 0;
    mt_rowmap = nullptr;
    knew = vnew = nullptr;
    new_kinv = new_vinv = 1.0f;
    new_kz = new_vz = 0.0f;
    new_slot = -1;
    new_blk = 0;
    owns_new = false;
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
  }

  // Q^T operands (lane (gq, n) holds head column n, 8 dims per MFMA) and the
  // score / output multipliers.
  __device__ void load_q(const PoolGeom& g, const DecodeLaunch& p, int seq, int kvh, int group) {
    qk_mul = p.scale * kLog2e;
    out_mul = 1.0f;
    if constexpr (ELEM == 1) {
      const int lhs = g.layers * g.kv_heads;
      const int lh = p.layer * g.kv_heads + kvh;
      qk_mul *= g.scales[lh];
      out_mul = g.scales[lhs + lh];
      if constexpr (KIND == kI8) {
        const _Float16 kb = static_cast<_Float16>(1152.0f + g.scales[4 * lhs + lh]);
        const _Float16 vb = static_cast<_Float16>(1152.0f + g.scales[5 * lhs + lh]);
        kbias = f16x2{kb, kb};
        vbias = f16x2{vb, vb};
      }
    }
    const _Float16* qs = static_cast<const _Float16*>(p.q) + static_cast<int64_t>(seq) * p.num_q_heads * kD;
#pragma unroll
    for (int nt = 0; nt < NT; ++nt) {
      const int col = nt * 16 + n;
      bool valid = col < group;
      const _Float16* qh = qs + static_cast<int64_t>(kvh * group + (valid ? col : 0)) * kD;
      if constexpr (MULTI) {
        valid = col < mt_ncols;
        const int c = valid ? col : 0;
        const int64_t row = mt_rowmap ? mt_rowmap[c / group] : static_cast<int64_t>(mt_row0) + c / group;
        qh = static_cast<const _Float16*>(p.q) + (row * p.num_q_heads + kvh * group + c % group) * kD;
      }
#pragma unroll
      for (int u = 0; u < NKU; ++u) {
        const int dim0 = (ELEM == 2) ? (u * 4 + gq) * 8 : ((u >> 1) * 4 + gq) * 16 + (u & 1) * 8;
        const f16x8 v = *reinterpret_cast<const f16x8*>(qh + dim0);
        qop[nt][u] = valid ? v : f16x8{0, 0, 0, 0, 0, 0, 0, 0};
      }
    }
    // The softmax needs qk_mul > 0, so that the largest raw score times
    // qk_mul is the largest logit: a negative scale's sign moves into q
    // (exact in fp16), and a zero scale (decode only; multi-token attention
    // refuses it) becomes 2^-100, which leaves every logit at most 2^-60 from
    // 0, i.e. every exponential exactly 1 in fp32, and keeps masked scores at
    // -inf.
    if (qk_mul < 0.0f) {
      qk_mul = -qk_mul;
#pragma unroll
      for (int nt = 0; nt < NT; ++nt)
#pragma unroll
        for (int u = 0; u < NKU; ++u) qop[nt][u] = -qop[nt][u];
    }
    qk_mul = fmaxf(qk_mul, 0x1p-100f);
  }

  // Fused scatter (owner wave only).  Before the stream, the lanes that will
  // hold token T - 1 in its step load their part of the new token: K: lanes
  // n == tr, chunks j*4+gq (X dims each); V: lanes gq == tr/4, dims
  // (j*X/4 + q)*16 + n, q < X/4; tr = (T - 1) mod 16 (fp8 pools: every lane
  // loads two dims, and the wave encodes them together).  Nothing waits
  // for these loads until that step, where the loaded K chunks and V
  // elements of the token are replaced by the new token in the pool's form
  // (fp16 bits or E4M3FN codes), so the step never reads the slot that this
  // very launch stores into.
  static constexpr int kRR = X / 4;
  __device__ void load_new() {
    new_tr = (T - 1) & 15;
    if constexpr (ELEM == 1) {
      // fp8 / int8: two dims per lane (the first D / 2 lanes), encoded by
      // those lanes together in the token's step.
      if (2 * lane_id() < D) {
        new_kh = *reinterpret_cast<const uint32_t*>(knew + 2 * lane_id());
        new_vh = *reinterpret_cast<const uint32_t*>(vnew + 2 * lane_id());
      }
      return;
    }
    if (n == new_tr) {
#pragma unroll
      for (int j = 0; j < NLD; ++j) {
        const int c = j * 4 + gq;
        newk[j][0] = *reinterpret_cast<const u32x4*>(knew + c * X);
      }
    }
    if (gq == (new_tr >> 2)) {
#pragma unroll
      for (int j = 0; j < NLD; ++j) {
#pragma unroll
        for (int q = 0; q < kRR; ++q) newv[j][q] = vnew[(j * kRR + q) * 16 + n];
      }
    }
  }

  // Whether the given slot is token T - 1's (a negative one is not).
  __device__ bool new_slot_ok() const {
    return new_slot >= 0 && static_cast<uint32_t>(new_blk) < static_cast<uint32_t>(num_blocks) &&
           new_slot == new_blk * BS + (T - 1) % BS;
  }

  __device__ int lane_id() const { return gq * 16 + n; }

  // fp8 / int8: the wave encodes the new token (two dims of K and of V per
  // lane, lane-parallel) into its LDS scratch: K codes at bytes 0..D-1, V
  // codes at D..2D-1, both in dim order; inject_k / inject_v read them back
  // in the tile layout.  DS operations of one wave run in order.
  __device__ void encode_new_to_lds() {
    const int d0 = 2 * lane_id();
    if (d0 >= D) return;
    const uint32_t k0 = encode_byte<KIND>(half_bits_to_float(new_kh) * new_kinv, new_kz);
    const uint32_t k1 = encode_byte<KIND>(half_bits_to_float(new_kh >> 16) * new_kinv, new_kz);
    const uint32_t v0 = encode_byte<KIND>(half_bits_to_float(new_vh) * new_vinv, new_vz);
    const uint32_t v1 = encode_byte<KIND>(half_bits_to_float(new_vh >> 16) * new_vinv, new_vz);
    *reinterpret_cast<uint16_t*>(lds_new + d0) = static_cast<uint16_t>(k0 | (k1 << 8));
    *reinterpret_cast<uint16_t*>(lds_new + kD + d0) = static_cast<uint16_t>(v0 | (v1 << 8));
  }

  // K chunks of the new token, in the pool's form, for lanes n == tr.
  __device__ void inject_k(Regs& r) {
    if constexpr (ELEM == 1) encode_new_to_lds();
    if (n != new_tr) return;
#pragma unroll
    for (int j = 0; j < NLD; ++j) {
      if constexpr (ELEM == 2) {
        r.k[j] = newk[j][0];
      } else {
        r.k[j] = *reinterpret_cast<const u32x4*>(lds_new + (j * 4 + gq) * X);
      }
    }
  }

  // V elements of the new token, in the pool's form, for lanes gq == tr/4.
  __device__ void inject_v(Regs& r) {
    if (gq != (new_tr >> 2)) return;
    const int tt = new_tr & 3;
#pragma unroll
    for (int j = 0; j < NLD; ++j) {
#pragma unroll
      for (int q = 0; q < kRR; ++q) {
        uint32_t val;
        if constexpr (ELEM == 2) val = __builtin_bit_cast(uint16_t, newv[j][q]);
        else val = lds_new[kD + (j * kRR + q) * 16 + n];
        const int e = q * 4 + tt;  // element of the 16-byte chunk
        constexpr int kBits = 8 * ELEM;
        constexpr uint32_t kMask = (1u << kBits) - 1u;
        const int dw = (e * kBits) >> 5, sh = (e * kBits) & 31;
#pragma unroll
        for (int d = 0; d < 4; ++d) {
          if (d == dw) r.v[j][d] = (r.v[j][d] & ~(kMask << sh)) | (val << sh);
        }
      }
    }
  }

  // The new token's tiles, as loaded and injected, go back to where they were
  // loaded from: the lanes holding its K chunks store them (16 bytes each),
  // the lanes holding its V elements store their whole 16-byte chunks (the
  // three other tokens of a chunk are rewritten unchanged: the block of
  // token T - 1 belongs to this sequence alone).
  __device__ uint64_t new_sub_offset(bool v) const {
    if constexpr (BS == 32) {
      const int sub = ((T - 1) >> 4) & 1;
      return static_cast<uint64_t>(sub) * (v ? 4 * 16 * X * ELEM : 16 * kD * ELEM);
    }
    return 0;
  }
  __device__ void store_new_k(const Regs& r) const {
    if (n != new_tr) return;
    uint8_t* kp = const_cast<uint8_t*>(kbase) + static_cast<uint64_t>(new_blk) * block_stride + new_sub_offset(false);
#pragma unroll
    for (int j = 0; j < NLD; ++j) *reinterpret_cast<u32x4*>(kp + koff[j]) = r.k[j];
  }
  __device__ void store_new_v(const Regs& r) const {
    if (gq != (new_tr >> 2)) return;
    uint8_t* vp = const_cast<uint8_t*>(vbase) + static_cast<uint64_t>(new_blk) * block_stride + new_sub_offset(true);
#pragma unroll
    for (int j = 0; j < NLD; ++j) *reinterpret_cast<u32x4*>(vp + voff[j]) = r.v[j];
  }

  // S^T = K Q^T for the 16 tokens of a K tile held as loaded (fp16 bits or
  // E4M3FN codes), unscaled.
  __device__ void raw_scores(const u32x4 (&kr)[NLD], f32x4 (&s)[NT]) const {
#pragma unroll
    for (int nt = 0; nt < NT; ++nt) s[nt] = f32x4{0, 0, 0, 0};
#pragma unroll
    for (int u = 0; u < NKU; ++u) {
      f16x8 kop;
      if constexpr (ELEM == 2) {
        kop = __builtin_bit_cast(f16x8, kr[u]);
      } else {
        const u32x4 raw = kr[u >> 1];
        f16x4 a, b;
        if constexpr (KIND == kI8) {
          a = i8x4_to_f16x4((u & 1) ? raw[2] : raw[0], kbias);
          b = i8x4_to_f16x4((u & 1) ? raw[3] : raw[1], kbias);
        } else {
          a = e4m3x4_to_f16x4((u & 1) ? raw[2] : raw[0]);
          b = e4m3x4_to_f16x4((u & 1) ? raw[3] : raw[1]);
        }
        kop = f16x8{a[0], a[1], a[2], a[3], b[0], b[1], b[2], b[3]};
      }
#pragma unroll
      for (int nt = 0; nt < NT; ++nt)
        s[nt] = __builtin_amdgcn_mfma_f32_16x16x32_f16(kop, qop[nt][u], s[nt], 0, 0, 0);
    }
  }

  __device__ void reset() {
    fresh = true;
#pragma unroll
    for (int nt = 0; nt < NT; ++nt) {
      m_run[nt] = -__builtin_inff();
      m_true[nt] = -__builtin_inff();
      l_part[nt] = 0.0f;
      lacc[nt] = f32x4{0, 0, 0, 0};
#pragma unroll
      for (int r = 0; r < NDT; ++r) oacc[nt][r] = f32x4{0, 0, 0, 0};
    }
  }

  // Block ids of the step starting at token tb (scalar loads; the table index
  // is clamped to the table width, so any tb is safe to ask for).  Token
  // positions are non-negative and below 2^31: 32-bit arithmetic keeps the
  // index math and the clamp on the scalar unit.
  __device__ void fetch_ids(int tb, int& lo, int& hi) const {
    const int b = static_cast<int>(static_cast<uint32_t>(tb) / BS);
    const int last = max_blocks - 1;
    lo = trow[b < last ? b : last];
    hi = 0;
    if constexpr (BS == 8) hi = trow[b + 1 < last ? b + 1 : last];
  }

  __device__ int phys_ok(int b) {
    if (static_cast<uint32_t>(b) >= static_cast<uint32_t>(num_blocks)) {
      bad |= kDevBadBlock;
      return 0;
    }
    return b;
  }

  // Nontemporal where every tile is read once (decode; multi-token items of
  // at most one wave's tokens, e.g. decode tokens); ordinary loads (CACHED)
  // for the wide multi-token items, whose waves re-read each other's key
  // tiles, and for decode over blocks that many sequences share: a block's sharers
  // run close together on one XCD (same KV head, nearby sequences), and with
  // nontemporal loads its lines leave L2 before the other sharers read them
  // (measured on MI355X, 160 beams sharing prefixes: 2.34x the unique bytes
  // fetched with nontemporal loads, 1.12x with ordinary ones).
  static __device__ u32x4 ld16(const uint8_t* a) {
    if constexpr (CACHED) return *reinterpret_cast<const u32x4*>(a);
    return __builtin_nontemporal_load(reinterpret_cast<const u32x4*>(a));
  }
  static __device__ u32x4 ld16(GlobalBytes a) {
    using GlobalChunk = const __attribute__((address_space(1))) u32x4*;
    if constexpr (CACHED) return *reinterpret_cast<GlobalChunk>(a);
    return __builtin_nontemporal_load(reinterpret_cast<GlobalChunk>(a));
  }

  // Loads of the step starting at token tb, whose blocks are id_lo (and
  // id_hi, the block of its second 8 tokens when blocks hold 8).
  // DO_K / DO_V: load only the K or only the V tile (multi-token pairs).
  template <bool DO_K = true, bool DO_V = true>
  __device__ void issue(Regs& r, int tb, int id_lo, int id_hi) {
    if constexpr (BS == 8) {
      const int b0 = phys_ok(id_lo);
      // The second block of the step exists only if its first token does.
      const int b1 = (tb + 8 < T) ? phys_ok(id_hi) : b0;
      const uint8_t* kp = kbase + static_cast<uint64_t>(n < 8 ? b0 : b1) * block_stride;
      const uint8_t* vp = vbase + static_cast<uint64_t>(gq < 2 ? b0 : b1) * block_stride;
#pragma unroll
      for (int j = 0; j < NLD; ++j) {
        if constexpr (DO_K) r.k[j] = ld16(kp + koff[j]);
        if constexpr (DO_V) r.v[j] = ld16(vp + voff[j]);
      }
    } else {
      (void)id_hi;
      const int b = phys_ok(id_lo);
      uint64_t koff_sub = 0, voff_sub = 0;
      if constexpr (BS == 32) {
        const int sub = (tb >> 4) & 1;
        koff_sub = static_cast<uint64_t>(sub) * 16 * kD * ELEM;
        voff_sub = static_cast<uint64_t>(sub) * 4 * 16 * X * ELEM;
      }
      // The tiles' base addresses are wave-uniform: held in scalar registers,
      // each load takes the lane's 32-bit offset (no 64-bit vector address math).
      const GlobalBytes kp = uniform_ptr(kbase + static_cast<uint64_t>(b) * block_stride + koff_sub);
      const GlobalBytes vp = uniform_ptr(vbase + static_cast<uint64_t>(b) * block_stride + voff_sub);
#pragma unroll
      for (int j = 0; j < NLD; ++j) {
        if constexpr (DO_K) r.k[j] = ld16(kp + koff[j]);
        if constexpr (DO_V) r.v[j] = ld16(vp + voff[j]);
      }
    }
  }

  // ---- MULTI: two steps at a time ------------------------------------------
  // The P.V product of two 16-token steps runs as one v_mfma_f32_16x16x32_f16
  // per (dim tile, column tile), twice the rate of two 16x16x16 products on
  // gfx950: the K index of lane group gq is tokens 4gq..4gq+3 of the first
  // step, then of the second, the same order for V^T and P^T.

  // Raw scores of one step (the scale is applied with the exponent), masked
  // by each column's causal limit (all masked when the step is padding);
  // only the steps at the limits take the masking branch.
  __device__ void pair_scores(const u32x4 (&kr)[NLD], int tb, bool is_real, f32x4 (&s)[NT]) const {
    raw_scores(kr, s);
    if (!is_real || tb + 16 > lim_min) {
#pragma unroll
      for (int nt = 0; nt < NT; ++nt) {
        const int vh = is_real ? lim[nt] - (tb + 4 * gq) : 0;
#pragma unroll
        for (int e = 0; e < 4; ++e)
          if (e >= vh) s[nt][e] = -__builtin_inff();
      }
    }
  }

  // Zeroes the V elements of tokens at or past the keys in use (NaN-safe);
  // a padding step is zeroed whole.
  __device__ void pair_mask_v(u32x4 (&v)[NLD], int tb, bool is_real) const {
    if (__builtin_expect(is_real && tb + 16 <= T, 1)) return;
    const int vh = is_real ? T - (tb + 4 * gq) : 0;
    const int vc = vh < 0 ? 0 : (vh > 4 ? 4 : vh);
#pragma unroll
    for (int j = 0; j < NLD; ++j) {
      if constexpr (ELEM == 2) {
        const uint32_t m01 = (vc > 0 ? 0x0000FFFFu : 0u) | (vc > 1 ? 0xFFFF0000u : 0u);
        const uint32_t m23 = (vc > 2 ? 0x0000FFFFu : 0u) | (vc > 3 ? 0xFFFF0000u : 0u);
        v[j] &= u32x4{m01, m23, m01, m23};
      } else {
        const uint32_t mb = vc >= 4 ? 0xFFFFFFFFu : ((1u << (8 * vc)) - 1u);
        v[j] &= u32x4{mb, mb, mb, mb};
      }
    }
  }

  // Online softmax over the 32 tokens of a pair (lazy rescaling), and the
  // probabilities as the P^T operands.  Scores arrive unscaled: qk_mul > 0
  // (load_q folds a negative scale's sign into q), so the largest raw score
  // times qk_mul is the largest logit, and each probability is one
  // exp2(fma(s, qk_mul, -reference)).
  __device__ void pair_softmax(f32x4 (&sa)[NT], f32x4 (&sb)[NT], f16x8 (&pop)[NT]) {
    static_assert(kLazy, "pairs use the lazy reference");
    bool need = false;
#pragma unroll
    for (int nt = 0; nt < NT; ++nt) {
      const float ma = fmaxf(fmaxf(sa[nt][0], sa[nt][1]), fmaxf(sa[nt][2], sa[nt][3]));
      const float mb = fmaxf(fmaxf(sb[nt][0], sb[nt][1]), fmaxf(sb[nt][2], sb[nt][3]));
      const float m = max_across_rows(fmaxf(ma, mb)) * qk_mul;
      m_true[nt] = fmaxf(m_true[nt], m);
      need |= m - m_run[nt] >= kRescaleSlack;
    }
    if (fresh) {
      fresh = false;
#pragma unroll
      for (int nt = 0; nt < NT; ++nt) m_run[nt] = m_true[nt];
    } else if (__any(need)) {
#pragma unroll
      for (int nt = 0; nt < NT; ++nt) rescale(nt, m_true[nt]);
    }
#pragma unroll
    for (int nt = 0; nt < NT; ++nt) {
      const float mref = (m_run[nt] == -__builtin_inff()) ? 0.0f : m_run[nt];
      float pe[8];
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        pe[e] = fast_exp2(__builtin_fmaf(sa[nt][e], qk_mul, -mref));
        pe[4 + e] = fast_exp2(__builtin_fmaf(sb[nt][e], qk_mul, -mref));
      }
      pop[nt] = f16x8{(_Float16)pe[0], (_Float16)pe[1], (_Float16)pe[2], (_Float16)pe[3],
                      (_Float16)pe[4], (_Float16)pe[5], (_Float16)pe[6], (_Float16)pe[7]};
    }
  }

  // The four tokens x 16 dims V^T operand of dim tile rr of one step.
  __device__ f16x4 v_operand(const u32x4 (&v)[NLD], int rr) const {
    if constexpr (ELEM == 2) {
      const u32x4 raw = v[rr >> 1];
      return __builtin_bit_cast(f16x4, (rr & 1) ? u32x2{raw[2], raw[3]} : u32x2{raw[0], raw[1]});
    } else {
      const u32x4 raw = v[rr >> 2];
      if constexpr (KIND == kI8) return i8x4_to_f16x4(raw[rr & 3], vbias);
      else return e4m3x4_to_f16x4(raw[rr & 3]);
    }
  }

  __device__ void pair_pv(const u32x4 (&va)[NLD], const u32x4 (&vb)[NLD], const f16x8 (&pop)[NT]) {
    const f16x8 ones{1, 1, 1, 1, 1, 1, 1, 1};
#pragma unroll
    for (int nt = 0; nt < NT; ++nt) lacc[nt] = __builtin_amdgcn_mfma_f32_16x16x32_f16(ones, pop[nt], lacc[nt], 0, 0, 0);
#pragma unroll
    for (int rr = 0; rr < NDT; ++rr) {
      const f16x4 a = v_operand(va, rr);
      const f16x4 b = v_operand(vb, rr);
      const f16x8 vop{a[0], a[1], a[2], a[3], b[0], b[1], b[2], b[3]};
#pragma unroll
      for (int nt = 0; nt < NT; ++nt)
        oacc[nt][rr] = __builtin_amdgcn_mfma_f32_16x16x32_f16(vop, pop[nt], oacc[nt][rr], 0, 0, 0);
    }
  }

  // The largest base-2 logit of one column over the step's 16 tokens, from
  // its four raw scores in each lane (qk_mul > 0).
  __device__ float col_max(const f32x4& sc) const {
    return max_across_rows(fmaxf(fmaxf(sc[0], sc[1]), fmaxf(sc[2], sc[3]))) * qk_mul;
  }

  // Moves column tile nt's reference to m_new, rescaling what it holds.
  __device__ void rescale(int nt, float m_new) {
    // MULTI: a column with nothing visible yet keeps its empty state.
    if (MULTI && m_new == -__builtin_inff()) return;
    const float alpha = fast_exp2(m_run[nt] - m_new);
    l_part[nt] *= alpha;
    if constexpr (MULTI) lacc[nt] *= alpha;
#pragma unroll
    for (int rr = 0; rr < NDT; ++rr) oacc[nt][rr] *= alpha;
    m_run[nt] = m_new;
  }

  // MULTI: the denominators as per-row parts (a quarter of the whole sum in
  // each of the four rows, exact), the form the merges sum across rows.
  __device__ void finish_l() {
#pragma unroll
    for (int nt = 0; nt < NT; ++nt) l_part[nt] = lacc[nt][0] * 0.25f;
  }

  // LAST: one of the stream's last kDepth scheduled steps, the only ones that
  // can reach the end of the context (the step holding token T - 1 is the
  // last real one) and hold the fused new token; the other steps are
  // compiled without the tail mask and the injection.
  template <bool LAST = false>
  __device__ void compute(Regs& r, int tb) {
    static_assert(!MULTI, "multi-token steps go through the pair functions");
    bool new_here = false;  // step holds the fused new token, to be used
    if constexpr (FUSE && LAST) {
      if (knew && tb + 16 >= T && new_slot_ok()) {
        new_here = true;
        owns_new = true;
        inject_k(r);
        store_new_k(r);
      }
    }
    // S^T = K Q^T
    f32x4 s[NT];
    raw_scores(r.k, s);
    // Scores of tokens tb + 4*gq + e for head column n; mask the tail.
    // vtail / valid_here: tokens of this lane's 4 that exist (also for the
    // V mask).  The tail is masked on the raw scores
    // (the slots past the context may hold anything), only in the last steps
    // (as selects: a branch straight after the score MFMAs has left the
    // compiler's wait states for their results out of the path that skips
    // it); each probability is then one exp2(fma(s, qk_mul, -ref)).
    const bool vtail = LAST && tb + 16 > T;
    const int valid_here = T - (tb + 4 * gq);
    if constexpr (LAST) {
      const int vh = vtail ? valid_here : 4;
#pragma unroll
      for (int nt = 0; nt < NT; ++nt)
#pragma unroll
        for (int e = 0; e < 4; ++e)
          if (e >= vh) s[nt][e] = -__builtin_inff();
    }
    if constexpr (kLazy) {
      // The reference moves only when a score exceeds it by kRescaleSlack or
      // more, so exponentials stay below 2^kRescaleSlack (exact in fp16 and
      // fp32) and the accumulators are rescaled rarely; the first step after a
      // reset takes its own maximum, with nothing to rescale.
      bool need = false;
#pragma unroll
      for (int nt = 0; nt < NT; ++nt) {
        const float m = col_max(s[nt]);
        m_true[nt] = fmaxf(m_true[nt], m);
        need |= m - m_run[nt] >= kRescaleSlack;
      }
      if (fresh) {
        fresh = false;
#pragma unroll
        for (int nt = 0; nt < NT; ++nt) m_run[nt] = m_true[nt];
      } else if (__any(need)) {
#pragma unroll
        for (int nt = 0; nt < NT; ++nt) rescale(nt, m_true[nt]);
      }
    } else {
      float mnew[NT];
      bool grow = false;
#pragma unroll
      for (int nt = 0; nt < NT; ++nt) {
        mnew[nt] = fmaxf(m_run[nt], col_max(s[nt]));
        grow |= mnew[nt] > m_run[nt];
      }
      if (__any(grow)) {
#pragma unroll
        for (int nt = 0; nt < NT; ++nt) rescale(nt, mnew[nt]);
      }
    }
    f16x4 pop[NT];
#pragma unroll
    for (int nt = 0; nt < NT; ++nt) {
      float pe[4];
      const float mref = m_run[nt];
#pragma unroll
      for (int e = 0; e < 4; ++e) pe[e] = fast_exp2(__builtin_fmaf(s[nt][e], qk_mul, -mref));
      l_part[nt] += (pe[0] + pe[1]) + (pe[2] + pe[3]);
      pop[nt] = f16x4{(_Float16)pe[0], (_Float16)pe[1], (_Float16)pe[2], (_Float16)pe[3]};
    }
    if constexpr (FUSE && LAST) {
      if (new_here) {
        inject_v(r);
        store_new_v(r);
      }
    }
    // Unused slots of the last block may hold anything (NaN included): zero them,
    // since 0 * NaN would poison the product.
    if (vtail) {
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
    for (int rr = 0; rr < NDT; ++rr) {
      f16x4 vop;
      if constexpr (ELEM == 2) {
        const u32x4 raw = r.v[rr >> 1];
        vop = __builtin_bit_cast(f16x4, (rr & 1) ? u32x2{raw[2], raw[3]} : u32x2{raw[0], raw[1]});
      } else {
        const u32x4 raw = r.v[rr >> 2];
        if constexpr (KIND == kI8) vop = i8x4_to_f16x4(raw[rr & 3], vbias);
        else vop = e4m3x4_to_f16x4(raw[rr & 3]);
      }
#pragma unroll
      for (int nt = 0; nt < NT; ++nt)
        oacc[nt][rr] = __builtin_amdgcn_mfma_f32_16x16x16f16(vop, pop[nt], oacc[nt][rr], 0, 0, 0);
    }
  }
};

// Ids of the first 2*kDepth - 1 steps of a stream, requested before the
// context length is known so the two loads overlap.
struct FirstIds {
  int lo[2 * kDepth - 1], hi[2 * kDepth - 1];
};

// Runs the scheduled steps j = 0 .. n-1 (n >= 1) of a wave through a
// kDepth-deep register pipeline.  tok_of(j) is the first token of step j when
// the step holds real tokens, and otherwise the first token of a real step
// whose tiles it re-reads; real(j) tells which.  Real steps are computed;
// after(j) is called for every scheduled step.  The steady state has no
// data-dependent branch around any vector load, so the compiler's wait counts
// see the same outstanding loads on every path and each step waits only for
// its own tiles; to keep it so, steps are padded to a multiple of kDepth with
// look-ahead loads that re-read a real step's tiles (cache hits).  The ids of
// a block of look-ahead steps are fetched one block ahead.
template <class Dec, class TokOf, class Real, class After>
__device__ inline void stream_steps(Dec& dec, int n, TokOf tok_of, Real real, FirstIds& f, After after) {
  constexpr int D = kDepth;
  const int n_pad = (n + D - 1) / D * D;
  auto tok_at = [&](int j) { return tok_of(j < n ? j : n - 1); };
  if (!real(2 * D - 2 < n ? 2 * D - 2 : n - 1) || n < 2 * D - 1) {
#pragma unroll
    for (int j = 0; j < 2 * D - 1; ++j) dec.fetch_ids(tok_at(j), f.lo[j], f.hi[j]);
  }
  typename Dec::Regs rr[D];
  int cur_lo[D], cur_hi[D], nxt_lo[D], nxt_hi[D];
#pragma unroll
  for (int d = 0; d < D - 1; ++d) dec.issue(rr[d], tok_at(d), f.lo[d], f.hi[d]);
#pragma unroll
  for (int d = 0; d < D; ++d) {
    cur_lo[d] = f.lo[d + D - 1];
    cur_hi[d] = f.hi[d + D - 1];
  }
  // One block of D scheduled steps; LAST: the final block, whose steps may
  // reach the end of the context and hold the fused new token.
  auto block = [&](int j, auto last) {
#pragma unroll
    for (int d = 0; d < D; ++d) dec.fetch_ids(tok_at(j + d + 2 * D - 1), nxt_lo[d], nxt_hi[d]);
#pragma unroll
    for (int d = 0; d < D; ++d) {
      dec.issue(rr[(d + D - 1) % D], tok_at(j + d + D - 1), cur_lo[d], cur_hi[d]);
      if (j + d < n) {
        if (real(j + d)) dec.template compute<decltype(last)::value>(rr[d], tok_of(j + d));
        after(j + d);
      }
    }
#pragma unroll
    for (int d = 0; d < D; ++d) {
      cur_lo[d] = nxt_lo[d];
      cur_hi[d] = nxt_hi[d];
    }
  };
  for (int j = 0; j < n_pad - D; j += D) block(j, std::false_type{});
  block(n_pad - D, std::true_type{});
}

// MULTI: runs steps j = 0 .. n-1 (padded to pairs) two at a time.  tok_of
// and real as for stream_steps.  Loads are split so that each has about one
// pair of work to hide behind: the next pair's K tiles are loaded as soon as
// this pair's scores have used each K tile, its V tiles after the P.V
// product.  Block ids are fetched a pair ahead.
template <class Dec, class TokOf, class Real>
__device__ inline void stream_pairs(Dec& dec, int n, TokOf tok_of, Real real) {
  constexpr int NT = Dec::kNT;
  const int pairs = (n + 1) >> 1;
  auto tok_at = [&](int j) { return tok_of(j < n ? j : n - 1); };
  auto real_at = [&](int j) { return j < n && real(j); };
  int lo[4], hi[4];
#pragma unroll
  for (int j = 0; j < 4; ++j) dec.fetch_ids(tok_at(j), lo[j], hi[j]);
  typename Dec::Regs a, b;
  dec.issue(a, tok_at(0), lo[0], hi[0]);
  dec.issue(b, tok_at(1), lo[1], hi[1]);
  for (int pr = 0; pr < pairs; ++pr) {
    const int j = 2 * pr;
    int nlo[2], nhi[2];
    dec.fetch_ids(tok_at(j + 4), nlo[0], nhi[0]);
    dec.fetch_ids(tok_at(j + 5), nlo[1], nhi[1]);
    const int ta = tok_at(j), tb = tok_at(j + 1);
    const bool ra = real_at(j), rb = real_at(j + 1);
    f32x4 sa[NT], sb[NT];
    dec.pair_scores(a.k, ta, ra, sa);
    dec.template issue<true, false>(a, tok_at(j + 2), lo[2], hi[2]);
    dec.pair_scores(b.k, tb, rb, sb);
    dec.template issue<true, false>(b, tok_at(j + 3), lo[3], hi[3]);
    f16x8 pop[NT];
    dec.pair_softmax(sa, sb, pop);
    dec.pair_mask_v(a.v, ta, ra);
    dec.pair_mask_v(b.v, tb, rb);
    dec.pair_pv(a.v, b.v, pop);
    dec.template issue<false, true>(a, tok_at(j + 2), lo[2], hi[2]);
    dec.template issue<false, true>(b, tok_at(j + 3), lo[3], hi[3]);
    lo[0] = lo[2]; hi[0] = hi[2]; lo[1] = lo[3]; hi[1] = hi[3];
    lo[2] = nlo[0]; hi[2] = nhi[0]; lo[3] = nlo[1]; hi[3] = nhi[1];
  }
}

// LDS of the four-wave merge.
template <int NT, int D>
struct MergeLds {
  float m[kWaves][NT * 16];
  float l[kWaves][NT * 16];
  float o[kWaves - 1][NT * 16][D + 4];  // rows padded by four floats
  float mt[kWaves][NT * 16];  // largest scores (lazy rescaling only)
};

// Merges the (reference, sum, O) of the workgroup's four waves for every head
// column and lets wave 0 emit(nt, col, acc[D / 16] = sum_w O_w * 2^(m_w - M), M, L,
// Mt) with M the largest reference, L = sum_w l_w * 2^(m_w - M) and Mt the
// largest score (Mt = M where the reference is the running maximum).  All
// four waves must call it; two barriers.
template <class Dec, class Emit>
__device__ inline void merge_waves(Dec& dec, MergeLds<Dec::kNT, Dec::kD>& sm, int w, int group, Emit emit) {
  constexpr int NT = Dec::kNT;
  constexpr int NDT = Dec::NDT;
  const int gq = dec.gq, n = dec.n;
#pragma unroll
  for (int nt = 0; nt < NT; ++nt) {
    const float l = sum_across_rows(dec.l_part[nt]);
    if (gq == 0) {
      sm.m[w][nt * 16 + n] = dec.m_run[nt];
      if constexpr (Dec::kLazy) sm.mt[w][nt * 16 + n] = dec.m_true[nt];
      sm.l[w][nt * 16 + n] = l;
    }
  }
  __syncthreads();
  float big_m[NT], big_mt[NT], big_l[NT], f[NT];
#pragma unroll
  for (int nt = 0; nt < NT; ++nt) {
    const int col = nt * 16 + n;
    float M = sm.m[0][col];
#pragma unroll
    for (int ww = 1; ww < kWaves; ++ww) M = fmaxf(M, sm.m[ww][col]);
    big_mt[nt] = M;
    if constexpr (Dec::kLazy) {
      float Mt = sm.mt[0][col];
#pragma unroll
      for (int ww = 1; ww < kWaves; ++ww) Mt = fmaxf(Mt, sm.mt[ww][col]);
      big_mt[nt] = Mt;
    }
    float L = 0.0f;
#pragma unroll
    for (int ww = 0; ww < kWaves; ++ww) {
      const float mw = sm.m[ww][col];
      L += (mw == -__builtin_inff()) ? 0.0f : sm.l[ww][col] * exp2f(mw - M);
    }
    big_m[nt] = M;
    big_l[nt] = L;
    f[nt] = (dec.m_run[nt] == -__builtin_inff()) ? 0.0f : exp2f(dec.m_run[nt] - M);
    if (w > 0 && col < group) {
#pragma unroll
      for (int rr = 0; rr < NDT; ++rr)
        *reinterpret_cast<f32x4*>(&sm.o[w - 1][col][rr * 16 + 4 * gq]) = dec.oacc[nt][rr] * f[nt];
    }
  }
  __syncthreads();
  if (w != 0) return;
#pragma unroll
  for (int nt = 0; nt < NT; ++nt) {
    const int col = nt * 16 + n;
    if (col >= group) continue;
    f32x4 acc[NDT];
#pragma unroll
    for (int rr = 0; rr < NDT; ++rr) {
      const int dim = rr * 16 + 4 * gq;
      acc[rr] = dec.oacc[nt][rr] * f[nt];
#pragma unroll
      for (int ww = 0; ww < kWaves - 1; ++ww) acc[rr] += *reinterpret_cast<const f32x4*>(&sm.o[ww][col][dim]);
    }
    emit(nt, col, acc, big_m[nt], big_l[nt], big_mt[nt]);
  }
}

// Merge of a shared-prefix decode: the pieces of one grouped sequence (its
// group's shared chunks and its own tokens) wrote partials m, l, o into slots
// slot0 .. slot0 + parts - 1; out = sum_c w_c o_c / sum_c w_c with
// w_c = l_c * 2^(m_c - max_c m_c), for every query head of the KV head.  One
// workgroup per (sequence, KV head); lanes take four dims of one head.
template <int D>
__device__ inline void sp_merge_rows(const DecodeLaunch& p, int seq, int kvh, int group, int64_t slot0,
                                     int parts) {
  const int hq = p.num_q_heads;
  const int64_t r0 = static_cast<int64_t>(kvh) * group;
  for (int e = threadIdx.x; e < group * (D / 4); e += kWaves * 64) {
    const int h = e / (D / 4), d4 = e % (D / 4);
    float M = -__builtin_inff();
    for (int c = 0; c < parts; ++c) M = fmaxf(M, p.part_m[(slot0 + c) * hq + r0 + h]);
    f32x4 acc = {0.0f, 0.0f, 0.0f, 0.0f};
    float den = 0.0f;
    for (int c = 0; c < parts; ++c) {
      const int64_t idx = (slot0 + c) * hq + r0 + h;
      const float mc = p.part_m[idx];
      const float wc = (mc == -__builtin_inff()) ? 0.0f : p.part_l[idx] * exp2f(mc - M);
      den += wc;
      acc += *reinterpret_cast<const f32x4*>(p.part_o + idx * D + 4 * d4) * wc;
    }
    const f32x4 v = acc * (1.0f / den);
    *reinterpret_cast<f16x4*>(static_cast<_Float16*>(p.out) + (static_cast<int64_t>(seq) * hq + r0 + h) * D +
                              4 * d4) = f16x4{(_Float16)v[0], (_Float16)v[1], (_Float16)v[2], (_Float16)v[3]};
  }
}

enum DecodeMode : int {
  kSingle = 0,   // one workgroup per (sequence, KV head), fp16 output
  kSplit4 = 1,   // a workgroup's four waves share each chunk of a chunk run
  kSplit1 = 2,   // each wave streams its own chunk run
  kPrivate = 3,  // kSingle from each sequence's start on, merged with the
                 // shared pass's partials (shared-prefix decode)
};

// Context length of a sequence, clamped to the table width; bad lengths set
// PA_DEV_BAD_LEN (by one lane of the grid's first wave of the unit).
template <int BS>
__device__ inline int context_len(const PoolGeom& g, const DecodeLaunch& p, int seq, bool report) {
  int T = p.lens[seq];
  const int t_cap = p.max_blocks * BS;
  if (T < 1 || T > t_cap) {
    if (report) atomicOr(g.status, kDevBadLen);
    T = T < 0 ? 0 : (T > t_cap ? t_cap : T);
  }
  return T;
}

// Paged decode for one layer.
//  kSingle: workgroup = (sequence, KV head); wave w takes steps w, w+4, ...
//    of the whole context; the waves merge and write the fp16 output.
//  kSplit4: workgroup = (unit, r): chunks [r*k, min((r+1)*k, C)) of the unit,
//    chunk by chunk; within a chunk wave w takes steps w, w+4, ...; at each
//    chunk end the waves merge and write that chunk's partials.
//  kSplit1: wave (unit, r): the same chunk run, streamed by one wave, which
//    writes each chunk's partials itself.
// Partials of chunk c of query head h: m = max_t s_t (base 2),
// l = sum_t 2^(s_t - m), o = sum_t 2^(s_t - m) v_t / l (times the fp8 V scale).
// Chunks at or past ceil(T / P) are not written.
// At least two waves per SIMD: left to itself, the compiler gives the
// two-tile (G > 16) variants 340 VGPR+AGPR registers and one wave per SIMD,
// though they fit in 256 without spills; with two, MQA decode ran 10-13%
// faster on MI355X (one-tile variants measured the same either way).
template <int D, int KIND, int BS, int NT, int MODE, bool FUSE, bool CACHED>
__device__ __forceinline__ void decode_body(const PoolGeom& g, const DecodeLaunch& p, uint32_t bid,
                                            MergeLds<NT, D>& sm) {
  constexpr int kD = D;
  constexpr int ELEM = kind_bytes(KIND);
  constexpr bool kOne = MODE == kSingle || MODE == kPrivate;  // one pass per (sequence, KV head)
  const int lane = threadIdx.x & 63;
  const int w = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);  // wave-uniform
  const int group = p.num_q_heads / g.kv_heads;
  const int64_t num_units = static_cast<int64_t>(p.num_seqs) * g.kv_heads;
  int64_t unit;
  int r = 0;
  if constexpr (kOne) {
    unit = bid;
  } else if constexpr (MODE == kSplit4) {
    // Workgroup b runs on XCD b mod 8: the runs of each block of eight
    // consecutive units are numbered so that all runs of a unit share one
    // XCD (its query and table row are then fetched by one L2), and units
    // keep their order between blocks.
    const int64_t wpu = p.waves_per_unit;
    const int64_t blk = static_cast<int64_t>(bid) / (8 * wpu);
    const int64_t within = static_cast<int64_t>(bid) % (8 * wpu);
    const int64_t ub = (num_units - 8 * blk) < 8 ? (num_units - 8 * blk) : 8;
    unit = 8 * blk + within % ub;
    r = static_cast<int>(within / ub);
  } else {
    const int64_t v = static_cast<int64_t>(bid) * kWaves + w;
    unit = v / p.waves_per_unit;
    r = static_cast<int>(v % p.waves_per_unit);
    if (unit >= num_units) return;  // whole waves only: no barrier in this mode
  }
  const int kvh = static_cast<int>(unit % g.kv_heads);
  int seq = static_cast<int>(unit / g.kv_heads);
  if (p.order) {
    // Units are taken in the caller's sequence order (longest first evens out
    // the CUs' loads); the entry is wave-uniform, so this is a scalar load.
    seq = ((const ConstI32*)p.order)[seq];
    if (static_cast<uint32_t>(seq) >= static_cast<uint32_t>(p.num_seqs)) {
      if (lane == 0 && (MODE == kSplit1 || w == 0)) atomicOr(g.status, kDevBadOrder);
      return;  // whole workgroup (whole wave in kSplit1)
    }
  }
  const int P = p.partition_tokens;
  const int c_begin = r * p.chunks_per_wave;
  // The unit's last run also takes any remainder chunks (see the plan).
  const int c_end = (r == p.waves_per_unit - 1 || c_begin + p.chunks_per_wave > p.num_partitions)
                        ? p.num_partitions
                        : c_begin + p.chunks_per_wave;
  const int qs = P >> 6;   // kSplit4: steps of each wave per chunk
  const int spc = P >> 4;  // kSplit1: steps per chunk
  // Shared-prefix decode, private pass: the tokens before s0 were attended by
  // the shared pass; s0 is a multiple of 16 inside the table (else 0).  The
  // plain single pass keeps s0 = 0 at compile time.
  int s0 = 0;
  int64_t sp_slot = 0;  // this piece's partial slot
  if constexpr (MODE == kPrivate) {
    s0 = ((const ConstI32*)p.starts)[seq];
    s0 = (s0 < 0 || static_cast<int64_t>(s0) >= static_cast<int64_t>(p.max_blocks) * BS) ? 0 : (s0 & ~15);
    if (s0 > 0) {
      const int sp_parts = (s0 + p.sp_chunk - 1) / p.sp_chunk + 1;  // shared chunks + this piece
      const int slot0 = ((const ConstI32*)p.slot0)[seq];
      if (slot0 < 0 || slot0 > p.sp_slots - sp_parts) {
        // Inconsistent with the plan: flagged, attended as a plain single pass.
        if (threadIdx.x == 0) atomicOr(g.status, kDevBadLen);
        s0 = 0;
      }
      sp_slot = static_cast<int64_t>(slot0) + sp_parts - 1;
    }
  }
  // First token of scheduled step j, before any clamping to the context.
  auto raw_tok = [&](int j) -> int64_t {
    if constexpr (kOne) return s0 + 16ll * (w + kWaves * j);
    else if constexpr (MODE == kSplit4) return static_cast<int64_t>(c_begin + j / qs) * P + 16 * (w + kWaves * (j % qs));
    else return static_cast<int64_t>(c_begin) * P + 16ll * j;
  };

  using Dec = WaveDecoder<D, KIND, BS, NT, FUSE, false, CACHED>;
  Dec dec;
  if constexpr (FUSE && ELEM == 1) {
    __shared__ __attribute__((aligned(16))) uint8_t new_codes[kWaves][2 * kD];
    dec.lds_new = new_codes[w];
  }
  dec.bind(g, p, seq, kvh, lane);
  FirstIds first;
#pragma unroll
  for (int j = 0; j < 2 * kDepth - 1; ++j) dec.fetch_ids(raw_tok(j), first.lo[j], first.hi[j]);
  const bool reporter = (MODE == kSplit1) ? (lane == 0 && r == 0) : (threadIdx.x == 0 && r == 0);
  const int T = context_len<BS>(g, p, seq, reporter);
  dec.T = T;
  // The one wave of the unit whose step holds token T - 1.
  bool owner = false;
  if constexpr (FUSE) {
    if (T > 0) {
      const int t_last = T - 1;
      if constexpr (kOne) {
        owner = t_last >= s0 && (((t_last - s0) >> 4) % kWaves) == w;
      } else {
        const int c_t = t_last / P;
        const bool in_run = c_t >= c_begin && c_t < c_end;
        if constexpr (MODE == kSplit4) owner = in_run && (((t_last - c_t * P) >> 4) % kWaves) == w;
        else owner = in_run;
      }
    }
  }
  if constexpr (FUSE) {
    if (owner) {
      // Fused scatter: the new token must be the context's last one, at the
      // slot the table gives token T - 1.  The slot, the table entry and the
      // scales are only requested here; the step holding token T - 1 checks
      // them, long after they have arrived.
      dec.new_slot = ((const ConstI32*)p.new_slots)[seq];
      dec.new_blk = dec.trow[(T - 1) / BS];
      const int64_t off = (static_cast<int64_t>(seq) * g.kv_heads + kvh) * kD;
      dec.knew = static_cast<const _Float16*>(p.k_new) + off;
      dec.vnew = static_cast<const _Float16*>(p.v_new) + off;
      if constexpr (ELEM == 1) {
        const int lhs = g.layers * g.kv_heads;
        const int lh = p.layer * g.kv_heads + kvh;
        dec.new_kinv = g.scales[2 * lhs + lh];
        dec.new_vinv = g.scales[3 * lhs + lh];
        if constexpr (KIND == kI8) {
          dec.new_kz = g.scales[4 * lhs + lh];
          dec.new_vz = g.scales[5 * lhs + lh];
        }
      }
    }
  }
  // The owner flags a slot that is not token T - 1's (a negative slot means:
  // no store); the store itself happened in the token's step.
  auto store_new = [&]() {
    if constexpr (FUSE) {
      if (owner && !dec.owns_new && dec.new_slot >= 0 && lane == 0) atomicOr(g.status, kDevBadSlot);
    }
  };

  if constexpr (kOne) {
    if (T <= s0) {
      // Nothing to attend to: defined output of zeros.  A context at or
      // below its shared tokens (a contract violation) is flagged and
      // contributes an empty part, so the output is the shared tokens' alone.
      if constexpr (MODE == kPrivate) {
        if (s0 > 0) {
          if (threadIdx.x == 0) atomicOr(g.status, kDevBadLen);
          const int64_t idx0 = sp_slot * p.num_q_heads + kvh * group;
          for (int i = threadIdx.x; i < group * kD; i += kWaves * 64) p.part_o[idx0 * kD + i] = 0.0f;
          for (int i = threadIdx.x; i < group; i += kWaves * 64) {
            p.part_m[idx0 + i] = -__builtin_inff();
            p.part_l[idx0 + i] = 0.0f;
          }
          return;
        }
      }
      for (int i = threadIdx.x; i < group * kD; i += kWaves * 64)
        static_cast<_Float16*>(p.out)[(static_cast<int64_t>(seq) * p.num_q_heads + kvh * group) * kD + i] = 0;
      return;
    }
  }
  // Chunks of the run that hold tokens, and the scheduled steps of each wave.
  const int c_last = (kOne) ? 0 : ((T + P - 1) / P < c_end ? (T + P - 1) / P : c_end);
  int n;
  if constexpr (kOne) {
    n = (T - s0 + 16 * kWaves - 1) / (16 * kWaves);  // same count for every wave
  } else if constexpr (MODE == kSplit4) {
    if (c_begin >= c_last) return;  // whole workgroup
    const int rest = static_cast<int>(T - static_cast<int64_t>(c_last - 1) * P);  // tokens of the run's last chunk
    n = (c_last - 1 - c_begin) * qs + ((rest < P ? rest : P) + 16 * kWaves - 1) / (16 * kWaves);
  } else {
    if (c_begin >= c_last) return;
    const int64_t tok1 = (static_cast<int64_t>(c_last) * P < T) ? static_cast<int64_t>(c_last) * P : T;
    n = static_cast<int>((tok1 - static_cast<int64_t>(c_begin) * P + 15) >> 4);
  }
  // Steps at or past the context re-read the context's last step.
  const int last_tok = ((T - 1) >> 4) << 4;
  auto real = [&](int j) { return raw_tok(j) < T; };
  auto tok_of = [&](int j) -> int { return real(j) ? static_cast<int>(raw_tok(j)) : last_tok; };

  dec.load_q(g, p, seq, kvh, group);
  dec.reset();
  if constexpr (FUSE) {
    if (dec.knew) dec.load_new();
  }
  const int gq = dec.gq;
  const int64_t row0 = static_cast<int64_t>(seq) * p.num_q_heads + kvh * group;

  if constexpr (kOne) {
    stream_steps(dec, n, tok_of, real, first, [](int) {});
    if (dec.bad && lane == 0) atomicOr(g.status, dec.bad);
    merge_waves(dec, sm, w, group, [&](int nt, int col, f32x4* acc, float M, float L, float Mt) {
      (void)nt;
      if (MODE == kPrivate && s0 > 0) {
        // The private tokens' partials, in the sequence's last slot.
        const int64_t idx = sp_slot * p.num_q_heads + kvh * group + col;
        const float inv_l = dec.out_mul / L;
        float* po = p.part_o + idx * kD + 4 * gq;
#pragma unroll
        for (int rr = 0; rr < D / 16; ++rr) *reinterpret_cast<f32x4*>(po + rr * 16) = acc[rr] * inv_l;
        if (gq == 0) {
          p.part_m[idx] = Mt;
          p.part_l[idx] = (!Dec::kLazy || M == Mt) ? L : L * exp2f(M - Mt);
        }
        return;
      }
      _Float16* po = static_cast<_Float16*>(p.out) + (row0 + col) * kD + 4 * gq;
      const float inv_l = dec.out_mul / L;
#pragma unroll
      for (int rr = 0; rr < D / 16; ++rr) {
        const f32x4 a = acc[rr] * inv_l;
        *reinterpret_cast<f16x4*>(po + rr * 16) = f16x4{(_Float16)a[0], (_Float16)a[1], (_Float16)a[2], (_Float16)a[3]};
      }
    });
    store_new();  // after the merge: its barriers would wait for these stores
  } else if constexpr (MODE == kSplit4) {
    auto after = [&](int j) {
      if ((j + 1) % qs != 0 && j + 1 != n) return;
      const int64_t c = c_begin + j / qs;
      merge_waves(dec, sm, w, group, [&](int nt, int col, f32x4* acc, float M, float L, float Mt) {
        (void)nt;
        const int64_t idx = (row0 + col) * p.num_partitions + c;
        const float inv_l = dec.out_mul / L;
        float* po = p.part_o + idx * kD + 4 * gq;
#pragma unroll
        for (int rr = 0; rr < D / 16; ++rr) *reinterpret_cast<f32x4*>(po + rr * 16) = acc[rr] * inv_l;
        if (gq == 0) {
          p.part_m[idx] = Mt;
          p.part_l[idx] = (!Dec::kLazy || M == Mt) ? L : L * exp2f(M - Mt);
        }
      });
      dec.reset();
    };
    stream_steps(dec, n, tok_of, real, first, after);
    if (dec.bad && lane == 0) atomicOr(g.status, dec.bad);
    store_new();
  } else {
    const int nn = dec.n;
    auto after = [&](int j) {
      if ((j + 1) % spc != 0 && j + 1 != n) return;
      const int64_t c = c_begin + j / spc;
#pragma unroll
      for (int nt = 0; nt < NT; ++nt) {
        const float l = sum_across_rows(dec.l_part[nt]);
        const int col = nt * 16 + nn;
        if (col < group) {
          const int64_t idx = (row0 + col) * p.num_partitions + c;
          const float inv_l = dec.out_mul / l;
          float* po = p.part_o + idx * kD + 4 * gq;
#pragma unroll
          for (int rr = 0; rr < D / 16; ++rr) *reinterpret_cast<f32x4*>(po + rr * 16) = dec.oacc[nt][rr] * inv_l;
          if (gq == 0) {
            const float mt = dec.top(nt);
            p.part_m[idx] = mt;
            p.part_l[idx] = (!Dec::kLazy || dec.m_run[nt] == mt) ? l : l * exp2f(dec.m_run[nt] - mt);
          }
        }
      }
      dec.reset();
    };
    stream_steps(dec, n, tok_of, real, first, after);
    if (dec.bad && lane == 0) atomicOr(g.status, dec.bad);
    store_new();
  }
}

template <int D, int KIND, int BS, int NT, int MODE, bool FUSE, bool CACHED>
__global__ __launch_bounds__(kWaves * 64) __attribute__((amdgpu_waves_per_eu(2)))
void decode_kernel(PoolGeom g, DecodeLaunch p) {
  __shared__ MergeLds<NT, D> sm;
  decode_body<D, KIND, BS, NT, MODE, FUSE, CACHED>(g, p, blockIdx.x, sm);
}

// Causal attention of a tile of new query tokens of one sequence over its
// paged context, for one KV head (youngju.dev "KV cache and paged
// attention", section "핵심 원리: KV 캐시란 무엇인가": a token's query meets
// the keys and values of itself and every earlier token; iq-blog ch.4: the
// scheduler mixes prefill chunks and decode tokens in one batch).
// Workgroup = (work item, KV head): up to multi_token_tile(G) tokens
// j0, j0+1, ... of its sequence, whose n_i query tokens are the last n_i of
// its T_i; token j sits at position T_i - n_i + j and sees that many keys
// plus one.  Columns are (token, head) pairs, 32 per wave (two MFMA tiles),
// i.e. tq = multi_token_wave_tile(G) tokens per wave.
//  * wide (the item holds more than tq tokens): wave w takes tokens
//    j0 + w*tq ... and streams every key they see on its own; the four
//    waves read the same key tiles at about the same time, so three of the
//    four reads hit the CU's cache (plain loads, not nontemporal ones);
//  * split (at most tq tokens, e.g. a decode token): the four waves take key
//    steps w, w+4, ... and merge in LDS, as the single-pass decode does.
template <class Dec>
__device__ inline void multi_token_setup(Dec& dec, int base, int nq, int group, int row0, int& kmax) {
  const int ncols = nq * group;
  kmax = base + nq;  // keys the last token sees
  dec.T = kmax;
  dec.lim_min = base + 1;
#pragma unroll
  for (int nt = 0; nt < Dec::kNT; ++nt) {
    const int col = nt * 16 + dec.n;
    dec.lim[nt] = col < ncols ? base + col / group + 1 : kmax;
  }
  dec.mt_row0 = row0;
  dec.mt_ncols = ncols;
}

// fp16 output of a wave's (or a merge's) accumulators for column col.
template <class Dec>
__device__ inline void multi_token_store(const DecodeLaunch& p, const Dec& dec, const f32x4* acc, float inv_l,
                                         int row0, int col, int kvh, int group) {
  constexpr int kD = Dec::kD;
  _Float16* po = static_cast<_Float16*>(p.out) +
                 ((static_cast<int64_t>(row0) + col / group) * p.num_q_heads + kvh * group + col % group) * kD +
                 4 * dec.gq;
#pragma unroll
  for (int rr = 0; rr < kD / 16; ++rr) {
    const f32x4 a = acc[rr] * inv_l;
    *reinterpret_cast<f16x4*>(po + rr * 16) = f16x4{(_Float16)a[0], (_Float16)a[1], (_Float16)a[2], (_Float16)a[3]};
  }
}

template <int D, int KIND, int BS>
__global__ __launch_bounds__(kWaves * 64) __attribute__((amdgpu_waves_per_eu(2)))
void multi_token_kernel(PoolGeom g, DecodeLaunch p) {
  constexpr int NT = 2;
  constexpr int kD = D;
  const int lane = threadIdx.x & 63;
  const int w = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int group = p.num_q_heads / g.kv_heads;
  const int tq = multi_token_wave_tile(group);
  const int item = static_cast<int>(blockIdx.x / g.kv_heads);
  const int kvh = static_cast<int>(blockIdx.x % g.kv_heads);
  const ConstI32* wk = (const ConstI32*)(p.work + 4 * static_cast<int64_t>(item));
  const int seq = wk[0], j0 = wk[1], row0 = wk[2], n_i = wk[3];
  const int nq_item = (n_i - j0) < kWaves * tq ? (n_i - j0) : kWaves * tq;
  const bool wide = nq_item > tq;  // uniform over the workgroup
  int T = p.lens[seq];
  if (T < n_i || T > p.max_blocks * BS) {
    // The context must hold the sequence's query tokens: flag it and give
    // the item's rows a defined output of zeros.
    if (threadIdx.x == 0) atomicOr(g.status, kDevBadLen);
    for (int i = threadIdx.x; i < nq_item * group * kD; i += kWaves * 64) {
      const int col = i / kD;
      static_cast<_Float16*>(p.out)[((static_cast<int64_t>(row0) + col / group) * p.num_q_heads + kvh * group +
                                     col % group) * kD + i % kD] = 0;
    }
    return;
  }
  int kmax;
  if (wide) {
    WaveDecoder<D, KIND, BS, NT, false, true, true> dec;  // key tiles shared by the four waves
    dec.bind(g, p, seq, kvh, lane);
    const int jw = w * tq;  // this wave's first token within the item
    if (jw >= nq_item) return;  // no tokens for this wave (no barrier on this path)
    const int nq = (nq_item - jw) < tq ? (nq_item - jw) : tq;
    auto raw_tok = [](int j) -> int { return 16 * j; };
    multi_token_setup(dec, T - n_i + j0 + jw, nq, group, row0 + jw, kmax);
    const int n = (kmax + 15) >> 4;
    const int last_tok = ((kmax - 1) >> 4) << 4;
    auto real = [&](int j) { return raw_tok(j) < kmax; };
    auto tok_of = [&](int j) -> int { return real(j) ? static_cast<int>(raw_tok(j)) : last_tok; };
    dec.load_q(g, p, seq, kvh, group);
    dec.reset();
    stream_pairs(dec, n, tok_of, real);
    dec.finish_l();
    if (dec.bad && lane == 0) atomicOr(g.status, dec.bad);
#pragma unroll
    for (int nt = 0; nt < NT; ++nt) {
      const float l = sum_across_rows(dec.l_part[nt]);
      const int col = nt * 16 + dec.n;
      if (col < nq * group) multi_token_store(p, dec, dec.oacc[nt], dec.out_mul / l, row0 + jw, col, kvh, group);
    }
  } else {
    WaveDecoder<D, KIND, BS, NT, false, true, false> dec;  // each key tile read once
    dec.bind(g, p, seq, kvh, lane);
    auto raw_tok = [&](int j) -> int { return 16 * (w + kWaves * j); };
    multi_token_setup(dec, T - n_i + j0, nq_item, group, row0, kmax);
    const int n = (kmax + 16 * kWaves - 1) / (16 * kWaves);
    const int last_tok = ((kmax - 1) >> 4) << 4;
    auto real = [&](int j) { return raw_tok(j) < kmax; };
    auto tok_of = [&](int j) -> int { return real(j) ? static_cast<int>(raw_tok(j)) : last_tok; };
    dec.load_q(g, p, seq, kvh, group);
    dec.reset();
    __shared__ MergeLds<NT, D> sm;
    stream_pairs(dec, n, tok_of, real);
    dec.finish_l();
    if (dec.bad && lane == 0) atomicOr(g.status, dec.bad);
    merge_waves(dec, sm, w, nq_item * group, [&](int, int col, f32x4* acc, float, float L, float) {
      multi_token_store(p, dec, acc, dec.out_mul / L, row0, col, kvh, group);
    });
  }
}

// Partials of a folded item's shared tokens, per (member, head) column.
template <int D>
struct FoldLds {
  float m[32];
  float l[32];
  float o[32][D + 4];  // rows padded by four floats
};

// Private tokens of one member of a folded shared-prefix item, by one wave:
// tokens ts .. T - 1 of sequence `seq` (with the fused write of its new token
// when p.new_slots is set), then the log-sum-exp merge with the item's shared
// partials of the member's columns col0 .. col0 + G - 1 (in `fl`) into the
// fp16 output.  A context at or below ts (a contract violation) is flagged
// and the output is the shared tokens' alone.
template <int D, int KIND, int BS, int NTP, bool FUSE, bool CACHED>
__device__ inline void folded_private(const PoolGeom& g, const DecodeLaunch& p, int seq, int kvh, int group,
                                      int ts, int col0, const FoldLds<D>& fl, uint8_t* lds_new, int lane) {
  constexpr int ELEM = kind_bytes(KIND);
  using Dec = WaveDecoder<D, KIND, BS, NTP, FUSE, false, CACHED>;
  Dec dec;
  if constexpr (FUSE && ELEM == 1) dec.lds_new = lds_new;
  dec.bind(g, p, seq, kvh, lane);
  const int T = context_len<BS>(g, p, seq, lane == 0);
  dec.T = T;
  dec.load_q(g, p, seq, kvh, group);
  dec.reset();
  const bool own = T > ts;  // this wave runs every private step, so it holds token T - 1
  if (!own && lane == 0) atomicOr(g.status, kDevBadLen);
  if constexpr (FUSE) {
    if (own && p.new_slots) {
      dec.new_slot = ((const ConstI32*)p.new_slots)[seq];
      dec.new_blk = dec.trow[(T - 1) / BS];
      const int64_t off = (static_cast<int64_t>(seq) * g.kv_heads + kvh) * D;
      dec.knew = static_cast<const _Float16*>(p.k_new) + off;
      dec.vnew = static_cast<const _Float16*>(p.v_new) + off;
      if constexpr (ELEM == 1) {
        const int lhs = g.layers * g.kv_heads;
        const int lh = p.layer * g.kv_heads + kvh;
        dec.new_kinv = g.scales[2 * lhs + lh];
        dec.new_vinv = g.scales[3 * lhs + lh];
        if constexpr (KIND == kI8) {
          dec.new_kz = g.scales[4 * lhs + lh];
          dec.new_vz = g.scales[5 * lhs + lh];
        }
      }
      dec.load_new();
    }
  }
  if (own) {
    const int n = (T - ts + 15) >> 4;
    const int last_tok = ((T - 1) >> 4) << 4;
    auto real = [&](int j) { return j < n; };
    auto tok_of = [&](int j) -> int { return j < n ? ts + 16 * j : last_tok; };
    FirstIds first;
#pragma unroll
    for (int j = 0; j < 2 * kDepth - 1; ++j) dec.fetch_ids(tok_of(j), first.lo[j], first.hi[j]);
    stream_steps(dec, n, tok_of, real, first, [](int) {});
    if constexpr (FUSE) {
      if (dec.knew && !dec.owns_new && dec.new_slot >= 0 && lane == 0) atomicOr(g.status, kDevBadSlot);
    }
  }
  if (dec.bad && lane == 0) atomicOr(g.status, dec.bad);
  const int gq = dec.gq;
#pragma unroll
  for (int nt = 0; nt < NTP; ++nt) {
    const float L = sum_across_rows(dec.l_part[nt]);
    const int c = nt * 16 + dec.n;
    if (c >= group) continue;
    const int cs = col0 + c;
    const float m_s = fl.m[cs], l_s = fl.l[cs];
    const float r = dec.m_run[nt];  // the reference of the accumulators (-inf: nothing attended)
    const float X = fmaxf(r, m_s);
    const float a = (r == -__builtin_inff()) ? 0.0f : exp2f(r - X);
    const float b = l_s * exp2f(m_s - X);
    const float inv = 1.0f / (L * a + b);
    _Float16* po = static_cast<_Float16*>(p.out) +
                   (static_cast<int64_t>(seq) * p.num_q_heads + kvh * group + c) * D + 4 * gq;
#pragma unroll
    for (int rr = 0; rr < D / 16; ++rr) {
      const f32x4 os = *reinterpret_cast<const f32x4*>(&fl.o[cs][rr * 16 + 4 * gq]);
      const f32x4 v = (dec.oacc[nt][rr] * (a * dec.out_mul) + os * b) * inv;
      *reinterpret_cast<f16x4*>(po + rr * 16) = f16x4{(_Float16)v[0], (_Float16)v[1], (_Float16)v[2], (_Float16)v[3]};
    }
  }
}

// Shared-prefix decode: one launch whose first workgroups read the blocks
// that groups of sequences share (beams of one search, requests on one cached
// system prompt: youngju.dev "KV cache and paged attention", section "prefix
// 공유와 copy-on-write") once for all the group's members, and whose other
// workgroups attend to each sequence's own tokens, every piece of a grouped
// sequence writing partials; a second launch (shared_merge_kernel) merges
// them.
//
// Shared piece (shared_body): an item is (first member, members, shared
// tokens ts, chunk c) and takes the group's tokens [c * chunk, min((c + 1) *
// chunk, ts)) for up to 32 / G members, whose query heads are the MFMA
// columns of one tile pair (column k: member k / G, head k % G); the four
// waves take key steps w, w + 4, ... and merge in LDS, and every (member,
// head) row gets its partials m (the largest score, base 2), l = sum 2^(s -
// m), o = sum 2^(s - m) v / l (times the V scale) in slot slot0[member] + c.
// The blocks are read through the first member's table, with ordinary loads
// where several items of a group re-read them, nontemporal ones otherwise.
template <int D, int KIND, int BS, int NTP, bool FUSE, bool CACHED>
__device__ __forceinline__ void shared_body(const PoolGeom& g, const DecodeLaunch& p, uint32_t bid,
                                            MergeLds<2, D>& sm, FoldLds<D>& fl, uint8_t* lds_new) {
  constexpr int NT = 2;
  const int lane = threadIdx.x & 63;
  const int w = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int group = p.num_q_heads / g.kv_heads;
  const int item = static_cast<int>(bid / g.kv_heads);
  const int kvh = static_cast<int>(bid % g.kv_heads);
  const ConstI32* wk = (const ConstI32*)(p.work + 4 * static_cast<int64_t>(item));
  const int m0 = wk[0], nm = wk[1], ts = wk[2], c = wk[3];
  const bool folded = c < 0;  // the whole shared run, then each member's own tokens in this workgroup
  const int chunk = p.sp_chunk;
  const int parts = folded ? 0 : (ts + chunk - 1) / chunk + 1;
  // The host checks the items when it uploads them; an item that does not
  // fit this launch (a member run outside the batch, more than 32 columns, a
  // member outside the batch or without room for its slots, a shared length
  // outside the table or not a multiple of 16, a chunk past it) is flagged
  // and its rows left alone.  Every wave reaches the same verdict, so the
  // workgroup leaves together.
  if (m0 < 0 || nm < 1 || nm * group > 32 || m0 > p.num_seqs - nm || ts < 16 || (ts & 15) != 0 ||
      static_cast<int64_t>(ts) > static_cast<int64_t>(p.max_blocks) * BS || c < -1 ||
      static_cast<int64_t>(c) * chunk >= ts) {
    if (threadIdx.x == 0) atomicOr(g.status, kDevBadLen);
    return;
  }
  const int32_t* mem = p.members + m0;
  const int mine = lane < nm ? ((const ConstI32*)mem)[lane] : 0;
  const int my_slot0 = (lane < nm && !folded) ? ((const ConstI32*)p.slot0)[mine] : 0;
  if (__ballot(static_cast<uint32_t>(mine) >= static_cast<uint32_t>(p.num_seqs) || my_slot0 < 0 ||
               my_slot0 > p.sp_slots - parts) != 0) {
    if (threadIdx.x == 0) atomicOr(g.status, kDevBadLen);
    return;
  }
  const int seq0 = __builtin_amdgcn_readfirstlane(mine);
  const int t0 = folded ? 0 : c * chunk;
  const int t1 = (folded || ts - t0 < chunk) ? ts : t0 + chunk;
  WaveDecoder<D, KIND, BS, NT, false, true, CACHED> dec;
  dec.bind(g, p, seq0, kvh, lane);
  const int ncols = nm * group;
  dec.T = t1;
  dec.lim_min = t1;
#pragma unroll
  for (int nt = 0; nt < NT; ++nt) dec.lim[nt] = t1;
  dec.mt_row0 = 0;
  dec.mt_ncols = ncols;
  dec.mt_rowmap = mem;
  auto raw_tok = [&](int j) -> int { return t0 + 16 * (w + kWaves * j); };
  const int n = (t1 - t0 + 16 * kWaves - 1) / (16 * kWaves);
  const int last_tok = ((t1 - 1) >> 4) << 4;
  auto real = [&](int j) { return raw_tok(j) < t1; };
  auto tok_of = [&](int j) -> int { return real(j) ? static_cast<int>(raw_tok(j)) : last_tok; };
  dec.load_q(g, p, seq0, kvh, group);
  dec.reset();
  stream_pairs(dec, n, tok_of, real);
  dec.finish_l();
  if (dec.bad && lane == 0) atomicOr(g.status, dec.bad);
  const int gq = dec.gq;
  if (folded) {
    // Shared partials into LDS, then each wave takes members w, w + 4, ...
    merge_waves(dec, sm, w, ncols, [&](int, int col, f32x4* acc, float M, float L, float Mt) {
      const float inv_l = dec.out_mul / L;
#pragma unroll
      for (int rr = 0; rr < D / 16; ++rr) *reinterpret_cast<f32x4*>(&fl.o[col][rr * 16 + 4 * gq]) = acc[rr] * inv_l;
      if (gq == 0) {
        fl.m[col] = Mt;
        fl.l[col] = (M == Mt) ? L : L * exp2f(M - Mt);
      }
    });
    __syncthreads();
    for (int mi = w; mi < nm; mi += kWaves)
      folded_private<D, KIND, BS, NTP, FUSE, CACHED>(g, p, ((const ConstI32*)mem)[mi], kvh, group, ts, mi * group,
                                                     fl, lds_new, lane);
    return;
  }
  merge_waves(dec, sm, w, ncols, [&](int, int col, f32x4* acc, float M, float L, float Mt) {
    const int seq = mem[col / group];
    const int64_t idx = (static_cast<int64_t>(((const ConstI32*)p.slot0)[seq]) + c) * p.num_q_heads +
                        kvh * group + col % group;
    const float inv_l = dec.out_mul / L;
    float* po = p.part_o + idx * D + 4 * gq;
#pragma unroll
    for (int rr = 0; rr < D / 16; ++rr) *reinterpret_cast<f32x4*>(po + rr * 16) = acc[rr] * inv_l;
    if (gq == 0) {
      p.part_m[idx] = Mt;
      p.part_l[idx] = (M == Mt) ? L : L * exp2f(M - Mt);
    }
  });
}

// The shared-prefix pieces: workgroups 0 .. items * Hkv - 1 are shared
// pieces, the rest (sequence, KV head) private pieces of the sequences
// listed in `order` (decode_body in mode kPrivate: tokens starts[i] .. T_i -
// 1 into the sequence's last slot, or the whole context straight into `out`
// for a sequence in no group; a folded item's members have none).  One LDS
// buffer serves either body.  The pieces are independent, so the private
// ones run beside the long shared ones.
// Merge launch: one workgroup per (sequence, KV head); sequences in no
// group leave at once.
template <int D>
__global__ __launch_bounds__(kWaves * 64) void shared_merge_kernel(PoolGeom g, DecodeLaunch p) {
  const int kvh = static_cast<int>(blockIdx.x % g.kv_heads);
  const int seq = static_cast<int>(blockIdx.x / g.kv_heads);
  const int s0 = ((const ConstI32*)p.starts)[seq];
  const int slot0 = ((const ConstI32*)p.slot0)[seq];
  if (s0 <= 0 || slot0 < 0 || static_cast<int64_t>(s0) >= static_cast<int64_t>(p.max_blocks) * g.block_size)
    return;
  const int parts = ((s0 & ~15) + p.sp_chunk - 1) / p.sp_chunk + 1;
  if (slot0 > p.sp_slots - parts) return;  // flagged by the pieces
  sp_merge_rows<D>(p, seq, kvh, p.num_q_heads / g.kv_heads, slot0, parts);
}

template <int D, int KIND, int BS, int NT, bool FUSE, bool CACHED>
__global__ __launch_bounds__(kWaves * 64) __attribute__((amdgpu_waves_per_eu(2)))
void shared_prefix_kernel(PoolGeom g, DecodeLaunch p) {
  __shared__ MergeLds<2, D> sm;
  const uint32_t n_shared = static_cast<uint32_t>(p.num_items) * g.kv_heads;
  if (blockIdx.x < n_shared) {
    __shared__ FoldLds<D> fl;
    __shared__ __attribute__((aligned(16))) uint8_t new_codes[kWaves][2 * D];
    shared_body<D, KIND, BS, NT, FUSE, CACHED>(g, p, blockIdx.x, sm, fl,
                                               new_codes[__builtin_amdgcn_readfirstlane(threadIdx.x >> 6)]);
  } else {
    decode_body<D, KIND, BS, NT, kPrivate, FUSE, CACHED>(g, p, blockIdx.x - n_shared,
                                                          *reinterpret_cast<MergeLds<NT, D>*>(&sm));
  }
}

// Log-sum-exp merge of the chunk partials of one (sequence, query head):
// out = sum_c w_c o_c / sum_c w_c with w_c = l_c * 2^(m_c - max_c m_c).
// One 256-thread workgroup per row.  The chunks go in blocks of 256: thread
// t computes the weight of chunk t of the block into LDS (one exponential
// per chunk, lane-parallel loads of m and l), then wave w accumulates the
// block's chunks w, w + 4, ... with every lane taking D / 64 of the D dims
// and reading each weight as an LDS broadcast (eight chunks' loads in flight
// per wave); the waves' sums meet in LDS.
constexpr int kReduceThreads = 256;
constexpr int kReduceUnroll = 8;

// DPL consecutive fp32 values of one lane (DPL = 1 or 2).
template <int DPL>
struct LaneDims {
  float v[DPL];
};
template <int DPL>
__device__ inline LaneDims<DPL> load_dims(const float* a) {
  LaneDims<DPL> r;
  if constexpr (DPL == 2) {
    const float2 x = *reinterpret_cast<const float2*>(a);
    r.v[0] = x.x;
    r.v[1] = x.y;
  } else {
    r.v[0] = *a;
  }
  return r;
}

template <int D, int BS>
__global__ __launch_bounds__(kReduceThreads) void lse_reduce_kernel(PoolGeom g, DecodeLaunch p) {
  constexpr int DPL = D / 64;  // dims per lane
  const int row = blockIdx.x;  // seq * Hq + head
  const int seq = row / p.num_q_heads;
  const int lane = threadIdx.x & 63;
  const int w = threadIdx.x >> 6;
  int T = p.lens[seq];
  const int t_cap = p.max_blocks * BS;
  T = T < 0 ? 0 : (T > t_cap ? t_cap : T);
  const int cv = (T + p.partition_tokens - 1) / p.partition_tokens;
  const int64_t base = static_cast<int64_t>(row) * p.num_partitions;
  const float* m = p.part_m + base;
  const float* l = p.part_l + base;
  const float* o = p.part_o + base * D + DPL * lane;

  __shared__ float sm_red[4];
  __shared__ float sm_w[kReduceThreads];
  __shared__ float sm_acc[4][D];
  __shared__ float sm_den[4];
  // 1. M = max_c m_c
  float M = -__builtin_inff();
  for (int c = threadIdx.x; c < cv; c += kReduceThreads) M = fmaxf(M, m[c]);
  for (int off = 32; off > 0; off >>= 1) M = fmaxf(M, __shfl_xor(M, off));
  if (lane == 0) sm_red[w] = M;
  __syncthreads();
  M = fmaxf(fmaxf(sm_red[0], sm_red[1]), fmaxf(sm_red[2], sm_red[3]));
  // 2. blocks of 256 chunks
  float acc[DPL] = {};
  float den = 0.0f;
  for (int cb = 0; cb < cv; cb += kReduceThreads) {
    const int nb = (cv - cb) < kReduceThreads ? (cv - cb) : kReduceThreads;
    {
      const int c = cb + static_cast<int>(threadIdx.x);
      sm_w[threadIdx.x] = c < cv ? l[c] * exp2f(m[c] - M) : 0.0f;
    }
    __syncthreads();
    for (int i0 = w; i0 < nb; i0 += 4 * kReduceUnroll) {
      LaneDims<DPL> ov[kReduceUnroll];
#pragma unroll
      for (int u = 0; u < kReduceUnroll; ++u) {
        const int i = i0 + 4 * u;
        ov[u] = i < nb ? load_dims<DPL>(o + static_cast<int64_t>(cb + i) * D) : LaneDims<DPL>{};
      }
#pragma unroll
      for (int u = 0; u < kReduceUnroll; ++u) {
        const int i = i0 + 4 * u;
        const float wt = i < nb ? sm_w[i] : 0.0f;
        den += wt;
#pragma unroll
        for (int e = 0; e < DPL; ++e) acc[e] += wt * ov[u].v[e];
      }
    }
    __syncthreads();  // sm_w is rewritten by the next block
  }
#pragma unroll
  for (int e = 0; e < DPL; ++e) sm_acc[w][DPL * lane + e] = acc[e];
  if (lane == 0) sm_den[w] = den;
  __syncthreads();
  if (threadIdx.x < D) {
    const int d = threadIdx.x;
    const float num = (sm_acc[0][d] + sm_acc[1][d]) + (sm_acc[2][d] + sm_acc[3][d]);
    const float dd = (sm_den[0] + sm_den[1]) + (sm_den[2] + sm_den[3]);
    _Float16* out = static_cast<_Float16*>(p.out) + static_cast<int64_t>(row) * D + d;
    *out = (_Float16)(cv > 0 ? num / dd : 0.0f);
  }
  (void)g;
}

// The same merge for at most 64 chunks, one wave per row and four rows per
// workgroup, without barriers: lane c takes chunk c's (m, l) and the weight
// w_c = l_c * 2^(m_c - max m); the weights reach every lane by readlane while
// each lane accumulates D / 64 of the D dims over all chunks.  All loads of a
// row are issued before any is used, so a row costs about one memory round
// trip (the 256-thread kernel above needs two, with barriers).
constexpr int kReduceSmallChunks = 64;

template <int D, int BS>
__global__ __launch_bounds__(kReduceThreads) void lse_reduce_small_kernel(PoolGeom g, DecodeLaunch p) {
  constexpr int DPL = D / 64;  // dims per lane
  const int lane = threadIdx.x & 63;
  const int64_t row = static_cast<int64_t>(blockIdx.x) * 4 + (threadIdx.x >> 6);  // seq * Hq + head
  if (row >= static_cast<int64_t>(p.num_seqs) * p.num_q_heads) return;
  const int seq = static_cast<int>(row / p.num_q_heads);
  int T = p.lens[seq];
  const int t_cap = p.max_blocks * BS;
  T = T < 0 ? 0 : (T > t_cap ? t_cap : T);
  const int cv = (T + p.partition_tokens - 1) / p.partition_tokens;  // <= num_partitions <= 64
  const int64_t base = row * p.num_partitions;
  const float* o = p.part_o + base * D + DPL * lane;
  const bool mine = lane < cv;
  const float mc = mine ? p.part_m[base + lane] : -__builtin_inff();
  const float lc = mine ? p.part_l[base + lane] : 0.0f;
  LaneDims<DPL> ov[kReduceSmallChunks / 4];
  float acc[DPL] = {};
  float den = 0.0f;
  float M = mc;
  for (int off = 32; off > 0; off >>= 1) M = fmaxf(M, __shfl_xor(M, off));
  const float wc = mine ? lc * exp2f(mc - M) : 0.0f;
  for (int c0 = 0; c0 < cv; c0 += kReduceSmallChunks / 4) {
#pragma unroll
    for (int u = 0; u < kReduceSmallChunks / 4; ++u) {
      const int c = c0 + u;
      ov[u] = c < cv ? load_dims<DPL>(o + static_cast<int64_t>(c) * D) : LaneDims<DPL>{};
    }
#pragma unroll
    for (int u = 0; u < kReduceSmallChunks / 4; ++u) {
      const int c = c0 + u;
      const float w = __builtin_bit_cast(float, __builtin_amdgcn_readlane(__builtin_bit_cast(int, wc), c & 63));
      const float wu = c < cv ? w : 0.0f;
      den += wu;
#pragma unroll
      for (int e = 0; e < DPL; ++e) acc[e] += wu * ov[u].v[e];
    }
  }
  _Float16* out = static_cast<_Float16*>(p.out) + row * D + DPL * lane;
#pragma unroll
  for (int e = 0; e < DPL; ++e) out[e] = (_Float16)(cv > 0 ? acc[e] / den : 0.0f);
  (void)g;
}

// Kernels are launched with hipExtLaunchKernel (launch_kernel): its start/stop
// events (null when not timing) are stamped by the dispatch itself, so timing a
// launch adds no barrier packets to the stream.
template <int D, int KIND, int BS, int NT, bool FUSE, bool CACHED>
hipError_t launch_decode_nt(const PoolGeom& g, const DecodeLaunch& d, hipStream_t s, hipEvent_t t0,
                            hipEvent_t t1) {
  const dim3 block(kWaves * 64);
  const int64_t units = static_cast<int64_t>(d.num_seqs) * g.kv_heads;
  switch (d.mode) {
    case kSingle:
      return launch_kernel(decode_kernel<D, KIND, BS, NT, kSingle, FUSE, CACHED>, dim3(static_cast<unsigned>(units)),
                           block, s, t0, t1, g, d);
    case kSplit4:
      return launch_kernel(decode_kernel<D, KIND, BS, NT, kSplit4, FUSE, CACHED>,
                           dim3(static_cast<unsigned>(units * d.waves_per_unit)), block, s, t0, t1, g, d);
    case kSplit1:
      return launch_kernel(decode_kernel<D, KIND, BS, NT, kSplit1, FUSE, CACHED>,
                           dim3(static_cast<unsigned>((units * d.waves_per_unit + kWaves - 1) / kWaves)), block,
                           s, t0, t1, g, d);
    default:
      return hipErrorInvalidValue;
  }
}

template <int D, int KIND, int BS, bool CACHED>
hipError_t launch_decode_loads(const PoolGeom& g, const DecodeLaunch& d, int nt, hipStream_t s,
                               hipEvent_t t0, hipEvent_t t1) {
  if (d.new_slots)
    return nt == 1 ? launch_decode_nt<D, KIND, BS, 1, true, CACHED>(g, d, s, t0, t1)
                   : launch_decode_nt<D, KIND, BS, 2, true, CACHED>(g, d, s, t0, t1);
  return nt == 1 ? launch_decode_nt<D, KIND, BS, 1, false, CACHED>(g, d, s, t0, t1)
                 : launch_decode_nt<D, KIND, BS, 2, false, CACHED>(g, d, s, t0, t1);
}

template <int D, int KIND, int BS>
hipError_t launch_decode_bs(const PoolGeom& g, const DecodeLaunch& d, int nt, hipStream_t s,
                            hipEvent_t t0, hipEvent_t t1) {
  return d.cached_loads ? launch_decode_loads<D, KIND, BS, true>(g, d, nt, s, t0, t1)
                        : launch_decode_loads<D, KIND, BS, false>(g, d, nt, s, t0, t1);
}

// Decode launch of one (head_dim, element kind): every block size, column
// tile count, schedule and fused / plain form.
template <int D, int KIND>
hipError_t launch_decode_kd(const PoolGeom& g, const DecodeLaunch& d, int nt, hipStream_t s, hipEvent_t t0,
                            hipEvent_t t1) {
  switch (g.block_size) {
    case 8: return launch_decode_bs<D, KIND, 8>(g, d, nt, s, t0, t1);
    case 16: return launch_decode_bs<D, KIND, 16>(g, d, nt, s, t0, t1);
    case 32: return launch_decode_bs<D, KIND, 32>(g, d, nt, s, t0, t1);
    default: return hipErrorInvalidValue;
  }
}

// Multi-token launch of one (head_dim, element kind).
template <int D, int KIND>
hipError_t launch_multi_token_kd(const PoolGeom& g, const DecodeLaunch& d, const dim3& grid, hipStream_t s,
                                 hipEvent_t t0, hipEvent_t t1) {
  const dim3 block(kWaves * 64);
  switch (g.block_size) {
    case 8: return launch_kernel(multi_token_kernel<D, KIND, 8>, grid, block, s, t0, t1, g, d);
    case 16: return launch_kernel(multi_token_kernel<D, KIND, 16>, grid, block, s, t0, t1, g, d);
    case 32: return launch_kernel(multi_token_kernel<D, KIND, 32>, grid, block, s, t0, t1, g, d);
    default: return hipErrorInvalidValue;
  }
}

// Shared-prefix launch of one (head_dim, element kind): grid = the shared
// items' workgroups, then one per (sequence, KV head).
template <int D, int KIND, int BS, bool FUSE, bool CACHED>
hipError_t launch_shared_prefix_f(const PoolGeom& g, const DecodeLaunch& d, int nt, hipStream_t s, hipEvent_t t0,
                                  hipEvent_t t1) {
  const dim3 grid(static_cast<unsigned>((static_cast<int64_t>(d.num_items) + d.sp_private) * g.kv_heads));
  const dim3 block(kWaves * 64);
  const bool merge = d.sp_slots > 0;  // some group's pieces wrote partials
  hipError_t e =
      nt == 1 ? launch_kernel(shared_prefix_kernel<D, KIND, BS, 1, FUSE, CACHED>, grid, block, s, t0,
                              merge ? nullptr : t1, g, d)
              : launch_kernel(shared_prefix_kernel<D, KIND, BS, 2, FUSE, CACHED>, grid, block, s, t0,
                              merge ? nullptr : t1, g, d);
  if (e != hipSuccess || !merge) return e;
  const dim3 mgrid(static_cast<unsigned>(static_cast<int64_t>(d.num_seqs) * g.kv_heads));
  return launch_kernel(shared_merge_kernel<D>, mgrid, block, s, nullptr, t1, g, d);
}

template <int D, int KIND, int BS>
hipError_t launch_shared_prefix_bs(const PoolGeom& g, const DecodeLaunch& d, int nt, hipStream_t s, hipEvent_t t0,
                                   hipEvent_t t1) {
  if (d.new_slots)
    return d.cached_loads ? launch_shared_prefix_f<D, KIND, BS, true, true>(g, d, nt, s, t0, t1)
                          : launch_shared_prefix_f<D, KIND, BS, true, false>(g, d, nt, s, t0, t1);
  return d.cached_loads ? launch_shared_prefix_f<D, KIND, BS, false, true>(g, d, nt, s, t0, t1)
                        : launch_shared_prefix_f<D, KIND, BS, false, false>(g, d, nt, s, t0, t1);
}

template <int D, int KIND>
hipError_t launch_shared_prefix_kd(const PoolGeom& g, const DecodeLaunch& d, int nt, hipStream_t s, hipEvent_t t0,
                                   hipEvent_t t1) {
  switch (g.block_size) {
    case 8: return launch_shared_prefix_bs<D, KIND, 8>(g, d, nt, s, t0, t1);
    case 16: return launch_shared_prefix_bs<D, KIND, 16>(g, d, nt, s, t0, t1);
    case 32: return launch_shared_prefix_bs<D, KIND, 32>(g, d, nt, s, t0, t1);
    default: return hipErrorInvalidValue;
  }
}

template <int D>
hipError_t launch_lse_reduce_d(const PoolGeom& g, const DecodeLaunch& d, hipStream_t s, hipEvent_t t0,
                               hipEvent_t t1) {
  const int64_t rows = static_cast<int64_t>(d.num_seqs) * d.num_q_heads;
  if (d.num_partitions <= kReduceSmallChunks) {
    const dim3 grid4(static_cast<unsigned>((rows + 3) / 4));
    switch (g.block_size) {
      case 8: return launch_kernel(lse_reduce_small_kernel<D, 8>, grid4, dim3(kReduceThreads), s, t0, t1, g, d);
      case 16: return launch_kernel(lse_reduce_small_kernel<D, 16>, grid4, dim3(kReduceThreads), s, t0, t1, g, d);
      case 32: return launch_kernel(lse_reduce_small_kernel<D, 32>, grid4, dim3(kReduceThreads), s, t0, t1, g, d);
      default: return hipErrorInvalidValue;
    }
  }
  const dim3 grid(static_cast<unsigned>(rows));
  switch (g.block_size) {
    case 8: return launch_kernel(lse_reduce_kernel<D, 8>, grid, dim3(kReduceThreads), s, t0, t1, g, d);
    case 16: return launch_kernel(lse_reduce_kernel<D, 16>, grid, dim3(kReduceThreads), s, t0, t1, g, d);
    case 32: return launch_kernel(lse_reduce_kernel<D, 32>, grid, dim3(kReduceThreads), s, t0, t1, g, d);
    default: return hipErrorInvalidValue;
  }
}

}  // namespace dk
}  // namespace pa
