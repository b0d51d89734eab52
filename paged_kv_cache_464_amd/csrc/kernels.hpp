// Launchers of the HIP kernels (gfx950).  All take a PoolGeom of a bound pool
// and enqueue on `stream`; they return the hipError_t of the launch.
#pragma once

#include <hip/hip_runtime.h>

#include <cstdint>

#include "layout.hpp"

namespace pa {

constexpr uint32_t kDevBadSlot = 1u;
constexpr uint32_t kDevBadBlock = 2u;
constexpr uint32_t kDevBadLen = 4u;

hipError_t launch_write_kv(const PoolGeom& g, int layer, const void* k_new, const void* v_new,
                           const int32_t* slots, int n_tokens, hipStream_t stream);
hipError_t launch_gather_kv(const PoolGeom& g, int layer, const int32_t* slots, int n_tokens,
                            void* k_out, void* v_out, hipStream_t stream);
hipError_t launch_copy_blocks(const PoolGeom& g, const int32_t* src, const int32_t* dst, int n,
                              hipStream_t stream);

struct DecodeLaunch {
  int layer;
  const void* q;
  const int32_t* tables;
  const int32_t* lens;
  void* out;       // fp16 [S][Hq][D] (single pass / reduce)
  float* part_m;   // [S][Hq][C]
  float* part_l;   // [S][Hq][C]
  float* part_o;   // [S][Hq][C][D]
  int num_seqs, num_q_heads, max_blocks;
  int mode;              // 0: single pass, 1: split, four waves per chunk, 2: split, one wave per run
  int partition_tokens;  // P: tokens per chunk (split modes)
  int num_partitions;    // C = ceil(max_blocks * block_size / P) (1 in a single pass)
  int chunks_per_wave;   // k: chunks in one run (split modes)
  int waves_per_unit;    // runs per (sequence, KV head) = ceil(C / k) (split modes)
  float scale;
};

// t0/t1: optional events stamped at the kernel's start and end (null: untimed).
hipError_t launch_decode(const PoolGeom& g, const DecodeLaunch& d, hipStream_t stream,
                         hipEvent_t t0 = nullptr, hipEvent_t t1 = nullptr);
hipError_t launch_lse_reduce(const PoolGeom& g, const DecodeLaunch& d, hipStream_t stream,
                             hipEvent_t t0 = nullptr, hipEvent_t t1 = nullptr);

}  // namespace pa
