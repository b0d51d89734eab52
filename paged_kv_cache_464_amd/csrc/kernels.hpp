// Launchers of the HIP kernels (gfx950).  All take a PoolGeom of a bound pool
// and enqueue on `stream`; they return the hipError_t of the launch.
#pragma once

#include <hip/hip_ext.h>
#include <hip/hip_runtime.h>

#include <cstdint>
#include <tuple>
#include <utility>

#include "layout.hpp"

namespace pa {

// Enqueues kernel(args...) on `stream` and returns the status of this launch
// itself (hipGetLastError would also report an error some earlier, unrelated
// call left on the thread).  t0/t1: optional events the dispatch stamps at the
// kernel's start and end.
template <class... P, class... A>
inline hipError_t launch_kernel(void (*kernel)(P...), dim3 grid, dim3 block, hipStream_t stream,
                                hipEvent_t t0, hipEvent_t t1, A&&... args) {
  std::tuple<P...> vals(std::forward<A>(args)...);
  void* ptrs[sizeof...(P) > 0 ? sizeof...(P) : 1];
  std::apply([&ptrs](auto&... v) {
    int i = 0;
    ((ptrs[i++] = static_cast<void*>(&v)), ...);
  }, vals);
  return hipExtLaunchKernel(reinterpret_cast<const void*>(kernel), grid, block, ptrs, 0, stream, t0, t1, 0);
}

constexpr uint32_t kDevBadSlot = 1u;
constexpr uint32_t kDevBadBlock = 2u;
constexpr uint32_t kDevBadLen = 4u;
constexpr uint32_t kDevBadOrder = 8u;

hipError_t launch_write_kv(const PoolGeom& g, int layer, const void* k_new, const void* v_new,
                           const int32_t* slots, int n_tokens, hipStream_t stream);
hipError_t launch_gather_kv(const PoolGeom& g, int layer, const int32_t* slots, int n_tokens,
                            void* k_out, void* v_out, hipStream_t stream);
hipError_t launch_stream_read(const void* buf, uint64_t bytes, uint32_t* sink, hipStream_t stream);
hipError_t launch_copy_blocks(const PoolGeom& g, const int32_t* src, const int32_t* dst, int n,
                              hipStream_t stream);

struct DecodeLaunch {
  int layer;
  const void* q;
  const int32_t* tables;
  const int32_t* lens;
  const int32_t* order;  // optional [S]: workgroup order of the sequences (null: 0..S-1)
  // Multi-token attention only: work items of four int32 (sequence, first
  // query token j0 of the tile, its query row, the sequence's query count),
  // one per workgroup and KV head.
  const int32_t* work;
  int num_items;
  // Optional fused scatter of each sequence's new token (null: none):
  // fp16 [S][Hkv][D] K and V of token T_i - 1, stored at new_slots[i].
  const void* k_new;
  const void* v_new;
  const int32_t* new_slots;
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
  int cached_loads;  // 1: ordinary K/V loads (blocks shared by many sequences); 0: nontemporal
  // Shared-prefix decode.  `work` holds items of four int32 (first member,
  // members, shared tokens, chunk) indexing `members` (sequence ids, group by
  // group); sequence i attends privately to tokens starts[i] .. T_i - 1.  A
  // grouped sequence's pieces (its group's shared chunks of sp_chunk tokens,
  // then its private tokens) write partials into slots slot0[i],
  // slot0[i] + 1, ... of part_m / part_l / part_o ([slot][Hq] / [slot][Hq] /
  // [slot][Hq][D], sp_slots slots), which a second launch merges into `out`.
  // A sequence in no group (starts[i] = 0) writes `out` directly.
  // Folded items (chunk -1) take a group's whole shared run and then each
  // member's own tokens in the same workgroup, writing `out` directly; the
  // private pieces are the sequences listed in `order` (sp_private of them).
  const int32_t* members;
  const int32_t* starts;
  const int32_t* slot0;
  int sp_chunk;
  int sp_slots;
  int sp_private;
};

// t0/t1: optional events stamped at the kernel's start and end (null: untimed).
hipError_t launch_decode(const PoolGeom& g, const DecodeLaunch& d, hipStream_t stream,
                         hipEvent_t t0 = nullptr, hipEvent_t t1 = nullptr);
hipError_t launch_lse_reduce(const PoolGeom& g, const DecodeLaunch& d, hipStream_t stream,
                             hipEvent_t t0 = nullptr, hipEvent_t t1 = nullptr);
// Shared-prefix decode: the shared chunks and every sequence's private
// tokens in one launch, then the merge of the grouped sequences' partials
// (d.work, d.num_items, d.members, d.starts, d.slot0, d.part_*, d.sp_chunk,
// d.sp_slots).
hipError_t launch_shared_prefix(const PoolGeom& g, const DecodeLaunch& d, hipStream_t stream,
                                hipEvent_t t0 = nullptr, hipEvent_t t1 = nullptr);
// Causal attention of several query tokens per sequence (d.work, d.num_items;
// d.q and d.out are [query rows][Hq][D]).
hipError_t launch_multi_token(const PoolGeom& g, const DecodeLaunch& d, hipStream_t stream,
                              hipEvent_t t0 = nullptr, hipEvent_t t1 = nullptr);
// Query tokens of one multi-token wave (32 (token, head) columns) and of one
// work item (a workgroup of four such waves), for a query-head group of
// `group`.
__host__ __device__ inline int multi_token_wave_tile(int group) { return group > 16 ? 1 : 32 / group; }
__host__ __device__ inline int multi_token_tile(int group) { return 4 * multi_token_wave_tile(group); }

}  // namespace pa
