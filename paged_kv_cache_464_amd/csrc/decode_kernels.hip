// Dispatch of the paged decode, multi-token and log-sum-exp reduce launches
// (gfx950) to the kernel templates of decode_engine.hpp: by head_dim (64 or
// 128) and element kind.  The decode and multi-token instantiations are
// compiled in decode_inst.hip, one object per (kind, head_dim).
#include "decode_engine.hpp"

namespace pa {
namespace dk {

#define PA_DECLARE_INST(D, KIND)                                                                              \
  extern template hipError_t launch_decode_kd<D, KIND>(const PoolGeom&, const DecodeLaunch&, int, hipStream_t, \
                                                       hipEvent_t, hipEvent_t);                                \
  extern template hipError_t launch_multi_token_kd<D, KIND>(const PoolGeom&, const DecodeLaunch&, const dim3&, \
                                                            hipStream_t, hipEvent_t, hipEvent_t);              \
  extern template hipError_t launch_shared_prefix_kd<D, KIND>(const PoolGeom&, const DecodeLaunch&, int,         \
                                                              hipStream_t, hipEvent_t, hipEvent_t);
PA_DECLARE_INST(64, kF16)
PA_DECLARE_INST(64, kF8)
PA_DECLARE_INST(64, kI8)
PA_DECLARE_INST(128, kF16)
PA_DECLARE_INST(128, kF8)
PA_DECLARE_INST(128, kI8)
#undef PA_DECLARE_INST

template <int D>
hipError_t decode_for_dim(const PoolGeom& g, const DecodeLaunch& d, int nt, hipStream_t s, hipEvent_t t0,
                          hipEvent_t t1) {
  switch (g.kind) {
    case kF16: return launch_decode_kd<D, kF16>(g, d, nt, s, t0, t1);
    case kF8: return launch_decode_kd<D, kF8>(g, d, nt, s, t0, t1);
    case kI8: return launch_decode_kd<D, kI8>(g, d, nt, s, t0, t1);
    default: return hipErrorInvalidValue;
  }
}

template <int D>
hipError_t multi_token_for_dim(const PoolGeom& g, const DecodeLaunch& d, const dim3& grid, hipStream_t s,
                               hipEvent_t t0, hipEvent_t t1) {
  switch (g.kind) {
    case kF16: return launch_multi_token_kd<D, kF16>(g, d, grid, s, t0, t1);
    case kF8: return launch_multi_token_kd<D, kF8>(g, d, grid, s, t0, t1);
    case kI8: return launch_multi_token_kd<D, kI8>(g, d, grid, s, t0, t1);
    default: return hipErrorInvalidValue;
  }
}

template <int D>
hipError_t shared_prefix_for_dim(const PoolGeom& g, const DecodeLaunch& d, int nt, hipStream_t s, hipEvent_t t0,
                                 hipEvent_t t1) {
  switch (g.kind) {
    case kF16: return launch_shared_prefix_kd<D, kF16>(g, d, nt, s, t0, t1);
    case kF8: return launch_shared_prefix_kd<D, kF8>(g, d, nt, s, t0, t1);
    case kI8: return launch_shared_prefix_kd<D, kI8>(g, d, nt, s, t0, t1);
    default: return hipErrorInvalidValue;
  }
}

}  // namespace dk

hipError_t launch_shared_prefix(const PoolGeom& g, const DecodeLaunch& d, hipStream_t s, hipEvent_t t0,
                                hipEvent_t t1) {
  const int64_t wgs = (static_cast<int64_t>(d.num_items) + d.sp_private) * g.kv_heads;
  if (wgs <= 0) return hipSuccess;
  if (!d.starts || !d.slot0 || (d.sp_private > 0 && !d.order) || d.sp_private < 0 ||
      d.sp_private > d.num_seqs || (d.num_items > 0 && (!d.work || !d.members)) ||
      d.num_items < 0 || wgs > 0x7FFFFFFF || d.sp_chunk < 64 || d.sp_chunk % 64 != 0)
    return hipErrorInvalidValue;
  const int nt = d.num_q_heads / g.kv_heads > 16 ? 2 : 1;
  switch (g.head_dim) {
    case 64: return dk::shared_prefix_for_dim<64>(g, d, nt, s, t0, t1);
    case 128: return dk::shared_prefix_for_dim<128>(g, d, nt, s, t0, t1);
    default: return hipErrorInvalidValue;
  }
}

hipError_t launch_decode(const PoolGeom& g, const DecodeLaunch& d, hipStream_t s, hipEvent_t t0,
                         hipEvent_t t1) {
  const int group = d.num_q_heads / g.kv_heads;
  const int nt = group > 16 ? 2 : 1;
  if (static_cast<int64_t>(d.num_seqs) * g.kv_heads <= 0) return hipSuccess;
  if (d.mode != dk::kSingle && d.mode != dk::kPrivate) {
    // The split schedules need whole steps per chunk (and per wave quarter).
    const int quantum = d.mode == dk::kSplit4 ? 64 : 16;
    if (d.waves_per_unit < 1 || d.chunks_per_wave < 1 || d.partition_tokens < quantum ||
        d.partition_tokens % quantum != 0)
      return hipErrorInvalidValue;
  }
  switch (g.head_dim) {
    case 64: return dk::decode_for_dim<64>(g, d, nt, s, t0, t1);
    case 128: return dk::decode_for_dim<128>(g, d, nt, s, t0, t1);
    default: return hipErrorInvalidValue;
  }
}

hipError_t launch_multi_token(const PoolGeom& g, const DecodeLaunch& d, hipStream_t s, hipEvent_t t0,
                              hipEvent_t t1) {
  const int64_t wgs = static_cast<int64_t>(d.num_items) * g.kv_heads;
  if (wgs <= 0) return hipSuccess;
  if (!d.work || wgs > 0x7FFFFFFF) return hipErrorInvalidValue;
  const dim3 grid(static_cast<unsigned>(wgs));
  switch (g.head_dim) {
    case 64: return dk::multi_token_for_dim<64>(g, d, grid, s, t0, t1);
    case 128: return dk::multi_token_for_dim<128>(g, d, grid, s, t0, t1);
    default: return hipErrorInvalidValue;
  }
}

hipError_t launch_lse_reduce(const PoolGeom& g, const DecodeLaunch& d, hipStream_t s, hipEvent_t t0,
                             hipEvent_t t1) {
  const int64_t rows = static_cast<int64_t>(d.num_seqs) * d.num_q_heads;
  if (rows <= 0) return hipSuccess;
  switch (g.head_dim) {
    case 64: return dk::launch_lse_reduce_d<64>(g, d, s, t0, t1);
    case 128: return dk::launch_lse_reduce_d<128>(g, d, s, t0, t1);
    default: return hipErrorInvalidValue;
  }
}

}  // namespace pa
