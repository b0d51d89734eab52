// One (element kind, head_dim) of the decode and multi-token kernels:
// compiled once per pair (the build passes PA_INST_KIND and PA_INST_D), so
// that the instantiations build in parallel.
#include "decode_engine.hpp"

#if !defined(PA_INST_KIND) || !defined(PA_INST_D)
#error "build with -DPA_INST_KIND=<0|1|2> -DPA_INST_D=<64|128>"
#endif

namespace pa {
namespace dk {

template hipError_t launch_decode_kd<PA_INST_D, PA_INST_KIND>(const PoolGeom&, const DecodeLaunch&, int,
                                                              hipStream_t, hipEvent_t, hipEvent_t);
template hipError_t launch_multi_token_kd<PA_INST_D, PA_INST_KIND>(const PoolGeom&, const DecodeLaunch&,
                                                                   const dim3&, hipStream_t, hipEvent_t,
                                                                   hipEvent_t);
template hipError_t launch_shared_prefix_kd<PA_INST_D, PA_INST_KIND>(const PoolGeom&, const DecodeLaunch&, int,
                                                                     hipStream_t, hipEvent_t, hipEvent_t);

}  // namespace dk
}  // namespace pa
