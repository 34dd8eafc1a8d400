// Host-only stand-ins for the kernel launchers and the one HIP runtime call the C-ABI layer
// makes, so that ra_api.cpp can be built and run on a machine without a GPU under the address,
// undefined-behaviour and thread sanitizers. Every launcher reports that no device is present.
#include "../../ring_sequence_parallelism_ra_amd/csrc/ra_internal.h"

extern "C" const char* hipGetErrorString(hipError_t) { return "no device (host-only build)"; }

namespace ra {
hipError_t launch_attn_bwd(const BwdArgs&, int, hipStream_t) { return hipErrorNoDevice; }
hipError_t bwd_scratch(float**) { return hipErrorNoDevice; }
hipError_t launch_attn_bf16(const AttnArgs&, int, int, hipStream_t) { return hipErrorNoDevice; }
hipError_t launch_attn_f32(const AttnArgs&, int, int, hipStream_t) { return hipErrorNoDevice; }
hipError_t launch_lse_merge(void*, float*, const void*, const float*, int64_t, int64_t, int64_t, int64_t, int, int,
                            hipStream_t) {
  return hipErrorNoDevice;
}
hipError_t launch_permute(const void* const*, void* const*, int, int64_t, int64_t, int64_t, int64_t, int64_t, int, int,
                          int, hipStream_t) {
  return hipErrorNoDevice;
}
hipError_t launch_debug_positions(Pos, int64_t, int64_t*, hipStream_t) { return hipErrorNoDevice; }
hipError_t launch_debug_mask(Pos, Pos, int64_t, int64_t, uint8_t*, hipStream_t) { return hipErrorNoDevice; }
}  // namespace ra
