// Stand-ins for the device side of libyarnattn.so, for a host-only build of
// the C ABI (api.cpp, freqs.cpp, decode_plan.cpp) under AddressSanitizer and
// UndefinedBehaviorSanitizer.  Every kernel launch and HIP runtime call
// reports "no device", so a call that passes validation and planning comes
// back as YR_ERR_HIP; the balanced decode split plans for 256 compute units.
#include <hip/hip_runtime.h>

#include "yr_internal.h"

namespace yr {
hipError_t launch_rope(const RopeArgs &, hipStream_t) { return hipErrorNoDevice; }
hipError_t launch_prefill_f32(const PrefillArgs &, hipStream_t) { return hipErrorNoDevice; }
hipError_t launch_prefill_bf16(const PrefillArgs &, hipStream_t) { return hipErrorNoDevice; }
hipError_t launch_decode(const DecodeArgs &, hipStream_t) { return hipErrorNoDevice; }
int decode_stream_wgs(hipStream_t) { return 256; }
hipError_t decode_fixed_scratch(hipStream_t, void **ptr) {
  *ptr = nullptr;
  return hipErrorNoDevice;
}
}  // namespace yr

extern "C" {
const char *hipGetErrorString(hipError_t) { return "no device (host-only build)"; }
hipError_t hipMemcpyAsync(void *, const void *, size_t, hipMemcpyKind, hipStream_t) {
  return hipErrorNoDevice;
}
hipError_t hipStreamSynchronize(hipStream_t) { return hipErrorNoDevice; }
}
