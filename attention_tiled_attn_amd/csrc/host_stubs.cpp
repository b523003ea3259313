// host_stubs.cpp - stand-ins for the kernels' launch functions and the few HIP
// runtime calls of api.cpp, for the sanitizer build of the C ABI only
// (build.py --sanitize): api.cpp compiled by a host compiler with address
// and undefined-behaviour sanitizers, linked with these instead of the device
// code and the HIP runtime. Every stand-in fails, so a call that passed the
// argument checks returns FLEXATTN_ERR_HIP rather than touching memory; the
// CPU tests expect every fake-pointer call to stop earlier.
#include <hip/hip_runtime_api.h>

#include "launch.h"

namespace fa {

hipError_t launch_attn_fwd(const FwdLaunch&, hipStream_t) { return hipErrorNoDevice; }
hipError_t launch_attn_decode(const FwdLaunch&, hipStream_t) { return hipErrorNoDevice; }
hipError_t launch_attn_fwd_pp(const FwdLaunch&, hipStream_t) { return hipErrorNoDevice; }
hipError_t launch_attn_bwd(const BwdLaunch&, hipStream_t) { return hipErrorNoDevice; }
hipError_t launch_block_mask(const MaskLaunch&, hipStream_t) { return hipErrorNoDevice; }
hipError_t static_scratch(int, void**) { return hipErrorNoDevice; }

}  // namespace fa

extern "C" {

hipError_t hipGetDevice(int* device) {
  if (device) *device = 0;
  return hipErrorNoDevice;
}
hipError_t hipStreamGetDevice(hipStream_t, hipDevice_t* device) {
  if (device) *device = 0;
  return hipErrorNoDevice;
}
const char* hipGetErrorString(hipError_t) { return "no device (sanitizer build)"; }

}  // extern "C"
