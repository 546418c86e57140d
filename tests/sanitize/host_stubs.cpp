// Host-only stand-ins for the sanitizer build of the C ABI: the kernel launchers and the two HIP
// runtime queries the ABI makes. No device code and no HIP runtime are linked: a call that passes
// validation reaches hipGetDeviceCount, which reports no device, and returns PF8_ENODEV; the
// launchers below are never reached, and nothing is ever launched.
#include "pf8_launch.h"

extern "C" {
hipError_t hipGetDeviceCount(int* count) {
  *count = 0;
  return hipErrorNoDevice;
}
hipError_t hipGetLastError(void) { return hipSuccess; }
}

namespace pf8 {
hipError_t launch_quant_rows(const void*, int64_t, int64_t, int64_t, void*, int64_t, float*, int64_t, hipStream_t) {
  return hipErrorInvalidDeviceFunction;
}
hipError_t launch_quant_cols(const void*, int64_t, int64_t, int64_t, void*, int64_t, float*, int64_t, hipStream_t) {
  return hipErrorInvalidDeviceFunction;
}
hipError_t launch_quant_dual(const void*, int64_t, int64_t, int64_t, void*, int64_t, float*, int64_t, void*, int64_t,
                             float*, int64_t, hipStream_t) {
  return hipErrorInvalidDeviceFunction;
}
hipError_t launch_quant_fwd(const void*, int64_t, int64_t, int64_t, void*, int64_t, float*, int64_t, void*, int64_t,
                            float*, int64_t, const void*, int64_t, int64_t, void*, int64_t, void*, int64_t, float*,
                            int64_t, hipStream_t) {
  return hipErrorInvalidDeviceFunction;
}
hipError_t launch_quant_w(const void*, int64_t, int64_t, int64_t, void*, int64_t, void*, int64_t, float*, int64_t,
                          hipStream_t) {
  return hipErrorInvalidDeviceFunction;
}
hipError_t launch_gemm(const GemmArgs&, bool, bool, hipStream_t) { return hipErrorInvalidDeviceFunction; }
hipError_t launch_gemm_bf16(const GemmArgs&, hipStream_t) { return hipErrorInvalidDeviceFunction; }
}  // namespace pf8
