// Host stubs for the sanitizer build of libcpattn's C-ABI layer: the HIP
// runtime calls it makes and the kernel launchers it enqueues.  Launchers do
// nothing and report success, so every host-side check and the ring driver's
// argument arithmetic run under AddressSanitizer / UBSan without a GPU.
#include "hip/hip_runtime.h"
#include "cpa_internal.h"

const char* hipGetErrorString(hipError_t) { return "stub"; }
hipError_t hipGetDevice(int* dev) { *dev = 0; return hipSuccess; }
hipError_t hipSetDevice(int) { return hipSuccess; }
hipError_t hipStreamGetDevice(hipStream_t, int* dev) { *dev = 0; return hipSuccess; }
hipError_t hipGetSymbolAddress(void** ptr, const void* symbol) {
  *ptr = const_cast<void*>(symbol);
  return hipSuccess;
}

namespace cpa {
hipError_t launch_partial_mfma(const void*, const void*, const void*, const int64_t*,
                               const int64_t*, float*, float*, int, int64_t, int64_t, int, bool,
                               float, hipStream_t) { return hipSuccess; }
hipError_t launch_ring_mfma(const void*, const void*, const void*, const int64_t*, const int64_t*,
                            float*, float*, int, int64_t, int, int, int, bool, float,
                            hipStream_t) { return hipSuccess; }
hipError_t launch_share_mfma(const void*, const void*, const void*, float*, float*, int, int64_t,
                             int, int, int, int, bool, float, bool, hipStream_t) { return hipSuccess; }
hipError_t launch_partial_rowwise(const void*, const void*, const void*, bool, const int64_t*,
                                  const int64_t*, float*, float*, int, int64_t, int64_t, int, bool,
                                  float, hipStream_t) { return hipSuccess; }
hipError_t launch_merge(float*, float*, const float*, const float*, int64_t, int, hipStream_t) {
  return hipSuccess;
}
hipError_t launch_permute(const void*, void*, int64_t, int64_t, int64_t, const int64_t*, int, int,
                          int, bool, hipStream_t) { return hipSuccess; }
hipError_t launch_check_offsets(const int64_t*, int64_t, int64_t, int64_t*, hipStream_t) {
  return hipSuccess;
}
hipError_t launch_rope(const void*, void*, bool, int64_t, int64_t, int64_t, int64_t, int,
                       const int64_t*, bool, double, bool, hipStream_t) { return hipSuccess; }
hipError_t launch_bwd_delta(const float*, const void*, bool, int64_t, int, float*, hipStream_t) {
  return hipSuccess;
}
hipError_t launch_bwd_mfma(const void*, const void*, const void*, const void*, const float*,
                           const float*, const int64_t*, const int64_t*, float*, float*, float*,
                           int, int64_t, int64_t, int64_t, int64_t, int, int, int, bool, float,
                           bool, hipStream_t) { return hipSuccess; }
hipError_t launch_bwd_delta_share(const float*, const void*, int, int64_t, int, int, int, float*,
                                  hipStream_t) { return hipSuccess; }
hipError_t launch_bwd_share_mfma(const void*, const void*, const void*, const void*, const float*,
                                 const float*, float*, float*, float*, int, int64_t, int, int, int,
                                 bool, float, hipStream_t) { return hipSuccess; }
hipError_t launch_bwd_rowwise(const void*, const void*, const void*, const void*, bool,
                              const float*, const float*, const int64_t*, const int64_t*, float*,
                              float*, float*, int, int64_t, int64_t, int, bool, float, bool,
                              hipStream_t) { return hipSuccess; }
}  // namespace cpa
