// Host-only stand-ins for the library's kernel launchers, so that the C ABI's
// argument validation (csrc/api.cpp) can be built with g++ under AddressSanitizer
// and UndefinedBehaviorSanitizer on a machine without a GPU.  Every validation path
// returns before a launcher would be called (the device check fails without a
// gfx950 device); if one is reached anyway the stub reports an error.
#include "internal.h"

namespace w8a8 {

hipError_t launch_quantize(const uint16_t*, int64_t, int64_t, int, bool, bool, void*, float*, hipStream_t) {
  return hipErrorInvalidValue;
}
hipError_t launch_gemm(Epi, bool, bool, bool, const void*, const float*, const void*, const float*,
                       const uint16_t*, void*, int64_t, int64_t, int64_t, hipStream_t) {
  return hipErrorInvalidValue;
}
hipError_t launch_swiglu(const uint16_t*, const uint16_t*, int64_t, uint16_t*, int64_t, int64_t, hipStream_t) {
  return hipErrorInvalidValue;
}
bool short_path_fits(int64_t, int64_t, int64_t, Epi) { return false; }
hipError_t launch_linear_short(Epi, const uint16_t*, const void*, bool, const float*, const uint16_t*, uint16_t*,
                               int64_t, int64_t, int64_t, int, void*, float*, hipStream_t) {
  return hipErrorInvalidValue;
}
hipError_t launch_pack_rows(const void*, int64_t, int64_t, void*, hipStream_t) { return hipErrorInvalidValue; }

}  // namespace w8a8
