// Measurement aid, not a step of the W8A8 path: the lane layout of
// v_mfma_f64_4x4x4f64, on which the quantizer's cross-quarter rotation stage
// relies (four independent 4x4x4 products per wave, one per group of lanes with
// equal bits 2-3).  Workgroup L (one wave) sets the A operand to 1 in lane L and 0
// elsewhere, B to lane + 1 in every lane, C to 0, and stores D of every lane to
// out[64 L + lane]: D is then nonzero exactly in the lanes whose (group, row)
// match lane L's A position, where it holds B of lane L's (group, k) at the
// lane's column -- which the test reads back as the A, B and D maps.
#include <hip/hip_runtime.h>
#include <cstdint>

namespace {

__global__ void __launch_bounds__(64) f64_mfma_layout_kernel(double* __restrict__ out) {
  const int L = blockIdx.x, lane = threadIdx.x;
  const double a = lane == L ? 1.0 : 0.0;
  const double b = (double)(lane + 1);
  out[L * 64 + lane] = __builtin_amdgcn_mfma_f64_4x4x4f64(a, b, 0.0, 0, 0, 0);
}

}  // namespace

// out: 64 x 64 doubles on the device.  Returns 0, or -1 on a bad argument / launch failure.
extern "C" int w8a8_probe_f64_mfma_layout(double* out, hipStream_t stream) {
  if (!out) return -1;
  hipLaunchKernelGGL(f64_mfma_layout_kernel, dim3(64), dim3(64), 0, stream, out);
  return hipGetLastError() == hipSuccess ? 0 : -1;
}
