// Measurement aid, not a step of the W8A8 path: the HBM rate a kernel with the
// quantizer's traffic and none of its arithmetic sustains -- the achievable
// streaming ceiling the quantizer is set against (the nominal 8 TB/s is not
// reached by any streaming kernel on this chip).
//
// Kind 0 reads bf16 elements and writes one byte per element (the high byte of
// each bf16: 2 bytes in, 1 byte out, the quantizer's ratio); kind 1 copies
// (2 bytes in, 2 bytes out).  Each thread owns kPieces 16-byte input pieces,
// issues all their loads before any store (as the quantizer issues a row's loads
// before its arithmetic), and consecutive threads take consecutive pieces, so
// every wave instruction reads one contiguous kilobyte.
#include <hip/hip_runtime.h>
#include <cstdint>

namespace {

constexpr int kThreads = 256;
constexpr int kPieces = 4;

typedef unsigned u32x4 __attribute__((ext_vector_type(4)));
typedef unsigned u32x2 __attribute__((ext_vector_type(2)));

template <int KIND>
__global__ void __launch_bounds__(kThreads) stream_kernel(const u32x4* __restrict__ x, void* __restrict__ y,
                                                          int64_t n16) {
  const int64_t base = (int64_t)blockIdx.x * kPieces * kThreads + threadIdx.x;
  u32x4 v[kPieces];
#pragma unroll
  for (int p = 0; p < kPieces; ++p) {
    const int64_t i = base + (int64_t)p * kThreads;
    v[p] = i < n16 ? x[i] : u32x4{0, 0, 0, 0};
  }
#pragma unroll
  for (int p = 0; p < kPieces; ++p) {
    const int64_t i = base + (int64_t)p * kThreads;
    if (i >= n16) continue;
    if constexpr (KIND == 0) {
      // v_perm_b32 bytes 0-3 come from the second operand, 4-7 from the first:
      // [b1, b3] of each word are the high bytes of its two bf16 values
      const unsigned lo = __builtin_amdgcn_perm(v[p].y, v[p].x, 0x07050301u);
      const unsigned hi = __builtin_amdgcn_perm(v[p].w, v[p].z, 0x07050301u);
      static_cast<u32x2*>(y)[i] = u32x2{lo, hi};
    } else {
      static_cast<u32x4*>(y)[i] = v[p];
    }
  }
}

}  // namespace

// x: n16 16-byte pieces (8 bf16 each) on the device; y: n16 * 8 bytes (kind 0) or
// n16 * 16 bytes (kind 1).  Returns 0, or -1 on a bad argument / launch failure.
extern "C" int w8a8_probe_stream(int kind, const void* x, void* y, int64_t n16, hipStream_t stream) {
  if (!x || !y || n16 <= 0 || (kind != 0 && kind != 1)) return -1;
  const int64_t per_block = (int64_t)kPieces * kThreads;
  const int64_t blocks = (n16 + per_block - 1) / per_block;
  if (blocks > 0x7fffffff) return -1;
  const u32x4* xv = static_cast<const u32x4*>(x);
  if (kind == 0)
    hipLaunchKernelGGL(stream_kernel<0>, dim3((unsigned)blocks), dim3(kThreads), 0, stream, xv, y, n16);
  else
    hipLaunchKernelGGL(stream_kernel<1>, dim3((unsigned)blocks), dim3(kThreads), 0, stream, xv, y, n16);
  return hipGetLastError() == hipSuccess ? 0 : -1;
}
