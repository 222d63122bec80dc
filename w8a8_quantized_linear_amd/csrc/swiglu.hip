// SwiGLU of separately projected gate and up values, for the unfused gate/up
// path ("Loading CLEF INT8" page: fuse_mlp=False disables the paired gate/up
// epilogue, so gate and up are two linears followed by their combination).
//
// What it computes: y[m][n] = bf16(silu(g) * u) with g = gate[m][n] and
// u = up[m][n] the bf16 outputs of the two projections, evaluated in fp32 with
// the same SiLU as the fused epilogue (silu_f32: sigmoid(g) = (g >= 0 ? 1 : e) /
// (1 + e) with e = exp(-|g|), which never overflows) and one
// round-to-nearest-even to bf16.
//
// Design: HBM bound (4 bytes read, 2 written per element).  One thread per 8
// consecutive elements of a row: two 16-byte loads, one 16-byte store; a wave
// covers 512 contiguous output elements.  gate and up rows are `ld` elements
// apart (the two halves of one [M, 2N] projection, or two separate [M, N]
// tensors with ld = N).
#include "epilogue_math.h"
#include "internal.h"

namespace w8a8 {
namespace {

typedef unsigned u32x4 __attribute__((ext_vector_type(4)));

__device__ __forceinline__ uint32_t swiglu_pair(uint32_t gw, uint32_t uw) {
  const float g0 = __uint_as_float(gw << 16), g1 = __uint_as_float(gw & 0xffff0000u);
  const float u0 = __uint_as_float(uw << 16), u1 = __uint_as_float(uw & 0xffff0000u);
  const float y0 = silu_f32(g0) * u0;
  const float y1 = silu_f32(g1) * u1;
  return bf16x2_rne(y0, y1);
}

__global__ void __launch_bounds__(256)
swiglu_bf16_kernel(const uint16_t* __restrict__ g, const uint16_t* __restrict__ u, int64_t ld,
                   uint16_t* __restrict__ y, int64_t N, int64_t chunks) {
  const int64_t j = (int64_t)blockIdx.x * 256 + threadIdx.x;
  if (j >= chunks) return;
  const int64_t per_row = N / 8;
  const int64_t m = j / per_row, c = (j % per_row) * 8;
  const u32x4 gv = __builtin_nontemporal_load(reinterpret_cast<const u32x4*>(g + m * ld + c));
  const u32x4 uv = __builtin_nontemporal_load(reinterpret_cast<const u32x4*>(u + m * ld + c));
  u32x4 out;
#pragma unroll
  for (int i = 0; i < 4; ++i) out[i] = swiglu_pair(gv[i], uv[i]);
  *reinterpret_cast<u32x4*>(y + m * N + c) = out;
}

}  // namespace

hipError_t launch_swiglu(const uint16_t* g, const uint16_t* u, int64_t ld, uint16_t* y, int64_t M,
                         int64_t N, hipStream_t stream) {
  const int64_t chunks = M * (N / 8);
  const int64_t blocks = (chunks + 255) / 256;
  if (blocks > 0x7fffffff) return hipErrorInvalidValue;
  hipLaunchKernelGGL(swiglu_bf16_kernel, dim3((unsigned)blocks), dim3(256), 0, stream, g, u, ld, y, N,
                     chunks);
  return hipGetLastError();
}

}  // namespace w8a8
