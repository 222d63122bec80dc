// Measurement aid, not a step of the W8A8 path: the accuracy of the gfx950 matrix
// instructions on an E4M3FN x E4M3FN contraction, which decides how the library's
// FP8 GEMM multiplies (the FP8 W8A8 scheme of the "clef-flash-FP8" card,
// Quantization table, accumulates its products in fp32).
//
// C[m][n] = sum_k dec(a[m][k]) * dec(b[n][k]) for E4M3FN codes a [M, K], b [N, K]
// (row-major), written as fp32 C [M, N], by one of four instruction routes:
//   kind 0: v_mfma_f32_32x32x16_fp8_fp8, chained through its fp32 accumulator;
//   kind 1: v_mfma_scale_f32_32x32x64_f8f6f4 (E4M3 operands, unit E8M0 scales),
//           chained through its fp32 accumulator;
//   kind 2: kind 0's instruction with a zero accumulator each time, its results
//           added in fp32 by the VALU (isolates the instruction's own summation);
//   kind 3: the codes widened exactly to bf16 and multiplied on
//           v_mfma_f32_32x32x16_bf16 (the library's route).
// One wave per 32 x 32 output block, operands loaded straight from memory: slow
// and simple, for accuracy only.  The k pairing of the two operands is the same
// in every route (lane half h supplies k [8h, 8h + 8) of each 16-deep step,
// [32h, 32h + 32) of each 64-deep step), which is all a dot product needs; the
// output layout is the MFMA's (lane l: column l % 32, rows 8q + 4 (l / 32) + r in
// register 4q + r).
#include <hip/hip_runtime.h>
#include <cstdint>

namespace {

typedef float v16f __attribute__((ext_vector_type(16)));
typedef int v8i __attribute__((ext_vector_type(8)));
typedef unsigned u32x2 __attribute__((ext_vector_type(2)));
typedef __bf16 v2bf __attribute__((ext_vector_type(2)));
typedef __bf16 v4bf __attribute__((ext_vector_type(4)));
typedef __bf16 v8bf __attribute__((ext_vector_type(8)));

__device__ __forceinline__ v8bf widen8(u32x2 v) {
  const v2bf p0 = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8((int)v.x, 1.0f, false);
  const v2bf p1 = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8((int)v.x, 1.0f, true);
  const v2bf p2 = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8((int)v.y, 1.0f, false);
  const v2bf p3 = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8((int)v.y, 1.0f, true);
  const v4bf lo = __builtin_shufflevector(p0, p1, 0, 1, 2, 3);
  const v4bf hi = __builtin_shufflevector(p2, p3, 0, 1, 2, 3);
  return __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7);
}

template <int KIND>
__global__ void __launch_bounds__(64)
fp8_contraction(const uint8_t* __restrict__ a, const uint8_t* __restrict__ b, float* __restrict__ c,
                int64_t M, int64_t N, int64_t K) {
  const int lane = threadIdx.x;
  const int64_t m0 = (int64_t)blockIdx.x * 32, n0 = (int64_t)blockIdx.y * 32;
  const int r = lane & 31, h = lane >> 5;
  const uint8_t* ar = a + (m0 + r) * K;
  const uint8_t* br = b + (n0 + r) * K;
  v16f acc = {};
  if constexpr (KIND == 1) {
    for (int64_t k = 0; k < K; k += 64) {
      const v8i av = *reinterpret_cast<const v8i*>(ar + k + 32 * h);
      const v8i bv = *reinterpret_cast<const v8i*>(br + k + 32 * h);
      // B operand = rows of a (output rows), A operand = rows of b: lane l ends up
      // with output row m0 + (l % 32)
      acc = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(bv, av, acc, 0, 0, 0, 127, 0, 127);
    }
  } else {
    for (int64_t k = 0; k < K; k += 16) {
      const long av = *reinterpret_cast<const long*>(ar + k + 8 * h);
      const long bv = *reinterpret_cast<const long*>(br + k + 8 * h);
      if constexpr (KIND == 0) {
        acc = __builtin_amdgcn_mfma_f32_32x32x16_fp8_fp8(bv, av, acc, 0, 0, 0);
      } else if constexpr (KIND == 2) {
        const v16f part = __builtin_amdgcn_mfma_f32_32x32x16_fp8_fp8(bv, av, v16f{}, 0, 0, 0);
#pragma unroll
        for (int i = 0; i < 16; ++i) acc[i] += part[i];
      } else {
        const v8bf aw = widen8(__builtin_bit_cast(u32x2, av));
        const v8bf bw = widen8(__builtin_bit_cast(u32x2, bv));
        acc = __builtin_amdgcn_mfma_f32_32x32x16_bf16(bw, aw, acc, 0, 0, 0);
      }
    }
  }
  // lane l holds output row m0 + l % 32, columns n0 + 8q + 4h + (0..3) in registers 4q + (0..3)
#pragma unroll
  for (int q = 0; q < 4; ++q)
#pragma unroll
    for (int i = 0; i < 4; ++i) c[(m0 + r) * N + n0 + 8 * q + 4 * h + i] = acc[4 * q + i];
}

}  // namespace

// Returns 0, or -1 for an unsupported kind or shape (M, N multiples of 32, K of 64).
extern "C" int w8a8_probe_fp8_contraction(int kind, const uint8_t* a, const uint8_t* b, float* c, int64_t M,
                                          int64_t N, int64_t K, hipStream_t stream) {
  if (M <= 0 || N <= 0 || K <= 0 || M % 32 || N % 32 || K % 64 || M / 32 > 65535 || N / 32 > 65535) return -1;
  if (!a || !b || !c) return -1;
  const dim3 grid((unsigned)(M / 32), (unsigned)(N / 32));
  switch (kind) {
    case 0: hipLaunchKernelGGL(fp8_contraction<0>, grid, dim3(64), 0, stream, a, b, c, M, N, K); break;
    case 1: hipLaunchKernelGGL(fp8_contraction<1>, grid, dim3(64), 0, stream, a, b, c, M, N, K); break;
    case 2: hipLaunchKernelGGL(fp8_contraction<2>, grid, dim3(64), 0, stream, a, b, c, M, N, K); break;
    case 3: hipLaunchKernelGGL(fp8_contraction<3>, grid, dim3(64), 0, stream, a, b, c, M, N, K); break;
    default: return -1;
  }
  return hipGetLastError() == hipSuccess ? 0 : -2;
}
