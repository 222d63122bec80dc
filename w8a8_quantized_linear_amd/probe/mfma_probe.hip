// Measurement aid, not a step of the W8A8 path: the rate the matrix cores sustain
// with operands in registers and no memory traffic -- the ceiling the GEMM is
// measured against at the clock the chip actually holds under load.
//
// Each wave runs `iters` rounds of four independent 32x32 MFMAs (int8 32x32x32,
// or bf16 32x32x16 -- the instruction the E4M3FN GEMM runs on), alternating
// between two operand sets for each operand so that the multipliers' inputs
// change from one instruction to the next, as they do in a GEMM.  The operands
// are fixed patterns of the lane index.  Every lane stores the sum of its 64
// accumulator values (int32, wrapping), so the result can be checked in closed
// form: over a wave, chain c adds iters * sum_{h,t} (sum_l a_{c%2}(l, t)) *
// (sum_l b_{c/2}(l, t)) with l over the 32 lanes of half h -- whatever the
// hardware's row, column and k order, as long as A and B pair k by lane half and
// position, which the GEMM relies on too.
#include <hip/hip_runtime.h>
#include <cstdint>

namespace {

typedef int v4i __attribute__((ext_vector_type(4)));
typedef int v16i __attribute__((ext_vector_type(16)));
typedef float v16f __attribute__((ext_vector_type(16)));
typedef __bf16 v8bf __attribute__((ext_vector_type(8)));

// Operand patterns (the same formulas are in the probe's test).
__device__ __forceinline__ int probe_i8(int lane, int set, int t, int which) {
  return ((lane * 7 + t * 13 + set * 29 + which * 71) % 255) - 127;
}
__device__ __forceinline__ int probe_bf16(int lane, int set, int t, int which) {
  return ((lane * 3 + t * 5 + set * 7 + which * 11) % 15) - 7;
}

template <bool BF16>
__global__ void __launch_bounds__(256) mfma_probe_kernel(int64_t iters, int32_t* __restrict__ sink) {
  const int lane = threadIdx.x & 63;
  v4i a[2], b[2];
#pragma unroll
  for (int r = 0; r < 2; ++r)
#pragma unroll
    for (int w = 0; w < 4; ++w) {
      uint32_t wa = 0, wb = 0;
      if constexpr (BF16) {   // 2 bf16 per word: small integers, exact products and sums
#pragma unroll
        for (int h = 0; h < 2; ++h) {
          const float fa = (float)probe_bf16(lane, r, 2 * w + h, 0), fb = (float)probe_bf16(lane, r, 2 * w + h, 1);
          wa |= (__float_as_uint(fa) >> 16) << (16 * h);
          wb |= (__float_as_uint(fb) >> 16) << (16 * h);
        }
      } else {                // 4 int8 per word
#pragma unroll
        for (int k = 0; k < 4; ++k) {
          wa |= (uint32_t)(probe_i8(lane, r, 4 * w + k, 0) & 0xff) << (8 * k);
          wb |= (uint32_t)(probe_i8(lane, r, 4 * w + k, 1) & 0xff) << (8 * k);
        }
      }
      a[r][w] = (int)wa;
      b[r][w] = (int)wb;
    }
  int32_t total = 0;
  if constexpr (BF16) {
    v16f acc[4] = {v16f{}, v16f{}, v16f{}, v16f{}};
    for (int64_t i = 0; i < iters; ++i) {
#pragma unroll
      for (int c = 0; c < 4; ++c)
        acc[c] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(v8bf, a[c & 1]),
                                                         __builtin_bit_cast(v8bf, b[c >> 1]), acc[c], 0, 0, 0);
    }
    float s = 0.0f;
#pragma unroll
    for (int c = 0; c < 4; ++c)
#pragma unroll
      for (int v = 0; v < 16; ++v) s += acc[c][v];
    total = (int32_t)s;    // an integer below 2^24 for the iteration counts the test uses
  } else {
    v16i acc[4] = {v16i{}, v16i{}, v16i{}, v16i{}};
    for (int64_t i = 0; i < iters; ++i) {
#pragma unroll
      for (int c = 0; c < 4; ++c) acc[c] = __builtin_amdgcn_mfma_i32_32x32x32_i8(a[c & 1], b[c >> 1], acc[c], 0, 0, 0);
    }
#pragma unroll
    for (int c = 0; c < 4; ++c)
#pragma unroll
      for (int v = 0; v < 16; ++v) total = (int32_t)((uint32_t)total + (uint32_t)acc[c][v]);
  }
  sink[(int64_t)blockIdx.x * 256 + threadIdx.x] = total;
}

}  // namespace

// Launches `blocks` workgroups of 4 waves; each wave runs `iters` rounds of four
// independent MFMAs (kind 0: int8 32x32x32, 65,536 ops each; kind 1: bf16
// 32x32x16, 32,768 flops each) and stores each lane's accumulator sum in sink
// [blocks * 256] (int32).  Ops per launch: blocks * 4 * iters * 4 * ops each.
// Returns 0, or -1 for a bad argument (1 <= iters <= 2^40, 1 <= blocks <= 65536).
extern "C" int w8a8_probe_mfma_rate(int kind, int64_t iters, int blocks, int32_t* sink, hipStream_t stream) {
  if ((kind != 0 && kind != 1) || iters < 1 || iters > ((int64_t)1 << 40) || blocks < 1 || blocks > 65536 || !sink)
    return -1;
  if (kind == 1)
    hipLaunchKernelGGL(mfma_probe_kernel<true>, dim3(blocks), dim3(256), 0, stream, iters, sink);
  else
    hipLaunchKernelGGL(mfma_probe_kernel<false>, dim3(blocks), dim3(256), 0, stream, iters, sink);
  return hipGetLastError() == hipSuccess ? 0 : -2;
}
