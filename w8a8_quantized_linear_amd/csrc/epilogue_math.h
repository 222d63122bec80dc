// Device-side arithmetic shared by the GEMM epilogues, the single-launch
// short-input kernel and the stand-alone SwiGLU kernel (no state; header-only):
// bf16 decode / round-to-nearest-even and the SiLU of the paired gate/up
// epilogue ("Loading CLEF INT8" page: fuse_mlp, gate/up packed into one weight).
#pragma once

#include <hip/hip_runtime.h>
#include <cstdint>

namespace w8a8 {

// Two fp32 values -> two bf16, round to nearest even, low half first.  The
// kernels run with fp32 denormals preserved and round-to-nearest-even, so the
// conversion gives the bits of rounding the exact fp32 value for every non-NaN
// input; gfx950 converts the pair in one instruction.
typedef __bf16 bf16x2_t __attribute__((ext_vector_type(2)));

__device__ __forceinline__ uint32_t bf16x2_rne(float lo, float hi) {
  const bf16x2_t v = {(__bf16)lo, (__bf16)hi};
  return __builtin_bit_cast(uint32_t, v);
}

// Four bf16 values (two 32-bit words) -> fp32.
__device__ __forceinline__ void bf16x4(uint2 b, float* f) {
  f[0] = __uint_as_float(b.x << 16);
  f[1] = __uint_as_float(b.x & 0xffff0000u);
  f[2] = __uint_as_float(b.y << 16);
  f[3] = __uint_as_float(b.y & 0xffff0000u);
}

// silu(g) = g * sigmoid(g), sigmoid(g) = (g >= 0 ? 1 : e) / (1 + e) with
// e = exp(-|g|) in (0, 1] (no overflow).  e comes from the hardware exp2 and the
// quotient from the hardware reciprocal: a few fp32 ulps in all, far below the
// bf16 rounding that follows, at a fraction of the instructions of expf and an
// IEEE division (an epilogue with one wave per SIMD is instruction bound).  The
// hardware exp2 flushes subnormal results, so it is taken of the exponent plus
// 64 and scaled back by an exact multiply by 2^-64: very negative gates (down
// to about -131) keep their tiny, possibly subnormal, e, and g * e * u keeps its
// value instead of becoming -0.
__device__ __forceinline__ float silu_f32(float g) {
  const float e = __builtin_amdgcn_exp2f(__builtin_fmaf(-fabsf(g), 1.44269504088896341f, 64.0f)) * 0x1p-64f;
  return g * ((g >= 0.0f ? 1.0f : e) * __builtin_amdgcn_rcpf(1.0f + e));
}

}  // namespace w8a8
