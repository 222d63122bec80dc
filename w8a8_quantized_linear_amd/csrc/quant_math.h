// Device-side arithmetic of the per-row quantizer, shared by the quantizer
// kernel and the single-launch short-input path (no state; header-only).
//
// The rotation, scale and code rules follow the per-token activation quantizer
// of the ConvRot INT8 path ("CLEF Calibrated INT8 ConvRot" card, notes under the
// latency table) and the E4M3 dynamic scheme ("clef-flash-FP8" card,
// Quantization table); the kernels' headers give the readings.
#pragma once

#include <hip/hip_runtime.h>
#include <cstdint>

namespace w8a8 {
namespace qm {

typedef unsigned u32x4 __attribute__((ext_vector_type(4)));

constexpr int kEPL = 32;  // bf16 elements per lane per chunk

// fl64(2^-3.5) = fl64(sqrt(2)/2) / 8
constexpr double kInvSqrt128 = 0x1.6a09e667f3bcdp-4;

__device__ __forceinline__ float bf16lo(uint32_t w) { return __uint_as_float(w << 16); }
__device__ __forceinline__ float bf16hi(uint32_t w) { return __uint_as_float(w & 0xffff0000u); }

__device__ __forceinline__ float wave_max(float v) {
#pragma unroll
  for (int o = 32; o >= 1; o >>= 1) v = fmaxf(v, __shfl_xor(v, o, 64));
  return v;
}

// fp64 value of the lane whose quad position differs in the bits of MASK (1 or 2).
template <int MASK>
__device__ __forceinline__ double quad_xor(double v) {
  // quad_perm selectors: lane i of each quad reads lane i ^ MASK
  constexpr int ctrl = MASK == 1 ? 0xB1 : 0x4E;  // [1,0,3,2] / [2,3,0,1]
  const long long bits = __double_as_longlong(v);
  const int lo = __builtin_amdgcn_mov_dpp((int)bits, ctrl, 0xF, 0xF, false);
  const int hi = __builtin_amdgcn_mov_dpp((int)(bits >> 32), ctrl, 0xF, 0xF, false);
  return __longlong_as_double(((long long)hi << 32) | (unsigned)lo);
}

__device__ __forceinline__ uint32_t pack_i8x4(float a, float b, float c, float d) {
  uint32_t ia = (uint32_t)(int)a & 0xffu, ib = (uint32_t)(int)b & 0xffu;
  uint32_t ic = (uint32_t)(int)c & 0xffu, id = (uint32_t)(int)d & 0xffu;
  return ia | (ib << 8) | (ic << 16) | (id << 24);
}

// Code of fl32(y / s) rounded half to even, via the reciprocal r = fl32(1/s).
__device__ __forceinline__ float int8_code(float y, float s, float r) {
  const float t = y * r;
  const float k = __builtin_rintf(t);
  // |t - y/s| <= 2^-16 and |fl32(y/s) - y/s| <= 2^-18 for |y/s| < 128: only a t
  // within 2^-15 of a half-integer can round differently from the IEEE
  // quotient.  (Written so that a non-finite t, from a subnormal s, also takes
  // the exact path.)
  if (__builtin_expect(!(fabsf(fabsf(t - k) - 0.5f) >= 0x1p-14f), 0)) return __builtin_rintf(y / s);
  return k;
}

// Codes of n values, clamped to +-127: int8_code's fast path for all of them;
// the IEEE quotient for those whose t lies near a half-integer, behind one
// branch per chunk that waves almost always skip (the chunk's smallest distance
// of |t - k| from 1/2 decides; a non-finite r, from a subnormal s, sends the
// whole chunk down the exact path).  r = 0 (a zero scale's stand-in) gives zero
// codes.
template <int n>
__device__ __forceinline__ void int8_codes(const float (&y)[n], float s, float r, float (&k)[n]) {
  float dmin = 1.0f;
#pragma unroll
  for (int j = 0; j < n; ++j) {
    const float t = y[j] * r;
    k[j] = __builtin_rintf(t);
    dmin = fminf(dmin, fabsf(fabsf(t - k[j]) - 0.5f));
  }
  if (__builtin_expect(!(dmin >= 0x1p-14f) || !(fabsf(r) <= 0x1.fffffep127f), 0)) {
#pragma unroll
    for (int j = 0; j < n; ++j)
      if (!(fabsf(fabsf(y[j] * r - k[j]) - 0.5f) >= 0x1p-14f)) k[j] = __builtin_rintf(y[j] / s);
  }
#pragma unroll
  for (int j = 0; j < n; ++j) k[j] = fminf(fmaxf(k[j], -127.0f), 127.0f);
}

// Exact rotation of one 32-element chunk: the lane holds elements 32p .. 32p+31
// of a 128-block, p = lane % 4 (its position in a DPP quad whose other lanes
// hold the rest of the block).  Block sums of the bf16 values are formed in
// fp64 -- 5 butterfly stages inside the lane, the last 2 across the quad --
// then multiplied by fl64(2^-3.5) and rounded once to fp32.
__device__ __forceinline__ void rotate_chunk(const u32x4 (&raw)[4], int lane, float (&y)[kEPL]) {
  double v[kEPL];
#pragma unroll
  for (int j = 0; j < 16; ++j) {
    const uint32_t w = raw[j / 4][j % 4];
    v[2 * j] = (double)bf16lo(w);
    v[2 * j + 1] = (double)bf16hi(w);
  }
  // element index bits 0..4 live in the lane
#pragma unroll
  for (int h = 1; h < kEPL; h <<= 1) {
#pragma unroll
    for (int j = 0; j < kEPL; ++j) {
      if (!(j & h)) {
        const double a = v[j], b = v[j | h];
        v[j] = a + b;
        v[j | h] = a - b;
      }
    }
  }
  // element index bits 5, 6 are the lane's position in its quad
  // (lower lane: v + p; upper lane: p - v; both exact)
  {
    const double sgn = (lane & 1) ? -1.0 : 1.0;
#pragma unroll
    for (int j = 0; j < kEPL; ++j) v[j] = __builtin_fma(sgn, v[j], quad_xor<1>(v[j]));
  }
  {
    const double sgn = (lane & 2) ? -1.0 : 1.0;
#pragma unroll
    for (int j = 0; j < kEPL; ++j) v[j] = __builtin_fma(sgn, v[j], quad_xor<2>(v[j]));
  }
#pragma unroll
  for (int j = 0; j < kEPL; ++j) y[j] = (float)(v[j] * kInvSqrt128);
}

}  // namespace qm
}  // namespace w8a8
