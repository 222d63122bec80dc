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

// Max over aligned groups of 4 (GROUP = 4) or 8 (GROUP = 8) lanes, in
// registers (DPP moves instead of LDS permutes): quad_perm swaps with the lane
// whose quad position differs in bit 0, then bit 1; for 8, row_half_mirror then
// brings lane 7 - i of the group, which holds the other quad's max.
template <int CTRL>
__device__ __forceinline__ float dpp_move(float x) {
  return __int_as_float(__builtin_amdgcn_mov_dpp(__float_as_int(x), CTRL, 0xF, 0xF, false));
}
template <int GROUP>
__device__ __forceinline__ float group_max(float v) {
  static_assert(GROUP == 4 || GROUP == 8, "groups of 4 or 8 lanes");
  v = fmaxf(v, dpp_move<0xB1>(v));     // quad_perm [1,0,3,2]
  v = fmaxf(v, dpp_move<0x4E>(v));     // quad_perm [2,3,0,1]
  if constexpr (GROUP == 8) v = fmaxf(v, dpp_move<0x141>(v));  // row_half_mirror
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

// Exact quotients.  Both code rules start from fl32(y / s): int8 rounds it half
// to even (|y| <= amax, so |y / s| <= 127 * (1 + 2^-23) and no clamp is ever
// needed), E4M3FN clamps it to +-448 and converts it.  With r = fl32(1/s)
// correctly rounded, t = fl32(y * r) lies within one ulp of y / s, so the
// residual e = y - t * s is exact in one FMA and fl32(t + e * r) is the
// correctly rounded quotient (Markstein's theorem for a correctly rounded
// reciprocal; also checked against the IEEE division on 1.7e10 random and
// near-tie pairs, no difference).  The residual is exact as long as
// exponent(t) + exponent(s) >= -103; the codes depend on the quotient only where
// |y / s| >= 2^-10 (E4M3FN's smallest rounding boundary; int8's is 1/2), so a
// scale of at least 2^-90 is enough.  A row with a smaller (nonzero) scale is
// first multiplied, values and scale alike, by 2^64: exact both ways
// (s >= 2^-149 lands at >= 2^-85, |y| <= 448 s stays far below overflow, and a
// power-of-two product of a subnormal loses no bits), and the real quotient is
// unchanged, so the codes are too.  For int8, adding 1.5 * 2^23 to the quotient
// rounds it to an integer, half to even, in the low bits of its
// representation, whose low byte is the two's-complement code.
constexpr float kRoundMagic = 12582912.0f;  // 1.5 * 2^23
constexpr float kTinyScale = 0x1p-90f;      // below this the row is rescaled
constexpr float kRescale = 0x1p64f;

// Scale and reciprocal the quotients of a row are formed with, and the factor
// its values must be multiplied by first (1, or 2^64 for a scale below 2^-90; a
// zero scale gives r = 0 and zero quotients).
struct QuotientScale {
  float s, r, pre;
};
__device__ __forceinline__ QuotientScale quotient_scale(float s) {
  const bool tiny = s < kTinyScale && s > 0.0f;
  const float sq = tiny ? s * kRescale : s;
  return QuotientScale{sq, s > 0.0f ? 1.0f / sq : 0.0f, tiny ? kRescale : 1.0f};
}

// Multiplies a lane's values by the row's pre-factor: one branch per lane,
// skipped by the whole wave unless one of its rows has a scale below 2^-90.
template <int N>
__device__ __forceinline__ void apply_prefactor(float (&v)[N], const QuotientScale& q) {
  if (q.pre != 1.0f) {
#pragma unroll
    for (int j = 0; j < N; ++j) v[j] *= q.pre;
  }
}

// fl32(y / s) for y carrying the row's pre-factor (see above).
__device__ __forceinline__ float quotient(float y, float s, float r) {
  const float t = y * r;
  return __builtin_fmaf(__builtin_fmaf(-t, s, y), r, t);
}

// Low byte = int8 code of y.
__device__ __forceinline__ uint32_t code_bits(float y, float s, float r) {
  return __float_as_uint(quotient(y, s, r) + kRoundMagic);
}

// Four codes packed as int8 bytes (byte i = code of y_i).
__device__ __forceinline__ uint32_t int8_codes4(float y0, float y1, float y2, float y3, float s, float r) {
  const uint32_t u0 = code_bits(y0, s, r), u1 = code_bits(y1, s, r);
  const uint32_t u2 = code_bits(y2, s, r), u3 = code_bits(y3, s, r);
  // v_perm_b32 selectors: 0..3 pick bytes of the second operand, 4..7 of the
  // first, 0x0c gives 0x00
  const uint32_t lo = __builtin_amdgcn_perm(u1, u0, 0x0c0c0400u);  // [u0.b0, u1.b0, 0, 0]
  const uint32_t hi = __builtin_amdgcn_perm(u3, u2, 0x04000c0cu);  // [0, 0, u2.b0, u3.b0]
  return lo | hi;
}

// The 128-point transform factors over the element index e = 32p + t: with
// j = 32q + u, H128[j][e] = H4[q][p] * H32[u][t] (Sylvester sign (-1)^popcount(j & e)).
// A lane holds the 32 elements of one quarter p of a block: it forms the 32-point
// transform of its quarter in fp64 (5 butterfly stages), and the 4-point transform
// across the block's 4 quarters combines lanes.  The block sums of the bf16 values
// are exact in fp64 (8-bit significands; unless the block's exponent spread
// exceeds ~38 bits), in any order; they are multiplied by fl64(2^-3.5) and rounded
// once to fp32.

// bf16 pairs -> fp64, then the in-lane 32-point transform.
__device__ __forceinline__ void transform32(const u32x4 (&raw)[4], double (&v)[kEPL]) {
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
}

// fl32(fl64(v * 2^-3.5)) for the lane's 32 transformed values.
__device__ __forceinline__ void scale_to_f32(const double (&v)[kEPL], float (&y)[kEPL]) {
#pragma unroll
  for (int j = 0; j < kEPL; ++j) y[j] = (float)(v[j] * kInvSqrt128);
}

// Exact rotation of one 32-element chunk, quarters in DPP quads: the lane holds
// quarter p = lane % 4 of its block (the other lanes of its quad hold the rest);
// the 4-point transform takes two exchange stages of quad_perm moves.
__device__ __forceinline__ void rotate_chunk(const u32x4 (&raw)[4], int lane, float (&y)[kEPL]) {
  double v[kEPL];
  transform32(raw, v);
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
  scale_to_f32(v, y);
}

// Exact rotation of one 32-element chunk, quarters 16 lanes apart: lane
// 16p + n holds quarter p of the block of column n (n < 16), so a wave holds 16
// blocks.  The 4-point transform across quarters is a matrix product on the fp64
// matrix core: v_mfma_f64_4x4x4f64 runs 4 independent 4x4x4 products, one per
// lane group of equal bits 2-3, with B[k][j] = lane 16k + 4b + j, A[i][k] = lane
// 16k + 4b + i and D[i][j] = lane 16i + 4b + j (b = the group; the layout is
// checked on the device by tests/test_gpu_f64_mfma_layout.py).  B is a value of quarter k of column 4b + j, A = H4, so D at
// lane 16q + n is sum_k H4[q][k] * (quarter k of column n): quarter q of the
// transform, landing in the lane that holds quarter q.  Products with +-1 are
// exact and the sums are those of the exact block sums, so the result is the
// quad form's bit for bit; the matrix core takes the 64 cross-lane products
// per value off the vector ALU, which the exact rotation keeps busy.
__device__ __forceinline__ void rotate_chunk_x16(const u32x4 (&raw)[4], int lane, float (&y)[kEPL]) {
  double v[kEPL];
  transform32(raw, v);
  // A[i][k] at lane 16k + 4b + i: H4[i][k] = (-1)^popcount(i & k)
  const double h = (__builtin_popcount((lane >> 4) & lane & 3) & 1) ? -1.0 : 1.0;
#pragma unroll
  for (int j = 0; j < kEPL; ++j) v[j] = __builtin_amdgcn_mfma_f64_4x4x4f64(h, v[j], 0.0, 0, 0, 0);
  scale_to_f32(v, y);
}

}  // namespace qm
}  // namespace w8a8
