// Per-row dynamic symmetric quantizer for gfx950 (stage 1 of the W8A8 path).
//
// What it computes: the per-token activation quantizer of the ConvRot INT8 path
// ("CLEF Calibrated INT8 ConvRot" card, notes under the latency table) and the
// per-token E4M3 activation quantizer of the FP8 dynamic scheme ("clef-flash-FP8"
// card, Quantization table); on weight rows it yields per-output-channel codes
// and scales taken straight from the weights (same card, note after recipe.yaml).
// For each row: optional rotation of every block of 128 by the normalized
// Sylvester Walsh-Hadamard transform, amax = max|y|, s = amax/127 (or /448),
// code = round-half-even(y/s) clamped to +-127 (or nearest E4M3FN of
// clamp(y/s, +-448)); a zero row gives s = 0 and zero codes.
//
// Design (HBM bound: 2 bytes read + 1 byte written per element):
//   * T threads own one row; each lane holds chunks of 16 consecutive bf16
//     (32 bytes, two 16-byte loads), all loads of a lane issued before any math.
//   * Rotation is exact: the block sums of 128 bf16 values are formed in fp64
//     (exact for 8-bit significands unless the block's exponent spread exceeds
//     ~38 bits) with 4 butterfly stages inside a lane and 3 across the 8 lanes
//     that share a block, then multiplied by fl64(2^-3.5) and rounded once to
//     fp32.  The quantized codes are therefore those of the exactly rotated row.
//   * amax by wave butterfly (shfl_xor) plus an LDS step across the row's waves.
//   * Codes use an IEEE fp32 division by s (correctly rounded), v_rndne_f32, and
//     for fp8 the hardware RNE converter after clamping to +-448.
//   * 16-byte coalesced stores of the codes.
#include "internal.h"

namespace w8a8 {
namespace {

constexpr int kEPL = 16;  // bf16 elements per lane per chunk

// fl64(2^-3.5) = fl64(sqrt(2)/2) / 8
constexpr double kInvSqrt128 = 0x1.6a09e667f3bcdp-4;

__device__ __forceinline__ float bf16lo(uint32_t w) { return __uint_as_float(w << 16); }
__device__ __forceinline__ float bf16hi(uint32_t w) { return __uint_as_float(w & 0xffff0000u); }

__device__ __forceinline__ float wave_max(float v) {
#pragma unroll
  for (int o = 32; o >= 1; o >>= 1) v = fmaxf(v, __shfl_xor(v, o, 64));
  return v;
}

__device__ __forceinline__ uint32_t pack_i8x4(float a, float b, float c, float d) {
  uint32_t ia = (uint32_t)(int)a & 0xffu, ib = (uint32_t)(int)b & 0xffu;
  uint32_t ic = (uint32_t)(int)c & 0xffu, id = (uint32_t)(int)d & 0xffu;
  return ia | (ib << 8) | (ic << 16) | (id << 24);
}

// T threads per row (64, 256 or 1024), CMAX chunks of 16 elements per lane.
template <int T, int CMAX, bool ROT, bool FP8>
__global__ void __launch_bounds__(T < 256 ? 256 : T)
quantize_rows(const uint16_t* __restrict__ x, int64_t M, int K, uint8_t* __restrict__ q,
              float* __restrict__ s_out) {
  constexpr int kRowsPerBlock = T < 256 ? 256 / T : 1;
  const int tid = threadIdx.x % T;
  const int64_t row = (int64_t)blockIdx.x * kRowsPerBlock + threadIdx.x / T;
  const int lane = threadIdx.x & 63;
  const int nchunks = K / kEPL;
  // Rows past M: the whole T-group leaves together (T is a multiple of 64 and a
  // block holds several rows only when T == 64, where no block barrier is used).
  if (row >= M) return;

  const uint16_t* xr = x + row * (int64_t)K;
  uint4 raw[CMAX][2];
#pragma unroll
  for (int i = 0; i < CMAX; ++i) {
    const int c = i * T + tid;
    if (c < nchunks) {
      const uint4* p = reinterpret_cast<const uint4*>(xr + (int64_t)c * kEPL);
      raw[i][0] = p[0];
      raw[i][1] = p[1];
    } else {
      raw[i][0] = make_uint4(0, 0, 0, 0);
      raw[i][1] = make_uint4(0, 0, 0, 0);
    }
  }

  float y[CMAX][kEPL];
  float amax = 0.0f;
#pragma unroll
  for (int i = 0; i < CMAX; ++i) {
    const uint32_t w[8] = {raw[i][0].x, raw[i][0].y, raw[i][0].z, raw[i][0].w,
                           raw[i][1].x, raw[i][1].y, raw[i][1].z, raw[i][1].w};
    if constexpr (ROT) {
      double v[kEPL];
#pragma unroll
      for (int j = 0; j < 8; ++j) {
        v[2 * j] = (double)bf16lo(w[j]);
        v[2 * j + 1] = (double)bf16hi(w[j]);
      }
      // element index bits 0..3 live in the lane
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
      // element index bits 4..6 are lane bits 0..2 (8 lanes per block of 128)
#pragma unroll
      for (int h = 1; h < 8; h <<= 1) {
        const double sgn = (lane & h) ? -1.0 : 1.0;
#pragma unroll
        for (int j = 0; j < kEPL; ++j) {
          const double p = __shfl_xor(v[j], h, 64);
          v[j] = __builtin_fma(sgn, v[j], p);  // lower lane: v + p; upper lane: p - v (exact)
        }
      }
#pragma unroll
      for (int j = 0; j < kEPL; ++j) y[i][j] = (float)(v[j] * kInvSqrt128);
    } else {
#pragma unroll
      for (int j = 0; j < 8; ++j) {
        y[i][2 * j] = bf16lo(w[j]);
        y[i][2 * j + 1] = bf16hi(w[j]);
      }
    }
    const bool valid = (i * T + tid) < nchunks;
#pragma unroll
    for (int j = 0; j < kEPL; ++j) amax = valid ? fmaxf(amax, fabsf(y[i][j])) : amax;
  }

  amax = wave_max(amax);
  if constexpr (T > 64) {
    __shared__ float red[T / 64];
    if (lane == 0) red[threadIdx.x / 64] = amax;
    __syncthreads();
#pragma unroll
    for (int wv = 0; wv < T / 64; ++wv) amax = fmaxf(amax, red[wv]);
  }

  constexpr float kQmax = FP8 ? 448.0f : 127.0f;
  const float s = amax / kQmax;  // IEEE division
  if (tid == 0) s_out[row] = s;
  const bool zero_row = !(amax > 0.0f);

  uint8_t* qr = q + row * (int64_t)K;
#pragma unroll
  for (int i = 0; i < CMAX; ++i) {
    const int c = i * T + tid;
    if (c >= nchunks) continue;
    uint32_t out[4];
#pragma unroll
    for (int g = 0; g < 4; ++g) {
      float t[4];
#pragma unroll
      for (int e = 0; e < 4; ++e) t[e] = zero_row ? 0.0f : y[i][4 * g + e] / s;
      if constexpr (FP8) {
#pragma unroll
        for (int e = 0; e < 4; ++e) t[e] = fminf(fmaxf(t[e], -448.0f), 448.0f);
        int wd = __builtin_amdgcn_cvt_pk_fp8_f32(t[0], t[1], 0, false);
        wd = __builtin_amdgcn_cvt_pk_fp8_f32(t[2], t[3], wd, true);
        out[g] = (uint32_t)wd;
      } else {
#pragma unroll
        for (int e = 0; e < 4; ++e) t[e] = fminf(fmaxf(__builtin_rintf(t[e]), -127.0f), 127.0f);
        out[g] = pack_i8x4(t[0], t[1], t[2], t[3]);
      }
    }
    *reinterpret_cast<uint4*>(qr + (int64_t)c * kEPL) = make_uint4(out[0], out[1], out[2], out[3]);
  }
}

template <int T, bool ROT, bool FP8>
hipError_t dispatch_cmax(int cmax, dim3 grid, const uint16_t* x, int64_t M, int K, uint8_t* q,
                         float* s, hipStream_t stream) {
  const dim3 block(T < 256 ? 256 : T);
  switch (cmax) {
#define W8A8_Q_CASE(C)                                                                     \
  case C:                                                                                  \
    hipLaunchKernelGGL((quantize_rows<T, C, ROT, FP8>), grid, block, 0, stream, x, M, K, q, s); \
    break;
    W8A8_Q_CASE(1) W8A8_Q_CASE(2) W8A8_Q_CASE(3) W8A8_Q_CASE(4)
    W8A8_Q_CASE(5) W8A8_Q_CASE(6) W8A8_Q_CASE(7) W8A8_Q_CASE(8)
#undef W8A8_Q_CASE
    default:
      return hipErrorInvalidValue;
  }
  return hipGetLastError();
}

template <bool ROT, bool FP8>
hipError_t dispatch_rows(const uint16_t* x, int64_t M, int K, uint8_t* q, float* s,
                         hipStream_t stream) {
  const int nchunks = K / kEPL;
  if (nchunks <= 64 * 8) {
    const int cmax = (nchunks + 63) / 64;
    const dim3 grid((unsigned)((M + 3) / 4));
    return dispatch_cmax<64, ROT, FP8>(cmax, grid, x, M, K, q, s, stream);
  }
  if (nchunks <= 256 * 8) {
    const int cmax = (nchunks + 255) / 256;
    return dispatch_cmax<256, ROT, FP8>(cmax, dim3((unsigned)M), x, M, K, q, s, stream);
  }
  const int cmax = (nchunks + 1023) / 1024;
  return dispatch_cmax<1024, ROT, FP8>(cmax, dim3((unsigned)M), x, M, K, q, s, stream);
}

}  // namespace

hipError_t launch_quantize(const uint16_t* x, int64_t M, int64_t K, int rot_block, bool fp8,
                           void* q, float* s, hipStream_t stream) {
  uint8_t* qb = static_cast<uint8_t*>(q);
  const int k = (int)K;
  if (rot_block == 128) {
    return fp8 ? dispatch_rows<true, true>(x, M, k, qb, s, stream)
               : dispatch_rows<true, false>(x, M, k, qb, s, stream);
  }
  return fp8 ? dispatch_rows<false, true>(x, M, k, qb, s, stream)
             : dispatch_rows<false, false>(x, M, k, qb, s, stream);
}

}  // namespace w8a8
