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
//   * T threads own one row; each lane holds chunks of 32 elements (four
//     16-byte loads), all loads of a lane issued before any math: with rotation
//     32 consecutive elements, without it pieces laid out so that each wave
//     load instruction reads one contiguous kilobyte.
//   * Rotation is exact: the block sums of 128 bf16 values are formed in fp64
//     (exact for 8-bit significands unless the block's exponent spread exceeds
//     ~38 bits) -- the 32-point transform of each quarter block inside its lane
//     (5 butterfly stages), the 4-point transform across the quarters, which sit
//     16 lanes apart, on the fp64 matrix core (one v_mfma_f64_4x4x4f64 per
//     value, instead of two stages of cross-lane moves and FMAs on the vector
//     ALU, which the rotation keeps busy) -- then multiplied by fl64(2^-3.5) and
//     rounded once to fp32.  The codes are therefore those of the exactly
//     rotated row.
//   * amax by wave butterfly plus an LDS step across the row's waves.
//   * Codes from the exact quotient fl32(y / s), formed from r = fl32(1/s)
//     with one multiply and two FMAs (a correctly rounded reciprocal makes one
//     correction step exact; quant_math.h states the argument): int8 rounds it
//     half to even by adding 1.5 * 2^23 (no branch, no clamp), E4M3FN clamps
//     it to +-448 and takes the hardware RNE converter.
//   * Code stores, row-major or in the GEMM's packed layout (blocks of 32 rows
//     x 64 bytes, block (r / 32, k / 64) at byte ((r / 32) * (K / 64) + k / 64)
//     * 2048): with rotation a lane's 32 contiguous codes go out as two
//     16-byte stores, without it as 8-byte pieces that tile each wave's
//     instruction into one contiguous span.  Neither straddles a 64-byte group,
//     so the packed form only changes the address.
#include "internal.h"
#include "quant_math.h"

namespace w8a8 {
namespace {

using namespace qm;

constexpr int kXcds = 8;

// Block id -> the block's place in row order.  The hardware deals consecutive
// block ids to the 8 XCDs in turn; giving every XCD a contiguous range of rows
// keeps neighbouring rows -- which share 128-byte lines in the packed layout
// (64 bytes of each of two rows) -- in one L2, so each line is written back once.
__device__ __forceinline__ int64_t row_block_of(int bid, int nblocks) {
  const int q = nblocks / kXcds, r = nblocks % kXcds;
  const int xcd = bid % kXcds, idx = bid / kXcds;
  return (xcd < r) ? (int64_t)xcd * (q + 1) + idx : (int64_t)r * (q + 1) + (int64_t)(xcd - r) * q + idx;
}

// T threads per row (a multiple of 64), CMAX chunks of 32 elements per lane.
template <int T>
constexpr int rows_per_block() { return (T < 256 && 256 % T == 0) ? 256 / T : 1; }

template <int T, int CMAX, bool ROT, bool FP8>
__global__ void __launch_bounds__(T * rows_per_block<T>())
quantize_rows(const uint16_t* __restrict__ x, int64_t M, int K, uint8_t* __restrict__ q,
              float* __restrict__ s_out, bool packed) {
  constexpr int kRowsPerBlock = rows_per_block<T>();
  constexpr int kWavesPerRow = T / 64;
  const int tid = threadIdx.x % T;
  const int64_t row = row_block_of(blockIdx.x, gridDim.x) * kRowsPerBlock + threadIdx.x / T;
  const int lane = threadIdx.x & 63;
  // A row past M (only in the last block) is computed on row M - 1 and not
  // stored, so that every wave reaches the block barrier below.
  const bool live = row < M;
  const uint16_t* xr = x + (live ? row : M - 1) * (int64_t)K;
  typedef unsigned u32x4 __attribute__((ext_vector_type(4)));
  typedef unsigned u32x2 __attribute__((ext_vector_type(2)));
  // A lane's chunk i is four pieces of 8 elements.  With rotation the pieces are
  // consecutive (32 contiguous elements: a quarter of a 128-block per lane; lane
  // 16p + n holds quarter p of column n, so a wave's chunk covers 16 consecutive
  // blocks, 4 KB, each load instruction touching the same 64 16-byte pieces of
  // them as any other lane order would).
  // Without rotation any placement works, so the wave's 64 lanes take
  // consecutive 16-byte pieces of a 2048-element span: every load and store
  // instruction then covers one contiguous kilobyte (half as many cache lines
  // per instruction as 64-byte-strided lanes).
  auto piece = [&](int i, int p) -> int {
    if constexpr (ROT) return ((i * (T / 64) + tid / 64) * 16 + (lane & 15)) * 128 + (lane >> 4) * kEPL + 8 * p;
    else return (i * (T / 64) + tid / 64) * (64 * kEPL) + p * 512 + lane * 8;
  };
  // Every load is unconditional, and all are issued before any arithmetic: a piece
  // past K re-reads a piece of the row's first block (with rotation the 4 lanes of
  // the column read the whole first block, so their rotated values are that block's), which leaves
  // the amax unchanged and is never stored.  (Conditional loads let the compiler wait
  // for the first pieces before issuing the rest: 191 against 170 us at
  // 12,016 x 17,408 rotated.  Plain loads rather than non-temporal ones: 170 -> 160 us.)
  u32x4 raw[CMAX][4];
#pragma unroll
  for (int i = 0; i < CMAX; ++i)
#pragma unroll
    for (int v = 0; v < 4; ++v) {
      const int e = piece(i, v);
      const int src = e < K ? e : (ROT ? (lane >> 4) * kEPL + 8 * v : 8 * v);
      raw[i][v] = *reinterpret_cast<const u32x4*>(xr + src);
    }
  __builtin_amdgcn_sched_barrier(0);

  float y[CMAX][kEPL];
  float amax = 0.0f;
#pragma unroll
  for (int i = 0; i < CMAX; ++i) {
    if constexpr (ROT) {
      rotate_chunk_x16(raw[i], lane, y[i]);
    } else {
#pragma unroll
      for (int j = 0; j < 16; ++j) {
        const uint32_t w = raw[i][j / 4][j % 4];
        y[i][2 * j] = bf16lo(w);
        y[i][2 * j + 1] = bf16hi(w);
      }
    }
    // (pieces past K repeat the first block, which leaves the amax unchanged)
#pragma unroll
    for (int j = 0; j < kEPL; ++j) amax = fmaxf(amax, fabsf(y[i][j]));
  }

  amax = wave_max(amax);
  if constexpr (kWavesPerRow > 1) {
    __shared__ float red[kWavesPerRow * kRowsPerBlock];
    const int wave_in_block = threadIdx.x / 64;
    if (lane == 0) red[wave_in_block] = amax;
    __syncthreads();
    const int first = (threadIdx.x / T) * kWavesPerRow;
#pragma unroll
    for (int wv = 0; wv < kWavesPerRow; ++wv) amax = fmaxf(amax, red[first + wv]);
  }

  constexpr float kQmax = FP8 ? 448.0f : 127.0f;
  const float s = amax / kQmax;  // IEEE division
  if (!live) return;
  if (tid == 0) s_out[row] = s;
  const QuotientScale qs = quotient_scale(s);
  const uint32_t zero_mask = s > 0.0f ? ~0u : 0u;
#pragma unroll
  for (int i = 0; i < CMAX; ++i) apply_prefactor(y[i], qs);

  // element e of this row (e % 8 == 0) goes to qr + (e & ~63) * kstride + (e & 63)
  uint8_t* qr = q + (packed ? (row / 32) * 32 * (int64_t)K + (row % 32) * 64 : row * (int64_t)K);
  const int kstride = packed ? 32 : 1;
  // codes of the 8 elements of piece v of chunk i, as two 32-bit words (codes are
  // formed per piece, so that only 8 of them are live at a time)
  auto encode8 = [&](int i, int v, uint32_t* out) __attribute__((always_inline)) {
#pragma unroll
    for (int g = 0; g < 2; ++g) {
      float t[4];
      if constexpr (FP8) {
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          // (the correction step turns y = -0 into +0; the quotient takes y's sign)
          const float yv = y[i][8 * v + 4 * g + e];
          t[e] = fminf(fmaxf(__builtin_copysignf(quotient(yv, qs.s, qs.r), yv), -448.0f), 448.0f);
        }
        int wd = __builtin_amdgcn_cvt_pk_fp8_f32(t[0], t[1], 0, false);
        wd = __builtin_amdgcn_cvt_pk_fp8_f32(t[2], t[3], wd, true);
        out[g] = (uint32_t)wd & zero_mask;  // a zero row's codes are +0
      } else {
        const float* yg = &y[i][8 * v + 4 * g];
        out[g] = int8_codes4(yg[0], yg[1], yg[2], yg[3], qs.s, qs.r);  // (r = 0 for a zero row: zero codes)
      }
    }
  };
#pragma unroll
  for (int i = 0; i < CMAX; ++i) {
    if constexpr (ROT) {
      // the lane's 32 codes are contiguous (and 32-byte aligned, so inside one
      // 64-byte group of the packed layout): two 16-byte stores
      const int e0 = piece(i, 0);
      if (e0 >= K) continue;
#pragma unroll
      for (int h = 0; h < 2; ++h) {
        uint32_t lo[2], hi[2];
        encode8(i, 2 * h, lo);
        encode8(i, 2 * h + 1, hi);
        const int e = e0 + 16 * h;
        *reinterpret_cast<u32x4*>(qr + ((e & ~63) * kstride + (e & 63))) = u32x4{lo[0], lo[1], hi[0], hi[1]};
      }
    } else {
#pragma unroll
      for (int v = 0; v < 4; ++v) {
        const int e0 = piece(i, v);
        if (e0 >= K) continue;
        uint32_t out[2];
        encode8(i, v, out);
        *reinterpret_cast<u32x2*>(qr + ((e0 & ~63) * kstride + (e0 & 63))) = u32x2{out[0], out[1]};
      }
    }
  }
}

template <int T, bool ROT, bool FP8>
hipError_t dispatch_cmax(int cmax, const uint16_t* x, int64_t M, int K, uint8_t* q, float* s,
                         bool packed, hipStream_t stream) {
  constexpr int kRowsPerBlock = rows_per_block<T>();
  const dim3 block(T * kRowsPerBlock);
  const dim3 grid((unsigned)((M + kRowsPerBlock - 1) / kRowsPerBlock));
  switch (cmax) {
#define W8A8_Q_CASE(C)                                                                     \
  case C:                                                                                  \
    hipLaunchKernelGGL((quantize_rows<T, C, ROT, FP8>), grid, block, 0, stream, x, M, K, q, s, packed); \
    break;
    W8A8_Q_CASE(1) W8A8_Q_CASE(2) W8A8_Q_CASE(3) W8A8_Q_CASE(4)
#undef W8A8_Q_CASE
    default:
      return hipErrorInvalidValue;
  }
  return hipGetLastError();
}

// Threads per row T (a multiple of 64, at most 256, at most 4 chunks of 32
// elements per lane): the largest T whose lane slots exceed the row's chunks by
// at most 25% (fewest slots if none does) -- fewer chunks per lane means more
// waves in flight and shorter dependency chains.  (Measured with the current
// arithmetic: 16,384 x 4,096, 35.5 us with T = 128 against 37.9 us with
// T = 64; 1,502 x 4,096 rotated, 10.4 us with T = 128 against 13.4 us with
// T = 64; 12,016 x 17,408 rotated, 197 us with T = 192 (3 chunks) against
// 354, 300 and 282 us with T = 320, 576 and 1024.)  Rows longer than 4 x 256
// chunks (K > 32768) use 1024 threads.
template <bool ROT, bool FP8>
hipError_t dispatch_rows(const uint16_t* x, int64_t M, int K, uint8_t* q, float* s, bool packed,
                         hipStream_t stream) {
  const int nchunks = K / kEPL;
  if (nchunks > 4 * 256) {
    const int cmax = (nchunks + 1023) / 1024;
    if (cmax > 4) return hipErrorInvalidValue;
    return dispatch_cmax<1024, ROT, FP8>(cmax, x, M, K, q, s, packed, stream);
  }
  int best_t = 0, min_slots_t = 256, min_slots = 1 << 30;
  for (int t = 64; t <= 256; t += 64) {
    const int slots = (nchunks + t - 1) / t * t;
    if (slots > 4 * t) continue;
    if (slots < min_slots) { min_slots = slots; min_slots_t = t; }
    if (4 * slots > 5 * nchunks) continue;                  // more than 25% idle lanes
    best_t = t;
  }
  if (best_t == 0) best_t = min_slots_t;
  const int cmax = (nchunks + best_t - 1) / best_t;
  switch (best_t) {
    case 64: return dispatch_cmax<64, ROT, FP8>(cmax, x, M, K, q, s, packed, stream);
    case 128: return dispatch_cmax<128, ROT, FP8>(cmax, x, M, K, q, s, packed, stream);
    case 192: return dispatch_cmax<192, ROT, FP8>(cmax, x, M, K, q, s, packed, stream);
    default: return dispatch_cmax<256, ROT, FP8>(cmax, x, M, K, q, s, packed, stream);
  }
}

}  // namespace

hipError_t launch_quantize(const uint16_t* x, int64_t M, int64_t K, int rot_block, bool fp8,
                           bool packed, void* q, float* s, hipStream_t stream) {
  uint8_t* qb = static_cast<uint8_t*>(q);
  const int k = (int)K;
  if (packed && K % 64 != 0) return hipErrorInvalidValue;
  if (rot_block == 128) {
    return fp8 ? dispatch_rows<true, true>(x, M, k, qb, s, packed, stream)
               : dispatch_rows<true, false>(x, M, k, qb, s, packed, stream);
  }
  return fp8 ? dispatch_rows<false, true>(x, M, k, qb, s, packed, stream)
             : dispatch_rows<false, false>(x, M, k, qb, s, packed, stream);
}

}  // namespace w8a8
