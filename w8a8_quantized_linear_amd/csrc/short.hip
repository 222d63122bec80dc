// Single-launch path for short inputs: per-token quantization, integer GEMM and
// epilogue in one kernel.
//
// What it computes: exactly what the two-kernel whole path computes -- the
// activation quantizer of the ConvRot INT8 path ("CLEF Calibrated INT8 ConvRot"
// card, notes under the latency table: optional exact block-128 rotation,
// s = amax/127, round-half-even codes) followed by the integer GEMM and the fused
// dequant or paired gate/up SwiGLU epilogue (same card, Benefits list; "Loading
// CLEF INT8", fuse_mlp) -- with bit-identical codes and scales.  The pages note
// that INT8 loses to BF16 on short inputs; at these sizes two launches and a
// round trip of the codes through memory cost more than the arithmetic.
//
// Design.  A workgroup owns 32 token rows and 64 weight rows (64 output
// columns, or 32 gate + 32 up rows) and runs three phases:
//   0. every wave issues the direct-to-LDS loads of all its weight stages
//      (a quarter of K, 32 bytes per stage, its own LDS region), so they land
//      while the rows are quantized;
//   1. it quantizes its own 32 rows into LDS (8 lanes per row, each holding up
//      to 4 chunks of 32 rotated values in registers: one pass over the row),
//      and the workgroups of the first weight tile also write the codes (packed
//      layout) and scales to the workspace;
//   2. each of the 4 waves multiplies its quarter of K from LDS, with no
//      barriers;
//   3. the int32 partial sums of waves 1..3 are added to wave 0's through LDS
//      (exact) and wave 0 runs the usual epilogue.
// Every tile quantizes its rows again; this is meant for batches whose whole
// quantization costs less than a kernel launch.
#include <type_traits>

#include "epilogue_math.h"
#include "internal.h"
#include "quant_math.h"

namespace w8a8 {
namespace {

using namespace qm;
typedef int v4i __attribute__((ext_vector_type(4)));
typedef int v16i __attribute__((ext_vector_type(16)));
typedef unsigned u32x2 __attribute__((ext_vector_type(2)));

constexpr int kBM = 32, kBW = 64;        // token rows, weight rows per tile
constexpr int kMaxK = 1024;
constexpr int kStages = kMaxK / 4 / 32;  // weight stages per wave (all resident)
constexpr int kStageB = kBW * 32;        // 64 rows x 32 bytes of K
constexpr int kCPL = kMaxK / kEPL / 8;   // chunks of 32 elements per lane (8 lanes per row)

__device__ __forceinline__ void dma16(const uint8_t* g, uint8_t* l) {
#if defined(__HIP_DEVICE_COMPILE__)
  __builtin_amdgcn_global_load_lds(g, l, 16, 0, 0);
#endif
}

template <int n>
__device__ __forceinline__ void wait_vm() {
  static_assert(n >= 0 && n < 64, "vmcnt range");
  __builtin_amdgcn_s_waitcnt((n & 15) | (7 << 4) | (15 << 8) | ((n >> 4) << 14));
}


template <Epi EPI, bool ROT, bool PB>
__global__ void __launch_bounds__(256)
linear_short(const uint16_t* __restrict__ x, const uint8_t* __restrict__ w,
             const float* __restrict__ s_ch, const uint16_t* __restrict__ bias,
             uint16_t* __restrict__ y, int64_t M, int64_t N, int K, uint8_t* __restrict__ q_ws,
             float* __restrict__ s_ws, int tiles_n) {
  constexpr int A_BYTES = kBM * (kMaxK + 16);
  constexpr int B_BYTES = 4 * kStages * kStageB;
  static_assert(3 * 2 * 16 * 64 * 4 <= B_BYTES, "partial sums fit in the weight stages");
  __shared__ __attribute__((aligned(1024))) uint8_t lds[A_BYTES + B_BYTES];
  __shared__ float s_rows[kBM];
  const int a_stride = K + 16;                 // 16-byte skew per row: conflict-free fragment reads
  uint8_t* a_lds = lds;
  uint8_t* b_lds = lds + A_BYTES;

  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int tile_m = blockIdx.x / tiles_n, tile_n = blockIdx.x % tiles_n;
  const int64_t mb = (int64_t)tile_m * kBM;
  const int64_t nb = (EPI == Epi::kSwiglu) ? (int64_t)tile_n * (kBW / 2) : (int64_t)tile_n * kBW;

  // ---- phase 0: wave `wave` loads its weight rows for K range [wave * K/4, (wave + 1) * K/4) ----
  // Weight stage: 64 rows x 32 bytes in LDS, row r at 32r, its two 16-byte
  // chunks swapped for rows with bit 2 set (conflict-free fragment reads).
  // One load instruction covers 32 rows: lane -> slot p = 64 i + lane, row p / 2.
  const int kq = K / 4, steps = kq / 32;
  const int64_t k_begin = (int64_t)wave * kq;
  // (b_base is per lane: the up rows of a gate/up tile need not start on a
  // 32-row boundary, so the loads use the 64-bit vector address form)
  uint32_t b_off[2];
  const uint8_t* b_base[2];
#pragma unroll
  for (int i = 0; i < 2; ++i) {
    const int p = 64 * i + lane, r = p / 2, c = (p & 1) ^ ((r >> 2) & 1);
    int64_t row;                               // absolute weight row (clamped: unused rows re-read the last)
    if constexpr (EPI == Epi::kSwiglu) {
      const int64_t col = min<int64_t>(nb + (r % 32), N - 1);
      row = r < 32 ? col : N + col;
    } else {
      row = min<int64_t>(nb + r, N - 1);
    }
    // relative to a 32-row-aligned base so the per-lane offset stays small
    const int64_t base_row = row / 32 * 32;
    b_base[i] = w + base_row * K;
    const int64_t rel = row - base_row;
    b_off[i] = PB ? (uint32_t)(rel * 64 + c * 16) : (uint32_t)(rel * K + c * 16);
  }
  uint8_t* ring = b_lds + wave * (kStages * kStageB);
  // stage st of this wave -> its own LDS slot st (steps <= kStages)
  for (int st = 0; st < steps; ++st) {
    const int64_t k = k_begin + (int64_t)st * 32;
    const uint32_t koff = PB ? (uint32_t)((k / 64) * 2048 + (k % 64)) : (uint32_t)k;
    uint8_t* dst = ring + st * kStageB;
#pragma unroll
    for (int i = 0; i < 2; ++i) dma16(b_base[i] + (b_off[i] + koff), dst + i * 1024);
  }
  // ---- phase 1: quantize rows mb .. mb+31 into LDS --------------------------
  {
    const int r = tid >> 3, q = tid & 7;       // 8 lanes per row; lanes 4q'..4q'+3 form DPP quads
    const int64_t m = mb + r;
    const bool live = m < M;
    const uint16_t* xr = x + (live ? m : M - 1) * (int64_t)K;
    const int nchunks = K / kEPL;              // chunk c = 8 i + q of the row is this lane's chunk i
    u32x4 raw[kCPL][4];
#pragma unroll
    for (int i = 0; i < kCPL; ++i) {
      const int c = 8 * i + q;
#pragma unroll
      for (int p = 0; p < 4; ++p)
        raw[i][p] = c < nchunks ? *reinterpret_cast<const u32x4*>(xr + c * kEPL + 8 * p) : u32x4{0, 0, 0, 0};
    }
    float v[kCPL][kEPL];
    float amax = 0.0f;
#pragma unroll
    for (int i = 0; i < kCPL; ++i) {
      if constexpr (ROT) {
        rotate_chunk(raw[i], lane, v[i]);
      } else {
#pragma unroll
        for (int j = 0; j < 16; ++j) {
          const uint32_t wd = raw[i][j / 4][j % 4];
          v[i][2 * j] = bf16lo(wd);
          v[i][2 * j + 1] = bf16hi(wd);
        }
      }
#pragma unroll
      for (int j = 0; j < kEPL; ++j) amax = fmaxf(amax, fabsf(v[i][j]));
    }
#pragma unroll
    for (int o = 1; o < 8; o <<= 1) amax = fmaxf(amax, __shfl_xor(amax, o, 64));
    const float s = amax / 127.0f;             // IEEE division
    const QuotientScale qs = quotient_scale(s);
#pragma unroll
    for (int i = 0; i < kCPL; ++i) apply_prefactor(v[i], qs);
    const bool write_ws = tile_n == 0 && live;
    if (q == 0) {
      s_rows[r] = s;
      if (write_ws) s_ws[m] = s;
    }
    uint8_t* qg = q_ws + (m / 32) * 32 * (int64_t)K + (m % 32) * 64;   // packed row m
#pragma unroll
    for (int i = 0; i < kCPL; ++i) {
      const int c = 8 * i + q;
      if (c >= nchunks) continue;
      uint32_t wd[8];
#pragma unroll
      for (int g = 0; g < 8; ++g)
        wd[g] = int8_codes4(v[i][4 * g], v[i][4 * g + 1], v[i][4 * g + 2], v[i][4 * g + 3], qs.s, qs.r);
      const u32x4 lo = u32x4{wd[0], wd[1], wd[2], wd[3]}, hi = u32x4{wd[4], wd[5], wd[6], wd[7]};
      uint8_t* la = a_lds + r * a_stride + c * kEPL;
      *reinterpret_cast<u32x4*>(la) = lo;
      *reinterpret_cast<u32x4*>(la + 16) = hi;
      if (write_ws) {
        const int k = c * kEPL;                // 32 codes inside one 64-byte group
        uint8_t* dst = qg + (k / 64) * 2048 + (k % 64);
        *reinterpret_cast<u32x4*>(dst) = lo;
        *reinterpret_cast<u32x4*>(dst + 16) = hi;
      }
    }
  }
  // every wave's weight stages have landed (its own loads), and everyone's codes
  wait_vm<0>();
  __syncthreads();

  // ---- phase 2: multiply this wave's quarter of K from LDS -------------------
  v16i acc[2] = {v16i{}, v16i{}};
  const int frag_row = lane & 31, frag_half = lane >> 5;
  for (int s = 0; s < steps; ++s) {
    const uint8_t* bs = ring + s * kStageB;
    const int k = (int)(k_begin + s * 32) + 16 * frag_half;
    const v4i fa = *reinterpret_cast<const v4i*>(a_lds + frag_row * a_stride + k);
    v4i fb[2];
#pragma unroll
    for (int t = 0; t < 2; ++t) {
      const int r = 32 * t + frag_row, c = frag_half ^ ((r >> 2) & 1);
      fb[t] = *reinterpret_cast<const v4i*>(bs + r * 32 + c * 16);
    }
#pragma unroll
    for (int t = 0; t < 2; ++t) acc[t] = __builtin_amdgcn_mfma_i32_32x32x32_i8(fb[t], fa, acc[t], 0, 0, 0);
  }
  __syncthreads();

  // ---- phase 3: add the partial sums, epilogue ------------------------------
  int32_t* red = reinterpret_cast<int32_t*>(b_lds);
  if (wave > 0) {
#pragma unroll
    for (int t = 0; t < 2; ++t)
#pragma unroll
      for (int v = 0; v < 16; ++v) red[(((wave - 1) * 2 + t) * 16 + v) * 64 + lane] = acc[t][v];
  }
  __syncthreads();
  if (wave > 0) return;
#pragma unroll
  for (int src = 0; src < 3; ++src)
#pragma unroll
    for (int t = 0; t < 2; ++t)
#pragma unroll
      for (int v = 0; v < 16; ++v) acc[t][v] += red[((src * 2 + t) * 16 + v) * 64 + lane];

  // 32x32 block layout: lane holds token row frag_row, weight rows 8q + 4 h + 0..3
  const int64_t m = mb + frag_row;
  if (m >= M) return;
  const float st = s_rows[frag_row];
  uint16_t* yrow = y + m * N;
  if constexpr (EPI == Epi::kDequant) {
#pragma unroll
    for (int t = 0; t < 2; ++t)
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        const int64_t n0 = nb + t * 32 + 8 * q + 4 * frag_half;
        if (n0 >= N) continue;
        const float4 sc = *reinterpret_cast<const float4*>(s_ch + n0);
        float bv[4] = {0.f, 0.f, 0.f, 0.f};
        if (bias) bf16x4(*reinterpret_cast<const uint2*>(bias + n0), bv);
        const float scv[4] = {sc.x, sc.y, sc.z, sc.w};
        uint16_t o[4];
#pragma unroll
        for (int v = 0; v < 4; ++v) o[v] = f32_to_bf16_rne(__builtin_fmaf((float)acc[t][4 * q + v], st * scv[v], bv[v]));
        *reinterpret_cast<uint2*>(yrow + n0) =
            make_uint2((uint32_t)o[0] | ((uint32_t)o[1] << 16), (uint32_t)o[2] | ((uint32_t)o[3] << 16));
      }
  } else {  // SwiGLU: block 0 holds gate rows, block 1 the matching up rows
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      const int64_t n0 = nb + 8 * q + 4 * frag_half;
      if (n0 >= N) continue;
      const float4 sg = *reinterpret_cast<const float4*>(s_ch + n0);
      const float4 su = *reinterpret_cast<const float4*>(s_ch + N + n0);
      float bg[4] = {0.f, 0.f, 0.f, 0.f}, bu[4] = {0.f, 0.f, 0.f, 0.f};
      if (bias) {
        bf16x4(*reinterpret_cast<const uint2*>(bias + n0), bg);
        bf16x4(*reinterpret_cast<const uint2*>(bias + N + n0), bu);
      }
      const float sgv[4] = {sg.x, sg.y, sg.z, sg.w}, suv[4] = {su.x, su.y, su.z, su.w};
      uint16_t o[4];
#pragma unroll
      for (int v = 0; v < 4; ++v) {
        const float g = __builtin_fmaf((float)acc[0][4 * q + v], st * sgv[v], bg[v]);
        const float u = __builtin_fmaf((float)acc[1][4 * q + v], st * suv[v], bu[v]);
        o[v] = f32_to_bf16_rne(silu_f32(g) * u);
      }
      *reinterpret_cast<uint2*>(yrow + n0) =
          make_uint2((uint32_t)o[0] | ((uint32_t)o[1] << 16), (uint32_t)o[2] | ((uint32_t)o[3] << 16));
    }
  }
}

template <Epi EPI, bool ROT>
hipError_t launch_k(const uint16_t* x, const void* w, bool w_packed, const float* s_ch,
                    const uint16_t* bias, uint16_t* y, int64_t M, int64_t N, int64_t K, void* q_ws,
                    float* s_ws, hipStream_t stream) {
  const int64_t tiles_m = (M + kBM - 1) / kBM;
  const int64_t cols = (EPI == Epi::kSwiglu) ? kBW / 2 : kBW;
  const int64_t tiles_n = (N + cols - 1) / cols;
  if (tiles_m * tiles_n > 0x7fffffff) return hipErrorInvalidValue;
  const dim3 grid((unsigned)(tiles_m * tiles_n)), block(256);
  const uint8_t* wb = static_cast<const uint8_t*>(w);
  uint8_t* qb = static_cast<uint8_t*>(q_ws);
  if (w_packed)
    hipLaunchKernelGGL((linear_short<EPI, ROT, true>), grid, block, 0, stream, x, wb, s_ch, bias, y, M, N,
                       (int)K, qb, s_ws, (int)tiles_n);
  else
    hipLaunchKernelGGL((linear_short<EPI, ROT, false>), grid, block, 0, stream, x, wb, s_ch, bias, y, M, N,
                       (int)K, qb, s_ws, (int)tiles_n);
  return hipGetLastError();
}

}  // namespace

// One workgroup per CU (~97 KiB of LDS): the single launch pays off while the
// tiles fit in one round on the 256 CUs (measured: 298 x 1,024 x 1,024 in 13.9 us
// against 18.3 us for two kernels; 320 tiles of a gate/up shape take 25 us).
bool short_path_fits(int64_t M, int64_t N, int64_t K, Epi epi) {
  if (epi == Epi::kRawI32 || K > kShortMaxK || M > kShortMaxM) return false;
  const int64_t cols = (epi == Epi::kSwiglu) ? kBW / 2 : kBW;
  return ((M + kBM - 1) / kBM) * ((N + cols - 1) / cols) <= kShortMaxTiles;
}

hipError_t launch_linear_short(Epi epi, const uint16_t* x, const void* w, bool w_packed,
                               const float* s_ch, const uint16_t* bias, uint16_t* y, int64_t M,
                               int64_t N, int64_t K, int rot_block, void* q_ws, float* s_ws,
                               hipStream_t stream) {
  static_assert(kShortMaxK == kMaxK, "one K capacity");
  if (K > kMaxK || K % 128 != 0) return hipErrorInvalidValue;
  if (epi == Epi::kSwiglu)
    return rot_block ? launch_k<Epi::kSwiglu, true>(x, w, w_packed, s_ch, bias, y, M, N, K, q_ws, s_ws, stream)
                     : launch_k<Epi::kSwiglu, false>(x, w, w_packed, s_ch, bias, y, M, N, K, q_ws, s_ws, stream);
  if (epi == Epi::kDequant)
    return rot_block ? launch_k<Epi::kDequant, true>(x, w, w_packed, s_ch, bias, y, M, N, K, q_ws, s_ws, stream)
                     : launch_k<Epi::kDequant, false>(x, w, w_packed, s_ch, bias, y, M, N, K, q_ws, s_ws, stream);
  return hipErrorInvalidValue;
}

}  // namespace w8a8
