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
// columns, or 32 gate + 32 up rows); 4 waves, each multiplying one quarter of
// K.  The critical path is the row loads, then the quantization (vector ALU
// bound: every tile quantizes its rows again), then a short MFMA phase and the
// epilogue, so everything else is issued early and kept off that path:
//   0. every lane issues the loads of its share of the 32 rows, then the
//      channel scales and bias of the outputs it will write;
//   1. the rows are quantized into LDS (8 lanes per row; without rotation each
//      load instruction reads one contiguous 128-byte piece per row, with it a
//      lane holds 32 consecutive elements of a 128-block).  The MFMA
//      fragments of the wave's weights are loaded on the way, half after the
//      row amax and half after the first codes: each weight byte of the tile
//      feeds exactly one lane, so the fragments go straight to registers (no
//      LDS staging).  All loads are unconditional register loads, so the
//      compiler's waits drain them in order, piece by piece;
//   2. each wave multiplies its quarter of K (token codes from LDS, weights
//      from registers), while the workgroups of the first weight tile write
//      the codes (packed layout) and scales to the workspace;
//   3. the int32 partial sums of the 4 waves meet in LDS (exact) and every
//      thread finishes 8 (SwiGLU: 4) outputs of one row with one store.
// Every tile quantizes its rows again; this is meant for batches whose whole
// quantization costs less than a kernel launch.
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
constexpr int kSteps = kMaxK / 4 / 32;   // 32-deep MFMA steps per wave (a quarter of K)
constexpr int kCPL = kMaxK / kEPL / 8;   // chunks of 32 elements per lane (8 lanes per row)

template <Epi EPI, bool ROT, bool PB>
__global__ void __launch_bounds__(256)
linear_short(const uint16_t* __restrict__ x, const uint8_t* __restrict__ w,
             const float* __restrict__ s_ch, const uint16_t* __restrict__ bias,
             uint16_t* __restrict__ y, int64_t M, int64_t N, int K, uint8_t* __restrict__ q_ws,
             float* __restrict__ s_ws, int tiles_n) {
  constexpr bool SWIGLU = EPI == Epi::kSwiglu;
  constexpr int A_BYTES = kBM * (kMaxK + 16);
  // partial sums after the MFMA phase, over the codes:
  // [wave][block t][qq][half h][token row j] x 16 bytes (4 int32)
  constexpr int RED_BYTES = 4 * 2 * 4 * 2 * 32 * 16;
  static_assert(RED_BYTES <= A_BYTES, "partial sums fit over the codes");
  __shared__ __attribute__((aligned(1024))) uint8_t a_lds[A_BYTES];
  __shared__ float s_rows[kBM];
  const int a_stride = K + 16;                 // 16-byte skew per row: conflict-free fragment reads

  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int tile_m = blockIdx.x / tiles_n, tile_n = blockIdx.x % tiles_n;
  const int64_t mb = (int64_t)tile_m * kBM;
  const int64_t nb = SWIGLU ? (int64_t)tile_n * (kBW / 2) : (int64_t)tile_n * kBW;

  // ---- phase 0a: loads of this lane's share of row mb + r --------------------
  // 8 lanes per row.  Piece i*4+p of lane q (8 bf16 values, 16 bytes):
  //   rotation: chunk c = 8i + q (32 elements, a quarter of a 128-block; the 4
  //             lanes of a DPP quad hold one block), elements 32c + 8p ..;
  //   none:     elements 64 (4i + p) + 8q .. (the row's 8 lanes read 128
  //             contiguous bytes per instruction).
  // Pieces past K (K < 1024) read the same position of the row's first
  // 128-block instead: real values of the row, so the amax is unchanged (with
  // rotation the quad rotates block 0 again), and their codes are never stored.
  const int r = tid >> 3, q = tid & 7;
  const int64_t m = mb + r;
  const bool live = m < M;
  const uint16_t* xr = x + (live ? m : M - 1) * (int64_t)K;
  auto elem = [&](int i, int p) -> int {
    if constexpr (ROT) return (8 * i + q) * kEPL + 8 * p;
    else return 64 * (4 * i + p) + 8 * q;
  };
  u32x4 raw[kCPL][4];
#pragma unroll
  for (int i = 0; i < kCPL; ++i)
#pragma unroll
    for (int p = 0; p < 4; ++p) {
      const int e = elem(i, p);
      raw[i][p] = *reinterpret_cast<const u32x4*>(xr + (e < K ? e : e & 127));
    }

  // ---- this lane's weight fragments for the wave's quarter of K (loaded in phase 1) ----
  // MFMA 32x32x32 operand: lane (row rr % 32 = lane % 32, half = lane / 32)
  // holds bytes 16 half .. 16 half + 15 of a 32-byte step of weight row rr,
  // for the two 32-row blocks t (rows 32 t + lane % 32 of the tile).  Steps
  // past K / 128 repeat the last one (never multiplied).
  const int frag_row = lane & 31, frag_half = lane >> 5;
  const int kq = K / 4, steps = kq / 32;
  const int k_begin = wave * kq;
  v4i fb[kSteps][2];
  const uint8_t* wr[2];
#pragma unroll
  for (int t = 0; t < 2; ++t) {
    int64_t row;                               // absolute weight row (clamped: unused rows re-read the last)
    if constexpr (SWIGLU) {
      const int64_t col = min<int64_t>(nb + frag_row, N - 1);
      row = t == 0 ? col : N + col;
    } else {
      row = min<int64_t>(nb + 32 * t + frag_row, N - 1);
    }
    wr[t] = PB ? w + (row / 32) * 32 * (int64_t)K + (row % 32) * 64 : w + row * (int64_t)K;
  }
  auto load_steps = [&](int first, int last) __attribute__((always_inline)) {
#pragma unroll
    for (int st = first; st < last; ++st)
#pragma unroll
      for (int t = 0; t < 2; ++t) {
        const int k = k_begin + 32 * min(st, steps - 1) + 16 * frag_half;
        fb[st][t] = *reinterpret_cast<const v4i*>(wr[t] + (PB ? (k / 64) * 2048 + (k % 64) : k));
      }
  };

  // ---- phase 0b: channel scales and bias of this thread's outputs ----------
  // Output role: token row er = tid % 32, column group ec = tid / 32 -- 8
  // columns nb + 8 ec .. (SwiGLU: 4 columns nb + 4 ec .., gate and up).
  const int er = tid & 31, ec = tid >> 5;
  constexpr int kOutCols = SWIGLU ? 4 : 8;
  const int64_t n0 = nb + (int64_t)kOutCols * ec;
  const bool col_live = n0 < N;                // N % 8 == 0: the group is whole or absent
  // dequant: columns n0 .. n0+3 and n0+4 .. n0+7; SwiGLU: gate n0 .., up N + n0 ..
  // (a thread past N reads column 0; kept raw until the epilogue)
  const int64_t c0 = col_live ? n0 : 0, c1 = SWIGLU ? N + c0 : c0 + 4;
  const float4 sc0 = *reinterpret_cast<const float4*>(s_ch + c0);
  const float4 sc1 = *reinterpret_cast<const float4*>(s_ch + c1);
  // (no bias: the same offsets of s_ch, which is at least as long, are read and
  // ignored; a conditional load would make the compiler drain every load)
  const uint16_t* bsrc = bias ? bias : reinterpret_cast<const uint16_t*>(s_ch);
  const uint2 bw0 = *reinterpret_cast<const uint2*>(bsrc + c0);
  const uint2 bw1 = *reinterpret_cast<const uint2*>(bsrc + c1);
  // (all of the above issued before any row arithmetic)
  __builtin_amdgcn_sched_barrier(0);

  // ---- phase 1: quantize rows mb .. mb+31 into LDS --------------------------
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
  // first half of the weight fragments: issued once the row pieces have been
  // read, so that they do not hold up the row loads (the second half follows
  // the first codes; this split measured fastest)
  __builtin_amdgcn_sched_barrier(0);
  load_steps(0, kSteps / 2);
  __builtin_amdgcn_sched_barrier(0);
  amax = group_max<8>(amax);                   // the row's 8 lanes
  const float s = amax / 127.0f;               // IEEE division
  const QuotientScale qs = quotient_scale(s);
#pragma unroll
  for (int i = 0; i < kCPL; ++i) apply_prefactor(v[i], qs);
  if (q == 0) s_rows[r] = s;
  // codes of piece i*4+p: words cw[i][2p], cw[i][2p+1]
  uint32_t cw[kCPL][8];
#pragma unroll
  for (int i = 0; i < kCPL; ++i) {
#pragma unroll
    for (int g = 0; g < 8; ++g)
      cw[i][g] = int8_codes4(v[i][4 * g], v[i][4 * g + 1], v[i][4 * g + 2], v[i][4 * g + 3], qs.s, qs.r);
    if (i == 0) {
      // second half of the weight fragments
      __builtin_amdgcn_sched_barrier(0);
      load_steps(kSteps / 2, kSteps);
      __builtin_amdgcn_sched_barrier(0);
    }
  }
#pragma unroll
  for (int i = 0; i < kCPL; ++i) {
    if constexpr (ROT) {
      const int e = elem(i, 0);
      if (e >= K) continue;
      uint8_t* la = a_lds + r * a_stride + e;
      *reinterpret_cast<u32x4*>(la) = u32x4{cw[i][0], cw[i][1], cw[i][2], cw[i][3]};
      *reinterpret_cast<u32x4*>(la + 16) = u32x4{cw[i][4], cw[i][5], cw[i][6], cw[i][7]};
    } else {
#pragma unroll
      for (int p = 0; p < 4; ++p) {
        const int e = elem(i, p);
        if (e >= K) continue;
        *reinterpret_cast<u32x2*>(a_lds + r * a_stride + e) = u32x2{cw[i][2 * p], cw[i][2 * p + 1]};
      }
    }
  }
  __syncthreads();                             // every row's codes are in LDS

  // ---- workspace: codes (packed layout) and scales, first weight tile only ----
  if (tile_n == 0 && live) {
    if (q == 0) s_ws[m] = s;
    uint8_t* qg = q_ws + (m / 32) * 32 * (int64_t)K + (m % 32) * 64;   // packed row m
#pragma unroll
    for (int i = 0; i < kCPL; ++i) {
      if constexpr (ROT) {
        const int e = elem(i, 0);              // 32 codes inside one 64-byte group
        if (e >= K) continue;
        uint8_t* dst = qg + (e / 64) * 2048 + (e % 64);
        *reinterpret_cast<u32x4*>(dst) = u32x4{cw[i][0], cw[i][1], cw[i][2], cw[i][3]};
        *reinterpret_cast<u32x4*>(dst + 16) = u32x4{cw[i][4], cw[i][5], cw[i][6], cw[i][7]};
      } else {
#pragma unroll
        for (int p = 0; p < 4; ++p) {
          const int e = elem(i, p);            // 8 codes inside one 64-byte group
          if (e >= K) continue;
          *reinterpret_cast<u32x2*>(qg + (e / 64) * 2048 + (e % 64)) = u32x2{cw[i][2 * p], cw[i][2 * p + 1]};
        }
      }
    }
  }

  // ---- phase 2: multiply this wave's quarter of K ----------------------------
  v16i acc[2] = {v16i{}, v16i{}};
#pragma unroll
  for (int st = 0; st < kSteps; ++st) {
    if (st >= steps) break;                    // uniform
    const int k = k_begin + 32 * st + 16 * frag_half;
    const v4i fa = *reinterpret_cast<const v4i*>(a_lds + frag_row * a_stride + k);
#pragma unroll
    for (int t = 0; t < 2; ++t) acc[t] = __builtin_amdgcn_mfma_i32_32x32x32_i8(fb[st][t], fa, acc[t], 0, 0, 0);
  }
  __syncthreads();                             // every wave is done with the codes

  // ---- phase 3: partial sums through LDS, epilogue ---------------------------
  // 32x32 block layout: lane (j = lane % 32, h = lane / 32) holds token row j,
  // weight rows 8 qq + 4 h + 0..3 of block t in acc[t][4 qq .. 4 qq + 3].
  v4i* red = reinterpret_cast<v4i*>(a_lds);
#pragma unroll
  for (int t = 0; t < 2; ++t)
#pragma unroll
    for (int qq = 0; qq < 4; ++qq)
      red[(((wave * 2 + t) * 4 + qq) * 2 + frag_half) * 32 + frag_row] =
          v4i{acc[t][4 * qq], acc[t][4 * qq + 1], acc[t][4 * qq + 2], acc[t][4 * qq + 3]};
  __syncthreads();
  // this thread's 8 sums: dequant -> block t = ec / 4, rows 8 (ec % 4) + 0..7
  // (halves 0 and 1); SwiGLU -> rows 4 ec + 0..3 (qq = ec / 2, h = ec % 2) of
  // the gate block (t = 0) and of the up block (t = 1)
  const int t0 = SWIGLU ? 0 : ec / 4, t1 = SWIGLU ? 1 : ec / 4;
  const int qq = SWIGLU ? ec / 2 : ec % 4, h0 = SWIGLU ? ec % 2 : 0, h1 = SWIGLU ? ec % 2 : 1;
  v4i s0 = v4i{0, 0, 0, 0}, s1 = v4i{0, 0, 0, 0};
#pragma unroll
  for (int wv = 0; wv < 4; ++wv) {
    s0 += red[(((wv * 2 + t0) * 4 + qq) * 2 + h0) * 32 + er];
    s1 += red[(((wv * 2 + t1) * 4 + qq) * 2 + h1) * 32 + er];
  }
  const int64_t me = mb + er;
  if (me >= M || !col_live) return;
  const float st = s_rows[er];
  const float sc[8] = {sc0.x, sc0.y, sc0.z, sc0.w, sc1.x, sc1.y, sc1.z, sc1.w};
  float bv[8] = {0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f};
  if (bias) {
    bf16x4(bw0, bv);
    bf16x4(bw1, bv + 4);
  }
  const int32_t sums[8] = {s0[0], s0[1], s0[2], s0[3], s1[0], s1[1], s1[2], s1[3]};
  uint16_t* yrow = y + me * N + n0;
  if constexpr (!SWIGLU) {
    float o[8];
#pragma unroll
    for (int e = 0; e < 8; ++e) o[e] = __builtin_fmaf((float)sums[e], st * sc[e], bv[e]);
    *reinterpret_cast<u32x4*>(yrow) =
        u32x4{bf16x2_rne(o[0], o[1]), bf16x2_rne(o[2], o[3]), bf16x2_rne(o[4], o[5]), bf16x2_rne(o[6], o[7])};
  } else {
    float o[4];
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      const float g = __builtin_fmaf((float)sums[e], st * sc[e], bv[e]);
      const float u = __builtin_fmaf((float)sums[4 + e], st * sc[4 + e], bv[4 + e]);
      o[e] = silu_f32(g) * u;
    }
    *reinterpret_cast<u32x2*>(yrow) = u32x2{bf16x2_rne(o[0], o[1]), bf16x2_rne(o[2], o[3])};
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

// One workgroup of 4 waves per CU (its registers fill the SIMDs): the single
// launch pays off while the tiles fit in one round on the 256 CUs, since every
// tile quantizes its rows again (measured: 298 x 1,024 x 1,024 in 6.8 us per
// call against 14.1 us for the quantizer and GEMM as two launches).
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
