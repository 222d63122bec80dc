// Integer (and E4M3FN) GEMM with fused epilogues for gfx950 (stages 2 and 3 of
// the W8A8 path).
//
// What it computes: acc[m][n] = sum_k a[m][k] * b[n][k] over int8 codes (exact
// int32) or E4M3FN codes (fp32 accumulation), followed in registers by
//   kRawI32 : acc as int32;
//   kDequant: bf16(acc * s_tok[m] * s_ch[n] + bias[n])  -- the scale and bias
//             fusion of the INT8 GEMM epilogue ("CLEF Calibrated INT8 ConvRot"
//             card, Benefits list);
//   kSwiglu : bf16(silu(g) * u) with g, u the dequantized values of packed rows
//             n and N + n -- the paired gate/up epilogue ("Loading CLEF INT8",
//             fuse_mlp; gate/up packed into one weight at load time).
//
// Design: both operands are K-contiguous ("NT"), so MFMA operands load with no
// transpose.  A 256-thread workgroup owns a 128 (tokens) x 128 (weight rows)
// tile; its four waves are arranged 2 x 2 and each accumulates a 64 x 64
// sub-tile with v_mfma_i32_16x16x64_i8.  E4M3FN operands are widened exactly to
// bf16 in registers and go through v_mfma_f32_16x16x32_bf16: the gfx950 fp8
// MFMAs sum groups of products at roughly 14-bit precision (measured: error
// ~2e-4 of the output rms at K = 4096, whatever the instruction width or
// accumulator chaining), which is not the fp32 accumulation the fp8 scheme
// calls for; the bf16 MFMA on the same values is accurate to fp32 rounding.  The weight fragment is the MFMA's A operand
// and the token fragment its B operand, so each lane ends up holding four
// consecutive output columns of one token row (8-byte bf16 stores).  K advances
// 128 bytes per step through two LDS buffers (global loads for step k+1 are in
// flight while step k computes; one barrier per step).  LDS rows are XOR
// swizzled in 16-byte units so the MFMA operand reads are bank-conflict free.
// Rows past M or past the weight's rows are loaded as zeros, which add exact
// zeros to the accumulators.
#include <type_traits>

#include "internal.h"

namespace w8a8 {
namespace {

typedef int v4i __attribute__((ext_vector_type(4)));
typedef int v8i __attribute__((ext_vector_type(8)));
typedef float v4f __attribute__((ext_vector_type(4)));
typedef __bf16 v2bf __attribute__((ext_vector_type(2)));
typedef __bf16 v4bf __attribute__((ext_vector_type(4)));
typedef __bf16 v8bf __attribute__((ext_vector_type(8)));

constexpr int BM = kGemmBM, BN = kGemmBN, BK = kGemmBK;
constexpr int kThreads = 256;
constexpr int kChunksPerRow = BK / 16;                              // 8 x 16 bytes
constexpr int kLoadsPerThread = BM * kChunksPerRow / kThreads;     // 4
constexpr int kTileBytes = BM * BK;                                // 16 KiB

// 16-byte chunk c of LDS row r is stored at chunk position c ^ f(r).
__device__ __forceinline__ int swz(int r, int c) { return (r * kChunksPerRow + (c ^ (r & 7))) * 16; }

// Eight E4M3FN codes -> eight bf16 values (exact: every E4M3FN value, subnormals
// included, is a bf16 value).
__device__ __forceinline__ v8bf e4m3x8_to_bf16(uint2 v) {
  const v2bf p0 = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8((int)v.x, 1.0f, false);
  const v2bf p1 = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8((int)v.x, 1.0f, true);
  const v2bf p2 = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8((int)v.y, 1.0f, false);
  const v2bf p3 = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8((int)v.y, 1.0f, true);
  const v4bf lo = __builtin_shufflevector(p0, p1, 0, 1, 2, 3);
  const v4bf hi = __builtin_shufflevector(p2, p3, 0, 1, 2, 3);
  return __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7);
}

__device__ __forceinline__ uint16_t f32_to_bf16_rne(float f) {
  uint32_t u = __float_as_uint(f);
  u += 0x7fffu + ((u >> 16) & 1u);
  return (uint16_t)(u >> 16);
}

template <Epi EPI>
__device__ __forceinline__ int64_t weight_row(int r, int64_t nb, int64_t N) {
  // LDS weight-tile row r -> global weight row (or -1 if out of range)
  if constexpr (EPI == Epi::kSwiglu) {
    const int64_t col = nb + (r & 63);                 // output column
    if (col >= N) return -1;
    return r < 64 ? col : N + col;                     // gate rows, then up rows
  } else {
    const int64_t n = nb + r;
    return n < N ? n : -1;
  }
}

template <Epi EPI, bool FP8>
__global__ void __launch_bounds__(kThreads)
gemm_tile(const uint8_t* __restrict__ a, const float* __restrict__ s_tok,
          const uint8_t* __restrict__ b, const float* __restrict__ s_ch,
          const uint16_t* __restrict__ bias, void* __restrict__ out,
          int64_t M, int64_t N, int64_t K, int tiles_m) {
  __shared__ __attribute__((aligned(16))) uint8_t lds[2][2][kTileBytes];  // [buf][a|b]

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = tid >> 6;
  const int wm = wave & 1, wn = wave >> 1;
  const int tile_m = blockIdx.x % tiles_m;
  const int tile_n = blockIdx.x / tiles_m;
  const int64_t mb = (int64_t)tile_m * BM;
  // weight-row tile base: kSwiglu tiles cover 64 output columns (128 packed rows)
  const int64_t nb = (EPI == Epi::kSwiglu) ? (int64_t)tile_n * (BN / 2) : (int64_t)tile_n * BN;

  // Per-thread global source rows for the staged loads.
  const uint8_t* a_src[kLoadsPerThread];
  const uint8_t* b_src[kLoadsPerThread];
  int lds_off[kLoadsPerThread];
#pragma unroll
  for (int i = 0; i < kLoadsPerThread; ++i) {
    const int id = tid + i * kThreads;
    const int r = id / kChunksPerRow, c = id % kChunksPerRow;
    const int64_t am = mb + r;
    a_src[i] = am < M ? a + am * K + c * 16 : nullptr;
    const int64_t bn = weight_row<EPI>(r, nb, N);
    b_src[i] = bn >= 0 ? b + bn * K + c * 16 : nullptr;
    lds_off[i] = swz(r, c);
  }

  uint4 ra[kLoadsPerThread], rb[kLoadsPerThread];
  auto gload = [&](int64_t k0) {
#pragma unroll
    for (int i = 0; i < kLoadsPerThread; ++i) {
      ra[i] = a_src[i] ? *reinterpret_cast<const uint4*>(a_src[i] + k0) : make_uint4(0, 0, 0, 0);
      rb[i] = b_src[i] ? *reinterpret_cast<const uint4*>(b_src[i] + k0) : make_uint4(0, 0, 0, 0);
    }
  };
  auto lstore = [&](int buf) {
#pragma unroll
    for (int i = 0; i < kLoadsPerThread; ++i) {
      *reinterpret_cast<uint4*>(&lds[buf][0][lds_off[i]]) = ra[i];
      *reinterpret_cast<uint4*>(&lds[buf][1][lds_off[i]]) = rb[i];
    }
  };

  // Accumulators: [n sub-tile][m sub-tile], 16x16 each.
  using Acc = typename std::conditional<FP8, v4f, v4i>::type;
  Acc acc[4][4];
#pragma unroll
  for (int i = 0; i < 4; ++i)
#pragma unroll
    for (int j = 0; j < 4; ++j) acc[i][j] = Acc{0, 0, 0, 0};

  // LDS rows this lane reads as MFMA operands.
  const int frag_row = lane & 15, frag_grp = lane >> 4;
  int b_rows[4], a_rows[4];
#pragma unroll
  for (int t = 0; t < 4; ++t) {
    a_rows[t] = wm * 64 + t * 16 + frag_row;
    if constexpr (EPI == Epi::kSwiglu)
      b_rows[t] = (t < 2 ? 0 : 64) + wn * 32 + (t & 1) * 16 + frag_row;
    else
      b_rows[t] = wn * 64 + t * 16 + frag_row;
  }

  const int64_t ksteps = K / BK;
  gload(0);
  lstore(0);
  __syncthreads();

  for (int64_t ks = 0; ks < ksteps; ++ks) {
    const int buf = (int)(ks & 1);
    if (ks + 1 < ksteps) gload((ks + 1) * BK);
    const uint8_t* la = lds[buf][0];
    const uint8_t* lb = lds[buf][1];
    if constexpr (FP8) {
      // E4M3FN codes are widened exactly to bf16 in registers and multiplied on
      // the bf16 MFMA, which accumulates in fp32.  Per 32-k sub-block i, lane
      // group g holds k bytes [32g + 8i, +8) of its row.
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        v8bf fa[4], fb[4];
#pragma unroll
        for (int t = 0; t < 4; ++t) {
          const int cb = 2 * frag_grp + (i >> 1), byte = (i & 1) * 8;
          fa[t] = e4m3x8_to_bf16(*reinterpret_cast<const uint2*>(la + swz(a_rows[t], cb) + byte));
          fb[t] = e4m3x8_to_bf16(*reinterpret_cast<const uint2*>(lb + swz(b_rows[t], cb) + byte));
        }
#pragma unroll
        for (int tn = 0; tn < 4; ++tn)
#pragma unroll
          for (int tm = 0; tm < 4; ++tm)
            acc[tn][tm] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(fb[tn], fa[tm], acc[tn][tm], 0, 0, 0);
      }
    } else {
#pragma unroll
      for (int kk = 0; kk < 2; ++kk) {
        // lane group g holds k bytes [64kk + 16g, +16)
        v4i fa[4], fb[4];
#pragma unroll
        for (int t = 0; t < 4; ++t) {
          const uint4 av = *reinterpret_cast<const uint4*>(la + swz(a_rows[t], 4 * kk + frag_grp));
          const uint4 bv = *reinterpret_cast<const uint4*>(lb + swz(b_rows[t], 4 * kk + frag_grp));
          fa[t] = v4i{(int)av.x, (int)av.y, (int)av.z, (int)av.w};
          fb[t] = v4i{(int)bv.x, (int)bv.y, (int)bv.z, (int)bv.w};
        }
#pragma unroll
        for (int tn = 0; tn < 4; ++tn)
#pragma unroll
          for (int tm = 0; tm < 4; ++tm)
            acc[tn][tm] = __builtin_amdgcn_mfma_i32_16x16x64_i8(fb[tn], fa[tm], acc[tn][tm], 0, 0, 0);
      }
    }
    if (ks + 1 < ksteps) lstore(buf ^ 1);
    __syncthreads();
  }

  // ---- epilogue: lane holds rows n = 4*(lane/16) + v (v = 0..3), column m = lane % 16
  const int n_in = 4 * frag_grp;
#pragma unroll
  for (int tm = 0; tm < 4; ++tm) {
    const int64_t m = mb + wm * 64 + tm * 16 + frag_row;
    if (m >= M) continue;
    if constexpr (EPI == Epi::kRawI32) {
#pragma unroll
      for (int tn = 0; tn < 4; ++tn) {
        const int64_t n0 = nb + wn * 64 + tn * 16 + n_in;
        if (n0 >= N) continue;
        const v4i v = reinterpret_cast<const v4i&>(acc[tn][tm]);
        *reinterpret_cast<int4*>(static_cast<int32_t*>(out) + m * N + n0) = make_int4(v.x, v.y, v.z, v.w);
      }
    } else {
      const float st = s_tok[m];
      uint16_t* yrow = static_cast<uint16_t*>(out) + m * N;
      if constexpr (EPI == Epi::kDequant) {
#pragma unroll
        for (int tn = 0; tn < 4; ++tn) {
          const int64_t n0 = nb + wn * 64 + tn * 16 + n_in;
          if (n0 >= N) continue;
          const float4 sc = *reinterpret_cast<const float4*>(s_ch + n0);
          float bv[4] = {0.f, 0.f, 0.f, 0.f};
          if (bias) {
            const uint2 bb = *reinterpret_cast<const uint2*>(bias + n0);
            bv[0] = __uint_as_float(bb.x << 16);
            bv[1] = __uint_as_float(bb.x & 0xffff0000u);
            bv[2] = __uint_as_float(bb.y << 16);
            bv[3] = __uint_as_float(bb.y & 0xffff0000u);
          }
          const float scv[4] = {sc.x, sc.y, sc.z, sc.w};
          uint16_t o[4];
#pragma unroll
          for (int v = 0; v < 4; ++v) {
            const float av = (float)acc[tn][tm][v];
            o[v] = f32_to_bf16_rne(__builtin_fmaf(av, st * scv[v], bv[v]));
          }
          *reinterpret_cast<uint2*>(yrow + n0) =
              make_uint2((uint32_t)o[0] | ((uint32_t)o[1] << 16), (uint32_t)o[2] | ((uint32_t)o[3] << 16));
        }
      } else {  // kSwiglu: sub-tiles 0,1 are gate, 2,3 the matching up rows
#pragma unroll
        for (int tn = 0; tn < 2; ++tn) {
          const int64_t n0 = nb + wn * 32 + tn * 16 + n_in;  // output column
          if (n0 >= N) continue;
          const float4 sg = *reinterpret_cast<const float4*>(s_ch + n0);
          const float4 su = *reinterpret_cast<const float4*>(s_ch + N + n0);
          float bg[4] = {0.f, 0.f, 0.f, 0.f}, bu[4] = {0.f, 0.f, 0.f, 0.f};
          if (bias) {
            const uint2 b0 = *reinterpret_cast<const uint2*>(bias + n0);
            const uint2 b1 = *reinterpret_cast<const uint2*>(bias + N + n0);
            bg[0] = __uint_as_float(b0.x << 16); bg[1] = __uint_as_float(b0.x & 0xffff0000u);
            bg[2] = __uint_as_float(b0.y << 16); bg[3] = __uint_as_float(b0.y & 0xffff0000u);
            bu[0] = __uint_as_float(b1.x << 16); bu[1] = __uint_as_float(b1.x & 0xffff0000u);
            bu[2] = __uint_as_float(b1.y << 16); bu[3] = __uint_as_float(b1.y & 0xffff0000u);
          }
          const float sgv[4] = {sg.x, sg.y, sg.z, sg.w}, suv[4] = {su.x, su.y, su.z, su.w};
          uint16_t o[4];
#pragma unroll
          for (int v = 0; v < 4; ++v) {
            const float g = __builtin_fmaf((float)acc[tn][tm][v], st * sgv[v], bg[v]);
            const float u = __builtin_fmaf((float)acc[tn + 2][tm][v], st * suv[v], bu[v]);
            const float silu = g / (1.0f + __expf(-g));
            o[v] = f32_to_bf16_rne(silu * u);
          }
          *reinterpret_cast<uint2*>(yrow + n0) =
              make_uint2((uint32_t)o[0] | ((uint32_t)o[1] << 16), (uint32_t)o[2] | ((uint32_t)o[3] << 16));
        }
      }
    }
  }
}

template <Epi EPI, bool FP8>
hipError_t launch_t(const void* a, const float* s_tok, const void* b, const float* s_ch,
                    const uint16_t* bias, void* out, int64_t M, int64_t N, int64_t K,
                    hipStream_t stream) {
  const int64_t tiles_m = (M + BM - 1) / BM;
  const int64_t cols_per_tile = (EPI == Epi::kSwiglu) ? BN / 2 : BN;
  const int64_t tiles_n = (N + cols_per_tile - 1) / cols_per_tile;
  const int64_t blocks = tiles_m * tiles_n;
  if (blocks > 0x7fffffff) return hipErrorInvalidValue;
  hipLaunchKernelGGL((gemm_tile<EPI, FP8>), dim3((unsigned)blocks), dim3(kThreads), 0, stream,
                     static_cast<const uint8_t*>(a), s_tok, static_cast<const uint8_t*>(b), s_ch, bias,
                     out, M, N, K, (int)tiles_m);
  return hipGetLastError();
}

}  // namespace

hipError_t launch_gemm(Epi epi, bool fp8, const void* a, const float* s_tok, const void* b,
                       const float* s_ch, const uint16_t* bias, void* out,
                       int64_t M, int64_t N, int64_t K, hipStream_t stream) {
  if (fp8) {
    if (epi == Epi::kDequant) return launch_t<Epi::kDequant, true>(a, s_tok, b, s_ch, bias, out, M, N, K, stream);
    return hipErrorInvalidValue;
  }
  switch (epi) {
    case Epi::kRawI32: return launch_t<Epi::kRawI32, false>(a, s_tok, b, s_ch, bias, out, M, N, K, stream);
    case Epi::kDequant: return launch_t<Epi::kDequant, false>(a, s_tok, b, s_ch, bias, out, M, N, K, stream);
    case Epi::kSwiglu: return launch_t<Epi::kSwiglu, false>(a, s_tok, b, s_ch, bias, out, M, N, K, stream);
  }
  return hipErrorInvalidValue;
}

}  // namespace w8a8
