// Second step of quantizing the SwiGLU output per token for the next linear
// (the first runs in the gate/up GEMM's epilogue): every 128-column block of a
// row holds codes q_b on its own scale s_b = amax_b / 127; the row's scale is
// s = max_b amax_b / 127 -- the per-token scale of the whole row ("CLEF
// Calibrated INT8 ConvRot" card, notes under the latency table: per-token int8
// activations) -- and each code becomes round-half-even(fl32(q_b * rho_b)) with
// rho_b = fl32(s_b / s) (0 when s = 0).  rho_b <= 1, so no clamp is needed, and
// the block that holds the row's amax (rho = 1) is left as it is.
//
// Design (HBM bound: 1 byte read + 1 byte written per code, in place, plus the
// block amax, N / 32 bytes per row): a workgroup owns one 32-row band of the
// packed layout and 8 consecutive blocks, i.e. 16 blocks of 32 rows x 64 bytes
// = 32 KiB of contiguous codes.  It first reduces its 32 rows' amax (8 lanes
// per row, stride-8 reads of the row's amax) and puts rho of its 32 x 8
// (row, block) pairs in LDS; each thread rewrites eight 16-byte pieces, whose
// loads are issued before the amax reduction (so they overlap it) and before
// any store (the codes are rewritten in place), and each wave instruction
// reads or writes one contiguous kilobyte.
#include "internal.h"
#include "quant_math.h"

namespace w8a8 {
namespace {

typedef unsigned u32x4 __attribute__((ext_vector_type(4)));

constexpr int kBlocksPerGroup = 8;  // 128-column blocks per workgroup

__global__ void __launch_bounds__(256)
requantize_blocks_kernel(uint8_t* __restrict__ codes, const float* __restrict__ amax, int64_t M,
                         int64_t N, int nblk, float* __restrict__ s_out) {
  __shared__ float rho[32][kBlocksPerGroup];
  const int tid = threadIdx.x;
  const int64_t band = blockIdx.x;
  const int group = blockIdx.y;

  // The codes do not depend on the scales: their loads (8 x 16 bytes per
  // thread) are issued first and fly while the row amax is reduced.
  const int64_t kblocks = N / 64;
  const int64_t kb0 = (int64_t)group * 2 * kBlocksPerGroup;
  const int nkb = (int)min<int64_t>(2 * kBlocksPerGroup, kblocks - kb0);
  uint8_t* base = codes + (band * kblocks + kb0) * 2048;
  constexpr int kIters = 2 * kBlocksPerGroup * 2048 / (256 * 16);
  u32x4 v[kIters];
  bool act[kIters];
#pragma unroll
  for (int it = 0; it < kIters; ++it) {
    const int d = it * 256 * 16 + tid * 16;
    act[it] = d < nkb * 2048 && band * 32 + (d % 2048) / 64 < M;
    if (act[it]) v[it] = *reinterpret_cast<const u32x4*>(base + d);
  }

  const int r = tid / 8, sub = tid % 8;
  const int64_t m = band * 32 + r;
  const bool live = m < M;
  const float* am = amax + (live ? m : 0) * nblk;
  float a = 0.0f;
  if (live)
    for (int b = sub; b < nblk; b += 8) a = fmaxf(a, am[b]);
  a = qm::group_max<8>(a);
  const float s = a / 127.0f;  // IEEE division
  if (live && group == 0 && sub == 0) s_out[m] = s;
  const int b = group * kBlocksPerGroup + sub;
  float rh = 0.0f;
  if (live && b < nblk && s > 0.0f) rh = (am[b] / 127.0f) / s;
  rho[r][sub] = rh;
  __syncthreads();

#pragma unroll
  for (int it = 0; it < kIters; ++it) {
    const int d = it * 256 * 16 + tid * 16;
    const float f = rho[(d % 2048) / 64][d / 4096];
    if (!act[it] || f == 1.0f) continue;  // (f == 1: the row's amax block, unchanged)
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      uint32_t o = 0;
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        const float q = (float)(int8_t)((v[it][i] >> (8 * e)) & 0xffu);
        const int k = (int)__builtin_rintf(q * f);
        o |= ((uint32_t)k & 0xffu) << (8 * e);
      }
      v[it][i] = o;
    }
    *reinterpret_cast<u32x4*>(base + d) = v[it];
  }
}

}  // namespace

hipError_t launch_requantize_blocks(uint8_t* codes, const float* amax, int64_t M, int64_t N,
                                    float* s, hipStream_t stream) {
  if (N % 64 != 0) return hipErrorInvalidValue;
  if (M == 0 || N == 0) return hipSuccess;
  const int64_t nblk = (N + 127) / 128;
  const int64_t bands = (M + 31) / 32;
  const int64_t groups = (nblk + kBlocksPerGroup - 1) / kBlocksPerGroup;
  if (bands > 0x7fffffff || groups > 65535 || nblk > 0x7fffffff) return hipErrorInvalidValue;
  hipLaunchKernelGGL(requantize_blocks_kernel, dim3((unsigned)bands, (unsigned)groups), dim3(256), 0, stream,
                     codes, amax, M, N, (int)nblk, s);
  return hipGetLastError();
}

}  // namespace w8a8
