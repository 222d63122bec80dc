// Measurement aid, not a step of the W8A8 path: the cost of the GEMM's MFMA
// operand reads from LDS (ds_read_b128) under different placements of the
// 16-byte chunks of 64-byte rows.
//
// The operand read: lanes 0-31 of a wave fetch chunk c of 32 consecutive rows,
// lanes 32-63 chunk c + 1 of the same rows.  Chunk c of row r sits at chunk
// position c ^ key(r).  Patterns:
//   0  reference: lane l reads the 16 bytes at 16 l (contiguous, no conflicts);
//   1  operand rows, key 0 (no swizzle);
//   2  operand rows, key ((r >> 1) ^ (r >> 3)) & 3;
//   3  operand rows, key (r ^ (r >> 2)) & 3 (the GEMM's key).
// Each of the 4 waves of a block reads 8 such fragments per iteration (rows
// 64 w + 32 t, chunk pair 2 (t & 1)) from a 16 KiB LDS buffer whose dword i holds
// i, and adds them into its accumulator; each lane writes the sum of its
// accumulator's 4 dwords, which the host can check: iters times the sum of the
// dword indices the lane read.  An opaque zero (a register move the compiler
// cannot see through) is added to every address so that the reads stay in the
// loop.
#include <hip/hip_runtime.h>
#include <cstdint>

namespace {

typedef unsigned v4u __attribute__((ext_vector_type(4)));

constexpr int kThreads = 256;
constexpr int kBytes = 16384;

__device__ __forceinline__ int key_of(int pattern, int r) {
  if (pattern == 2) return ((r >> 1) ^ (r >> 3)) & 3;
  if (pattern == 3) return (r ^ (r >> 2)) & 3;
  return 0;
}

__global__ void __launch_bounds__(kThreads) lds_probe_kernel(int pattern, int iters, int* __restrict__ out) {
  __shared__ __attribute__((aligned(1024))) uint8_t lds[kBytes];
  for (int i = threadIdx.x; i < kBytes / 4; i += kThreads) reinterpret_cast<int*>(lds)[i] = i;
  __syncthreads();
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int frag_row = lane & 31, frag_half = lane >> 5;
  int offs[8];
#pragma unroll
  for (int t = 0; t < 8; ++t) {
    if (pattern == 0) {
      offs[t] = (t * 1024 + lane * 16) % kBytes;
    } else {
      const int row = (wave * 64 + t * 32 + frag_row) % (kBytes / 64);
      const int c = 2 * (t & 1) + frag_half;
      offs[t] = (row * 4 + (c ^ key_of(pattern, row))) * 16;
    }
  }
  v4u acc = {0u, 0u, 0u, 0u};
  for (int it = 0; it < iters; ++it) {
    v4u v[8];
#pragma unroll
    for (int t = 0; t < 8; ++t) {
      int z;
      asm volatile("v_mov_b32 %0, 0" : "=v"(z));
      v[t] = *reinterpret_cast<const v4u*>(lds + offs[t] + z);
    }
#pragma unroll
    for (int t = 0; t < 8; ++t) acc += v[t];
  }
  out[(int64_t)blockIdx.x * kThreads + threadIdx.x] = (int)(acc.x + acc.y + acc.z + acc.w);
}

}  // namespace

// out: blocks * 256 int32 on the device.  Returns 0, or -1 on a bad argument or a
// launch failure.
extern "C" int w8a8_probe_lds(int pattern, int iters, int blocks, int* out, hipStream_t stream) {
  if (!out || pattern < 0 || pattern > 3 || iters < 1 || blocks < 1) return -1;
  hipLaunchKernelGGL(lds_probe_kernel, dim3((unsigned)blocks), dim3(kThreads), 0, stream, pattern, iters, out);
  return hipGetLastError() == hipSuccess ? 0 : -1;
}
