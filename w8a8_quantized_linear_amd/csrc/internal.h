// Internal declarations shared by the library's translation units (not installed,
// not part of the C ABI).  Kernel launchers return hipError_t from the launch.
#pragma once

#include <hip/hip_runtime.h>
#include <cstdint>

namespace w8a8 {

// Epilogues of the GEMM kernel.
enum class Epi : int { kRawI32 = 0, kDequant = 1, kSwiglu = 2 };

// Quantizer: rows of x [M, K] bf16 -> codes [M, K] (int8 or E4M3FN) + fp32 scale [M].
hipError_t launch_quantize(const uint16_t* x, int64_t M, int64_t K, int rot_block, bool fp8,
                           void* q, float* s, hipStream_t stream);

// GEMM + epilogue.  a: codes [M, K]; b: codes [Nw, K] (Nw = N, or 2N for SwiGLU);
// out: int32 [M, N] or bf16 [M, N].
hipError_t launch_gemm(Epi epi, bool fp8, const void* a, const float* s_tok, const void* b,
                       const float* s_ch, const uint16_t* bias, void* out,
                       int64_t M, int64_t N, int64_t K, hipStream_t stream);

}  // namespace w8a8
