// Internal declarations shared by the library's translation units (not installed,
// not part of the C ABI).  Kernel launchers return hipError_t from the launch.
#pragma once

#include <hip/hip_runtime.h>
#include <cstdint>

#include "w8a8.h"

namespace w8a8 {

// Epilogues of the GEMM kernel.
enum class Epi : int { kRawI32 = 0, kDequant = 1, kSwiglu = 2 };

// Epilogues that pair gate rows n with up rows N + n.
constexpr bool paired_epi(Epi e) { return e == Epi::kSwiglu; }

// Packed operand layout: blocks of 32 rows x 64 bytes, block (r / 32, k / 64) at
// byte ((r / 32) * (K / 64) + k / 64) * 2048, row r % 32 of the block at + 64 * (r % 32).
inline int64_t packed_rows(int64_t rows) { return (rows + 31) / 32 * 32; }

// Quantizer: rows of x [M, K] bf16 -> codes [M, K] (int8 or E4M3FN; row-major, or
// packed when `packed`) + fp32 scale [M].
hipError_t launch_quantize(const uint16_t* x, int64_t M, int64_t K, int rot_block, bool fp8,
                           bool packed, void* q, float* s, hipStream_t stream);

// GEMM + epilogue.  a: codes [M, K]; b: codes [Nw, K] (Nw = N, or 2N for SwiGLU),
// each row-major or packed; out: int32 [M, N] or bf16 [M, N].
hipError_t launch_gemm(Epi epi, bool fp8, bool packed_a, bool packed_b, const void* a,
                       const float* s_tok, const void* b, const float* s_ch, const uint16_t* bias,
                       void* out, int64_t M, int64_t N, int64_t K, hipStream_t stream);

// y [M, N] (dense) = bf16(silu(g) * u), g and u bf16 [M, N] with rows ld elements
// apart (N % 8 == 0, ld % 8 == 0).
hipError_t launch_swiglu(const uint16_t* g, const uint16_t* u, int64_t ld, uint16_t* y, int64_t M,
                         int64_t N, hipStream_t stream);

// Single-launch short-input whole path (int8 dequant or SwiGLU): quantizes x
// inside the GEMM kernel; writes the packed codes and the scales to q_ws / s_ws
// like the two-kernel path.  Used when short_path_fits().
constexpr int64_t kShortMaxK = 1024;
constexpr int64_t kShortMaxM = 512;
constexpr int64_t kShortMaxTiles = 256;   // tiles of 32 tokens x 64 weight rows
bool short_path_fits(int64_t M, int64_t N, int64_t K, Epi epi);
hipError_t launch_linear_short(Epi epi, const uint16_t* x, const void* w, bool w_packed,
                               const float* s_ch, const uint16_t* bias, uint16_t* y, int64_t M,
                               int64_t N, int64_t K, int rot_block, void* q_ws, float* s_ws,
                               hipStream_t stream);

// Argument checks of the whole-path entry points except the workspace and the
// device, in the library's order: shapes, rot_block, (M == 0: OK), pointers,
// alignment.
w8a8_status whole_path_checks(const void* x, const void* w, const float* s_ch, const uint16_t* bias,
                              const void* y, int64_t M, int64_t N, int64_t K, int rot_block);
// The shape and rot_block part of those checks alone.
w8a8_status whole_path_shape_checks(int64_t M, int64_t N, int64_t K, int rot_block);

// Row-major codes [rows, K] -> packed layout (K % 64 == 0; padding rows zero).
hipError_t launch_pack_rows(const void* src, int64_t rows, int64_t K, void* dst, hipStream_t stream);

}  // namespace w8a8
