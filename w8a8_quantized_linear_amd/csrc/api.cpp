// Host side of the C ABI declared in include/w8a8.h: argument validation,
// device check, workspace layout and kernel dispatch.  Every check runs before
// any HIP call that could enqueue work; nothing here allocates or synchronizes.
#include "w8a8.h"

#include <atomic>
#include <cstring>

#include "internal.h"

namespace {

constexpr int kMaxDevices = 64;
// 0 = unknown, 1 = gfx950, 2 = other
std::atomic<int> g_arch_ok[kMaxDevices];

bool aligned16(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }
size_t align256(size_t v) { return (v + 255u) & ~size_t(255u); }

w8a8_status check_device() {
  int dev = -1;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0) {
    (void)hipGetLastError();
    return W8A8_ERR_UNSUPPORTED_DEVICE;
  }
  if (dev >= kMaxDevices) return W8A8_ERR_UNSUPPORTED_DEVICE;
  int state = g_arch_ok[dev].load(std::memory_order_acquire);
  if (state == 0) {
    hipDeviceProp_t prop;
    if (hipGetDeviceProperties(&prop, dev) != hipSuccess) {
      (void)hipGetLastError();
      return W8A8_ERR_UNSUPPORTED_DEVICE;
    }
    state = (std::strncmp(prop.gcnArchName, "gfx950", 6) == 0) ? 1 : 2;
    g_arch_ok[dev].store(state, std::memory_order_release);
  }
  return state == 1 ? W8A8_OK : W8A8_ERR_UNSUPPORTED_DEVICE;
}

w8a8_status launched(hipError_t e) { return e == hipSuccess ? W8A8_OK : W8A8_ERR_LAUNCH; }

// Shape rules shared by the GEMM entry points.
w8a8_status check_gemm_shape(int64_t M, int64_t N, int64_t K) {
  if (M < 0 || N < 1 || K < 1) return W8A8_ERR_BAD_SHAPE;
  if (K > W8A8_MAX_K || K % 128 != 0 || N % 8 != 0) return W8A8_ERR_BAD_SHAPE;
  if (M > (int64_t)1 << 31 || N > (int64_t)1 << 30) return W8A8_ERR_BAD_SHAPE;
  return W8A8_OK;
}

// Order of the checks everywhere: shapes and scalar arguments, then (for M > 0)
// pointers and alignment, then the device.  M == 0 touches no memory, so it is
// OK with any pointers once the shapes are legal.
w8a8_status quantize(const uint16_t* x, int64_t M, int64_t K, int rot_block, bool fp8, bool packed,
                     void* q, float* s, hipStream_t stream) {
  if (M < 0 || K < 32 || K > W8A8_MAX_K || K % 32 != 0 || M > (int64_t)1 << 31) return W8A8_ERR_BAD_SHAPE;
  if (packed && K % 64 != 0) return W8A8_ERR_BAD_SHAPE;
  if (rot_block != 0 && rot_block != 128) return W8A8_ERR_BAD_ARGUMENT;
  if (rot_block == 128 && K % 128 != 0) return W8A8_ERR_BAD_SHAPE;
  if (M == 0) return W8A8_OK;
  if (!x || !q || !s) return W8A8_ERR_NULL_POINTER;
  if (!aligned16(x) || !aligned16(q) || !aligned16(s)) return W8A8_ERR_MISALIGNED;
  w8a8_status st;
  if ((st = check_device()) != W8A8_OK) return st;
  return launched(w8a8::launch_quantize(x, M, K, rot_block, fp8, packed, q, s, stream));
}

w8a8_status gemm_epilogue(w8a8::Epi epi, bool fp8, bool packed, const void* q, const float* s_tok,
                          const void* w, const float* s_ch, const uint16_t* bias, void* y, int64_t M,
                          int64_t N, int64_t K, hipStream_t stream) {
  const bool needs_scales = epi != w8a8::Epi::kRawI32;
  w8a8_status st = check_gemm_shape(M, N, K);
  if (st != W8A8_OK) return st;
  if (M == 0) return W8A8_OK;
  if (!q || !w || !y || (needs_scales && (!s_tok || !s_ch))) return W8A8_ERR_NULL_POINTER;
  if (!aligned16(q) || !aligned16(w) || !aligned16(y) || (bias && !aligned16(bias)) ||
      (needs_scales && (!aligned16(s_tok) || !aligned16(s_ch))))
    return W8A8_ERR_MISALIGNED;
  if ((st = check_device()) != W8A8_OK) return st;
  return launched(w8a8::launch_gemm(epi, fp8, packed, packed, q, s_tok, w, s_ch, bias, y, M, N, K, stream));
}

}  // namespace

namespace w8a8 {

w8a8_status whole_path_shape_checks(int64_t M, int64_t N, int64_t K, int rot_block) {
  w8a8_status st = check_gemm_shape(M, N, K);
  if (st != W8A8_OK) return st;
  if (rot_block != 0 && rot_block != 128) return W8A8_ERR_BAD_ARGUMENT;
  return W8A8_OK;
}

w8a8_status whole_path_checks(const void* x, const void* w, const float* s_ch, const uint16_t* bias,
                              const void* y, int64_t M, int64_t N, int64_t K, int rot_block) {
  w8a8_status st = whole_path_shape_checks(M, N, K, rot_block);
  if (st != W8A8_OK) return st;
  if (M == 0) return W8A8_OK;
  if (!x || !w || !s_ch || !y) return W8A8_ERR_NULL_POINTER;
  if (!aligned16(x) || !aligned16(w) || !aligned16(s_ch) || !aligned16(y) || (bias && !aligned16(bias)))
    return W8A8_ERR_MISALIGNED;
  return W8A8_OK;
}

}  // namespace w8a8

namespace {

// Whole path: quantize x into the workspace (packed layout), then the GEMM +
// epilogue against a row-major or packed weight.
w8a8_status whole_path(w8a8::Epi epi, bool fp8, bool w_packed, const uint16_t* x, const void* w,
                       const float* s_ch,
                       const uint16_t* bias, uint16_t* y, int64_t M, int64_t N, int64_t K,
                       int rot_block, void* workspace, size_t workspace_bytes, hipStream_t stream) {
  w8a8_status st = check_gemm_shape(M, N, K);
  if (st != W8A8_OK) return st;
  if (rot_block != 0 && rot_block != 128) return W8A8_ERR_BAD_ARGUMENT;
  if (M == 0) return W8A8_OK;
  if (workspace_bytes < w8a8_workspace_bytes(M, K)) return W8A8_ERR_BAD_ARGUMENT;
  if (!workspace) return W8A8_ERR_NULL_POINTER;
  if (!aligned16(workspace)) return W8A8_ERR_MISALIGNED;
  if ((st = w8a8::whole_path_checks(x, w, s_ch, bias, y, M, N, K, rot_block)) != W8A8_OK) return st;
  if ((st = check_device()) != W8A8_OK) return st;
  uint8_t* q = static_cast<uint8_t*>(workspace);
  float* s_tok = reinterpret_cast<float*>(q + align256(w8a8_packed_bytes(M, K)));
  // short batches: one kernel quantizes inside the GEMM (same codes, scales and outputs)
  if (!fp8 && w8a8::short_path_fits(M, N, K, epi))
    return launched(w8a8::launch_linear_short(epi, x, w, w_packed, s_ch, bias, y, M, N, K, rot_block, q,
                                              s_tok, stream));
  st = launched(w8a8::launch_quantize(x, M, K, rot_block, fp8, /*packed=*/true, q, s_tok, stream));
  if (st != W8A8_OK) return st;
  return launched(w8a8::launch_gemm(epi, fp8, /*packed_a=*/true, w_packed, q, s_tok, w, s_ch, bias, y,
                                    M, N, K, stream));
}

// The SwiGLU output quantized for the next linear: shape rules on top of the
// gate/up GEMM's (the output rows are the next linear's activations: N % 64 == 0
// for their packed layout, N % 128 == 0 when they are rotated).
w8a8_status check_swiglu_quant(int64_t M, int64_t N, int64_t K, int rot_in, int rot_out) {
  w8a8_status st = check_gemm_shape(M, N, K);
  if (st != W8A8_OK) return st;
  if (N % 64 != 0 || N > W8A8_MAX_K) return W8A8_ERR_BAD_SHAPE;
  if ((rot_in != 0 && rot_in != 128) || (rot_out != 0 && rot_out != 128)) return W8A8_ERR_BAD_ARGUMENT;
  if (rot_out == 128 && N % 128 != 0) return W8A8_ERR_BAD_SHAPE;
  return W8A8_OK;
}

}  // namespace

extern "C" {

const char* w8a8_status_string(w8a8_status s) {
  switch (s) {
    case W8A8_OK: return "W8A8_OK";
    case W8A8_ERR_NULL_POINTER: return "W8A8_ERR_NULL_POINTER: a required pointer is NULL";
    case W8A8_ERR_BAD_SHAPE: return "W8A8_ERR_BAD_SHAPE: M, N or K outside the supported range";
    case W8A8_ERR_MISALIGNED: return "W8A8_ERR_MISALIGNED: a pointer is not 16-byte aligned";
    case W8A8_ERR_BAD_ARGUMENT: return "W8A8_ERR_BAD_ARGUMENT: rot_block not 0/128 or workspace too small";
    case W8A8_ERR_UNSUPPORTED_DEVICE: return "W8A8_ERR_UNSUPPORTED_DEVICE: no gfx950 HIP device is current";
    case W8A8_ERR_LAUNCH: return "W8A8_ERR_LAUNCH: kernel launch failed";
    case W8A8_ERR_SCRATCH_TOO_SMALL:
      return "W8A8_ERR_SCRATCH_TOO_SMALL: the call needs more than the library's fixed scratch buffer "
             "(W8A8_NOALLOC_MAX_WORKSPACE bytes); use the entry point that takes a workspace";
  }
  return "W8A8 unknown status";
}

size_t w8a8_packed_bytes(int64_t rows, int64_t K) {
  if (rows <= 0 || K <= 0) return 0;
  return (size_t)w8a8::packed_rows(rows) * (size_t)K;
}

size_t w8a8_workspace_bytes(int64_t M, int64_t K) {
  if (M <= 0 || K <= 0) return 0;
  return align256(w8a8_packed_bytes(M, K)) + align256((size_t)M * sizeof(float));
}

size_t w8a8_swiglu_quant_workspace_bytes(int64_t M, int64_t N, int64_t K) {
  if (M <= 0 || N <= 0 || K <= 0) return 0;
  return w8a8_workspace_bytes(M, K) + align256((size_t)M * (size_t)N * sizeof(uint16_t));
}

w8a8_status w8a8_pack_weight(const void* w, int64_t rows, int64_t K, void* w_packed,
                             hipStream_t stream) {
  if (rows < 0 || K < 64 || K > W8A8_MAX_K || K % 64 != 0 || rows > (int64_t)1 << 31)
    return W8A8_ERR_BAD_SHAPE;
  if (rows == 0) return W8A8_OK;
  if (!w || !w_packed) return W8A8_ERR_NULL_POINTER;
  if (!aligned16(w) || !aligned16(w_packed)) return W8A8_ERR_MISALIGNED;
  w8a8_status st;
  if ((st = check_device()) != W8A8_OK) return st;
  return launched(w8a8::launch_pack_rows(w, rows, K, w_packed, stream));
}

w8a8_status w8a8_swiglu(const uint16_t* gate, const uint16_t* up, int64_t ld, uint16_t* y, int64_t M,
                        int64_t N, hipStream_t stream) {
  if (M < 0 || N < 8 || N % 8 != 0 || ld < N || ld % 8 != 0 || M > (int64_t)1 << 31 ||
      N > (int64_t)1 << 30)
    return W8A8_ERR_BAD_SHAPE;
  if (M == 0) return W8A8_OK;
  if (!gate || !up || !y) return W8A8_ERR_NULL_POINTER;
  if (!aligned16(gate) || !aligned16(up) || !aligned16(y)) return W8A8_ERR_MISALIGNED;
  w8a8_status st;
  if ((st = check_device()) != W8A8_OK) return st;
  return launched(w8a8::launch_swiglu(gate, up, ld, y, M, N, stream));
}

w8a8_status w8a8_quantize_act(const uint16_t* x, int64_t M, int64_t K, int rot_block, int8_t* q,
                              float* s_tok, hipStream_t stream) {
  return quantize(x, M, K, rot_block, false, false, q, s_tok, stream);
}

w8a8_status w8a8_quantize_act_fp8(const uint16_t* x, int64_t M, int64_t K, int rot_block,
                                  uint8_t* q, float* s_tok, hipStream_t stream) {
  return quantize(x, M, K, rot_block, true, false, q, s_tok, stream);
}

w8a8_status w8a8_quantize_act_packed(const uint16_t* x, int64_t M, int64_t K, int rot_block,
                                     int8_t* q_packed, float* s_tok, hipStream_t stream) {
  return quantize(x, M, K, rot_block, false, true, q_packed, s_tok, stream);
}

w8a8_status w8a8_quantize_act_fp8_packed(const uint16_t* x, int64_t M, int64_t K, int rot_block,
                                         uint8_t* q_packed, float* s_tok, hipStream_t stream) {
  return quantize(x, M, K, rot_block, true, true, q_packed, s_tok, stream);
}

w8a8_status w8a8_gemm_i32(const int8_t* q, const int8_t* w, int32_t* acc, int64_t M, int64_t N,
                          int64_t K, hipStream_t stream) {
  return gemm_epilogue(w8a8::Epi::kRawI32, false, false, q, nullptr, w, nullptr, nullptr, acc, M, N, K, stream);
}

w8a8_status w8a8_gemm_i32_packed(const int8_t* q_packed, const int8_t* w_packed, int32_t* acc, int64_t M,
                                 int64_t N, int64_t K, hipStream_t stream) {
  return gemm_epilogue(w8a8::Epi::kRawI32, false, true, q_packed, nullptr, w_packed, nullptr, nullptr, acc, M, N,
                       K, stream);
}

w8a8_status w8a8_gemm_dequant(const int8_t* q, const float* s_tok, const int8_t* w, const float* s_ch,
                              const uint16_t* bias, uint16_t* y, int64_t M, int64_t N, int64_t K,
                              hipStream_t stream) {
  return gemm_epilogue(w8a8::Epi::kDequant, false, false, q, s_tok, w, s_ch, bias, y, M, N, K, stream);
}

w8a8_status w8a8_gemm_swiglu(const int8_t* q, const float* s_tok, const int8_t* w_gateup,
                             const float* s_ch, const uint16_t* bias, uint16_t* y, int64_t M,
                             int64_t N, int64_t K, hipStream_t stream) {
  return gemm_epilogue(w8a8::Epi::kSwiglu, false, false, q, s_tok, w_gateup, s_ch, bias, y, M, N, K, stream);
}

w8a8_status w8a8_fp8_gemm_dequant(const uint8_t* q, const float* s_tok, const uint8_t* w,
                                  const float* s_ch, const uint16_t* bias, uint16_t* y, int64_t M,
                                  int64_t N, int64_t K, hipStream_t stream) {
  return gemm_epilogue(w8a8::Epi::kDequant, true, false, q, s_tok, w, s_ch, bias, y, M, N, K, stream);
}

w8a8_status w8a8_gemm_dequant_packed(const int8_t* q_packed, const float* s_tok, const int8_t* w_packed,
                                     const float* s_ch, const uint16_t* bias, uint16_t* y, int64_t M,
                                     int64_t N, int64_t K, hipStream_t stream) {
  return gemm_epilogue(w8a8::Epi::kDequant, false, true, q_packed, s_tok, w_packed, s_ch, bias, y, M, N,
                       K, stream);
}

w8a8_status w8a8_gemm_swiglu_packed(const int8_t* q_packed, const float* s_tok,
                                    const int8_t* w_gateup_packed, const float* s_ch,
                                    const uint16_t* bias, uint16_t* y, int64_t M, int64_t N, int64_t K,
                                    hipStream_t stream) {
  return gemm_epilogue(w8a8::Epi::kSwiglu, false, true, q_packed, s_tok, w_gateup_packed, s_ch, bias, y,
                       M, N, K, stream);
}

w8a8_status w8a8_fp8_gemm_dequant_packed(const uint8_t* q_packed, const float* s_tok,
                                         const uint8_t* w_packed, const float* s_ch,
                                         const uint16_t* bias, uint16_t* y, int64_t M, int64_t N,
                                         int64_t K, hipStream_t stream) {
  return gemm_epilogue(w8a8::Epi::kDequant, true, true, q_packed, s_tok, w_packed, s_ch, bias, y, M, N,
                       K, stream);
}

w8a8_status w8a8_linear(const uint16_t* x, const int8_t* w, const float* s_ch, const uint16_t* bias,
                        uint16_t* y, int64_t M, int64_t N, int64_t K, int rot_block, void* workspace,
                        size_t workspace_bytes, hipStream_t stream) {
  return whole_path(w8a8::Epi::kDequant, false, false, x, w, s_ch, bias, y, M, N, K, rot_block, workspace,
                    workspace_bytes, stream);
}

w8a8_status w8a8_gateup_swiglu(const uint16_t* x, const int8_t* w_gateup, const float* s_ch,
                               const uint16_t* bias, uint16_t* y, int64_t M, int64_t N, int64_t K,
                               int rot_block, void* workspace, size_t workspace_bytes,
                               hipStream_t stream) {
  return whole_path(w8a8::Epi::kSwiglu, false, false, x, w_gateup, s_ch, bias, y, M, N, K, rot_block,
                    workspace, workspace_bytes, stream);
}

w8a8_status w8a8_fp8_linear(const uint16_t* x, const uint8_t* w, const float* s_ch,
                            const uint16_t* bias, uint16_t* y, int64_t M, int64_t N, int64_t K,
                            int rot_block, void* workspace, size_t workspace_bytes,
                            hipStream_t stream) {
  return whole_path(w8a8::Epi::kDequant, true, false, x, w, s_ch, bias, y, M, N, K, rot_block, workspace,
                    workspace_bytes, stream);
}

w8a8_status w8a8_linear_packed(const uint16_t* x, const int8_t* w_packed, const float* s_ch,
                               const uint16_t* bias, uint16_t* y, int64_t M, int64_t N, int64_t K,
                               int rot_block, void* workspace, size_t workspace_bytes,
                               hipStream_t stream) {
  return whole_path(w8a8::Epi::kDequant, false, true, x, w_packed, s_ch, bias, y, M, N, K, rot_block,
                    workspace, workspace_bytes, stream);
}

w8a8_status w8a8_gateup_swiglu_packed(const uint16_t* x, const int8_t* w_gateup_packed,
                                      const float* s_ch, const uint16_t* bias, uint16_t* y, int64_t M,
                                      int64_t N, int64_t K, int rot_block, void* workspace,
                                      size_t workspace_bytes, hipStream_t stream) {
  return whole_path(w8a8::Epi::kSwiglu, false, true, x, w_gateup_packed, s_ch, bias, y, M, N, K,
                    rot_block, workspace, workspace_bytes, stream);
}

w8a8_status w8a8_fp8_linear_packed(const uint16_t* x, const uint8_t* w_packed, const float* s_ch,
                                   const uint16_t* bias, uint16_t* y, int64_t M, int64_t N, int64_t K,
                                   int rot_block, void* workspace, size_t workspace_bytes,
                                   hipStream_t stream) {
  return whole_path(w8a8::Epi::kDequant, true, true, x, w_packed, s_ch, bias, y, M, N, K, rot_block,
                    workspace, workspace_bytes, stream);
}

w8a8_status w8a8_gateup_swiglu_quant_packed(const uint16_t* x, const int8_t* w_gateup_packed,
                                            const float* s_ch, const uint16_t* bias, int64_t M,
                                            int64_t N, int64_t K, int rot_in, int rot_out,
                                            int8_t* q_packed, float* s_tok, void* workspace,
                                            size_t workspace_bytes, hipStream_t stream) {
  w8a8_status st = check_swiglu_quant(M, N, K, rot_in, rot_out);
  if (st != W8A8_OK) return st;
  if (M == 0) return W8A8_OK;
  if (workspace_bytes < w8a8_swiglu_quant_workspace_bytes(M, N, K)) return W8A8_ERR_BAD_ARGUMENT;
  if (!x || !w_gateup_packed || !s_ch || !q_packed || !s_tok || !workspace) return W8A8_ERR_NULL_POINTER;
  if (!aligned16(x) || !aligned16(w_gateup_packed) || !aligned16(s_ch) || !aligned16(q_packed) ||
      !aligned16(s_tok) || !aligned16(workspace) || (bias && !aligned16(bias)))
    return W8A8_ERR_MISALIGNED;
  if ((st = check_device()) != W8A8_OK) return st;
  // workspace: x codes (packed) | x scales | the bf16 SwiGLU output h [M, N]
  uint8_t* qx = static_cast<uint8_t*>(workspace);
  float* s_x = reinterpret_cast<float*>(qx + align256(w8a8_packed_bytes(M, K)));
  uint16_t* h = reinterpret_cast<uint16_t*>(reinterpret_cast<uint8_t*>(s_x) + align256((size_t)M * sizeof(float)));
  st = launched(w8a8::launch_quantize(x, M, K, rot_in, false, /*packed=*/true, qx, s_x, stream));
  if (st != W8A8_OK) return st;
  st = launched(w8a8::launch_gemm(w8a8::Epi::kSwiglu, false, /*packed_a=*/true, /*packed_b=*/true, qx, s_x,
                                  w_gateup_packed, s_ch, bias, h, M, N, K, stream));
  if (st != W8A8_OK) return st;
  return launched(w8a8::launch_quantize(h, M, N, rot_out, false, /*packed=*/true, q_packed, s_tok, stream));
}

}  // extern "C"
