// Calls every C entry point with the argument cases of tests/test_abi.py (bad
// shapes, NULL and misaligned pointers, zero rows, sizes near the limits) under
// AddressSanitizer and UndefinedBehaviorSanitizer.  Pointers are dummies that the
// library must never dereference.  Exit status 0 when every status is as expected.
#include <cstdio>

#include "w8a8.h"

static int failures = 0;
#define EXPECT(call, want)                                                              \
  do {                                                                                  \
    const int got = (int)(call);                                                        \
    if (got != (int)(want)) {                                                           \
      std::fprintf(stderr, "%s:%d: %s -> %d, expected %d\n", __FILE__, __LINE__, #call, \
                   got, (int)(want));                                                   \
      ++failures;                                                                       \
    }                                                                                   \
  } while (0)

int main() {
  void* A = reinterpret_cast<void*>(0x10000);
  void* U = reinterpret_cast<void*>(0x10008);
  auto a16 = static_cast<uint16_t*>(A);
  auto a8 = static_cast<int8_t*>(A);
  auto au8 = static_cast<uint8_t*>(A);
  auto af = static_cast<float*>(A);
  auto ai = static_cast<int32_t*>(A);
  const w8a8_status DEV = W8A8_ERR_UNSUPPORTED_DEVICE;

  for (int s = 0; s < 8; ++s) EXPECT(w8a8_status_string((w8a8_status)s)[0] == 'W', 1);
  EXPECT(w8a8_status_string((w8a8_status)99)[0] == 'W', 1);
  EXPECT(w8a8_packed_bytes(1502, 4096), (size_t)1504 * 4096);
  EXPECT(w8a8_packed_bytes(-3, 4096), 0);
  EXPECT(w8a8_workspace_bytes(1, 128), 32 * 128 + 256);
  EXPECT(w8a8_workspace_bytes(0, 128), 0);
  EXPECT(w8a8_swiglu_quant_workspace_bytes(4, 256, 512), w8a8_workspace_bytes(4, 512) + 4 * 256 * 2);

  EXPECT(w8a8_quantize_act(nullptr, 4, 128, 0, a8, af, nullptr), W8A8_ERR_NULL_POINTER);
  EXPECT(w8a8_quantize_act(a16, -1, 128, 0, a8, af, nullptr), W8A8_ERR_BAD_SHAPE);
  EXPECT(w8a8_quantize_act(a16, 4, 24, 0, a8, af, nullptr), W8A8_ERR_BAD_SHAPE);
  EXPECT(w8a8_quantize_act(a16, 4, 131072 + 32, 0, a8, af, nullptr), W8A8_ERR_BAD_SHAPE);
  EXPECT(w8a8_quantize_act(a16, 4, 128, 64, a8, af, nullptr), W8A8_ERR_BAD_ARGUMENT);
  EXPECT(w8a8_quantize_act(static_cast<uint16_t*>(U), 4, 128, 0, a8, af, nullptr), W8A8_ERR_MISALIGNED);
  EXPECT(w8a8_quantize_act(a16, 0, 128, 0, a8, af, nullptr), W8A8_OK);
  EXPECT(w8a8_quantize_act(a16, 4, 128, 0, a8, af, nullptr), DEV);
  EXPECT(w8a8_quantize_act_fp8_packed(a16, 4, 96, 0, au8, af, nullptr), W8A8_ERR_BAD_SHAPE);
  EXPECT(w8a8_quantize_act_packed(a16, 4, 128, 128, a8, af, nullptr), DEV);

  EXPECT(w8a8_gemm_i32(a8, a8, nullptr, 4, 8, 128, nullptr), W8A8_ERR_NULL_POINTER);
  EXPECT(w8a8_gemm_i32(a8, a8, ai, 4, 8, 64, nullptr), W8A8_ERR_BAD_SHAPE);
  EXPECT(w8a8_gemm_i32_packed(a8, a8, ai, 4, 12, 128, nullptr), W8A8_ERR_BAD_SHAPE);
  EXPECT(w8a8_gemm_i32_packed(a8, a8, ai, 4, 8, 128, nullptr), DEV);
  EXPECT(w8a8_gemm_dequant(a8, af, a8, af, static_cast<uint16_t*>(U), a16, 4, 8, 128, nullptr),
         W8A8_ERR_MISALIGNED);
  EXPECT(w8a8_gemm_dequant(a8, af, a8, af, nullptr, a16, (int64_t)1 << 32, 8, 128, nullptr), W8A8_ERR_BAD_SHAPE);
  EXPECT(w8a8_gemm_swiglu_packed(a8, af, a8, af, nullptr, a16, 4, 8, 128, nullptr), DEV);
  EXPECT(w8a8_fp8_gemm_dequant_packed(au8, af, au8, af, nullptr, a16, 0, 8, 128, nullptr), W8A8_OK);

  const size_t ws = w8a8_workspace_bytes(4, 256);
  EXPECT(w8a8_linear(a16, a8, af, nullptr, a16, 4, 8, 256, 0, nullptr, ws, nullptr), W8A8_ERR_NULL_POINTER);
  EXPECT(w8a8_linear(a16, a8, af, nullptr, a16, 4, 8, 256, 0, A, ws - 1, nullptr), W8A8_ERR_BAD_ARGUMENT);
  EXPECT(w8a8_linear(a16, a8, af, nullptr, a16, 4, 8, 256, 3, A, ws, nullptr), W8A8_ERR_BAD_ARGUMENT);
  EXPECT(w8a8_linear_packed(a16, a8, af, nullptr, a16, 4, 8, 256, 128, A, ws, nullptr), DEV);
  EXPECT(w8a8_gateup_swiglu_packed(nullptr, nullptr, nullptr, nullptr, nullptr, 0, 8, 256, 0, nullptr, 0, nullptr),
         W8A8_OK);
  EXPECT(w8a8_fp8_linear_packed(a16, au8, nullptr, nullptr, a16, 4, 8, 256, 0, A, ws, nullptr),
         W8A8_ERR_NULL_POINTER);

  EXPECT(w8a8_swiglu(a16, a16, 8, a16, 4, 16, nullptr), W8A8_ERR_BAD_SHAPE);
  EXPECT(w8a8_swiglu(a16, a16, 16, a16, 4, 16, nullptr), DEV);
  EXPECT(w8a8_pack_weight(A, 4, 96, A, nullptr), W8A8_ERR_BAD_SHAPE);
  EXPECT(w8a8_pack_weight(A, 4, 128, A, nullptr), DEV);

  const size_t wq = w8a8_swiglu_quant_workspace_bytes(4, 256, 512);
  EXPECT(w8a8_gateup_swiglu_quant_packed(a16, a8, af, nullptr, 4, 256, 512, 0, 128, a8, af, A, wq - 1, nullptr),
         W8A8_ERR_BAD_ARGUMENT);
  EXPECT(w8a8_gateup_swiglu_quant_packed(a16, a8, af, nullptr, 4, 192, 512, 0, 128, a8, af, A, wq, nullptr),
         W8A8_ERR_BAD_SHAPE);
  EXPECT(w8a8_gateup_swiglu_quant_packed(a16, a8, af, nullptr, 4, 256, 512, 0, 128, a8, af, A, wq, nullptr), DEV);

  if (failures) std::fprintf(stderr, "%d unexpected statuses\n", failures);
  else std::printf("all argument checks as expected\n");
  return failures ? 1 : 0;
}
