// The whole-path int8 projection without a caller workspace, for callers that
// cannot allocate device memory (code under HIP graph capture, serving loops,
// harnesses that forbid allocation).  The quantized activations and their scales
// -- the workspace of w8a8_linear_packed -- live in a fixed device array of this
// file instead; the kernels are the library's usual ones.
#include <atomic>
#include <mutex>

#include "internal.h"

namespace {

// One array per device (the runtime keeps a copy of a __device__ variable on every
// device the library runs on, until the process ends).
static __device__ __align__(256) uint8_t scratch[W8A8_NOALLOC_MAX_WORKSPACE];

constexpr int kMaxDevices = 64;
std::mutex g_scratch_mu;
std::atomic<uint8_t*> g_scratch[kMaxDevices];

// The device address of this device's copy of `scratch` (resolved once per device,
// with that device current).  In host code the array's name is only a handle for
// the runtime, never an address to pass to a kernel.
w8a8_status scratch_for_current_device(uint8_t** out) {
  int dev = -1;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDevices) {
    (void)hipGetLastError();
    return W8A8_ERR_UNSUPPORTED_DEVICE;
  }
  uint8_t* p = g_scratch[dev].load(std::memory_order_acquire);
  if (!p) {
    std::lock_guard<std::mutex> lock(g_scratch_mu);
    p = g_scratch[dev].load(std::memory_order_relaxed);
    if (!p) {
      void* addr = nullptr;
      if (hipGetSymbolAddress(&addr, HIP_SYMBOL(scratch)) != hipSuccess || !addr) {
        (void)hipGetLastError();
        return W8A8_ERR_LAUNCH;
      }
      p = static_cast<uint8_t*>(addr);
      g_scratch[dev].store(p, std::memory_order_release);
    }
  }
  *out = p;
  return W8A8_OK;
}

}  // namespace

extern "C" w8a8_status w8a8_linear_packed_noalloc(const uint16_t* x, const int8_t* w_packed,
                                                  const float* s_ch, const uint16_t* bias, uint16_t* y,
                                                  int64_t M, int64_t N, int64_t K, int rot_block,
                                                  hipStream_t stream) {
  // the allocating entry point's checks, in its order, with the scratch limit right
  // after the shapes
  w8a8_status st = w8a8::whole_path_shape_checks(M, N, K, rot_block);
  if (st != W8A8_OK || M == 0) return st;
  if (w8a8_workspace_bytes(M, K) > (size_t)W8A8_NOALLOC_MAX_WORKSPACE) return W8A8_ERR_SCRATCH_TOO_SMALL;
  if ((st = w8a8::whole_path_checks(x, w_packed, s_ch, bias, y, M, N, K, rot_block)) != W8A8_OK) return st;
  uint8_t* ws = nullptr;
  if ((st = scratch_for_current_device(&ws)) != W8A8_OK) return st;
  // the quantizer overwrites every code and scale the GEMM reads: nothing to clear
  return w8a8_linear_packed(x, w_packed, s_ch, bias, y, M, N, K, rot_block, ws,
                            (size_t)W8A8_NOALLOC_MAX_WORKSPACE, stream);
}
