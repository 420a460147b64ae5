// moe_layer_forward_static: the layer call with its workspace in a static
// device array, for callers that cannot allocate device memory (code under
// HIP graph capture, serving loops, harnesses that forbid hipMalloc).
#include <hip/hip_runtime.h>

#include <mutex>

#include "moe.h"
#include "moe_kernels.h"

namespace moe {
moe_status set_error(moe_status code, const char* fmt, ...);
}

namespace {

// One copy per GPU the library runs on, held until the process ends.  In
// host code `scratch` only names the symbol: its device address on the
// current GPU comes from hipGetSymbolAddress.
constexpr size_t kScratchBytes = size_t(MOE_STATIC_SCRATCH_BYTES);
__device__ __align__(256) uint8_t scratch[kScratchBytes];

constexpr int kMaxDevices = 64;
std::mutex g_mu;
void* g_ptr[kMaxDevices] = {};

// Device address of this GPU's scratch array (looked up once per device,
// with that device current).
moe_status scratch_ptr(void** out) {
  int dev = -1;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return moe::set_error(MOE_EHIP, "hipGetDevice: %s", hipGetErrorString(e));
  if (dev < 0 || dev >= kMaxDevices) return moe::set_error(MOE_EINVAL, "device %d beyond %d", dev, kMaxDevices);
  std::lock_guard<std::mutex> lk(g_mu);
  if (g_ptr[dev] == nullptr) {
    void* p = nullptr;
    e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    if (e != hipSuccess || p == nullptr)
      return moe::set_error(MOE_EHIP, "hipGetSymbolAddress(scratch): %s", hipGetErrorString(e));
    g_ptr[dev] = p;
  }
  *out = g_ptr[dev];
  return MOE_OK;
}

}  // namespace

extern "C" moe_status moe_layer_forward_static(const moe_layer_desc* desc, const moe_layer_weights* w, const void* x,
                                               int32_t n_tokens, float* y, int32_t* topk_idx_or_null,
                                               float* topk_w_or_null, float* shared_gate_or_null, moe_stream stream) {
  size_t need = 0;
  moe_status st = moe_workspace_bytes(desc, n_tokens, &need);
  if (st) return st;
  if (need > kScratchBytes)
    return moe::set_error(MOE_EWORKSPACE,
                          "%d tokens need %zu bytes of workspace; the static scratch holds %zu (use "
                          "moe_layer_forward with a workspace)",
                          n_tokens, need, kScratchBytes);
  if (n_tokens == 0) return moe_layer_forward(desc, w, x, 0, y, topk_idx_or_null, topk_w_or_null,
                                              shared_gate_or_null, nullptr, 0, stream);
  void* ws = nullptr;
  if ((st = scratch_ptr(&ws))) return st;
  return moe_layer_forward(desc, w, x, n_tokens, y, topk_idx_or_null, topk_w_or_null, shared_gate_or_null, ws,
                           kScratchBytes, stream);
}
