// attn_bwd_noalloc: the backward pass without a caller workspace, for
// callers that cannot allocate device memory (code under HIP graph capture,
// tight serving loops, harnesses that forbid hipMalloc).  The per-window
// table gradients go to a fixed device array of this library, `scratch`,
// instead of a workspace argument; nothing is allocated.
//
// `scratch` is a device symbol: in host code its name is only a stand-in,
// not a device address.  Its address on each device is taken once, with
// that device current, by hipGetSymbolAddress and kept per device; the
// kernels receive that pointer, as they receive the workspace in attn_bwd.
// Every call on a device shares that device's array: calls that overlap on
// one device (different streams, different host threads) race on it.  The
// kernels write every workspace element they read, so nothing needs
// clearing between calls.
#include <hip/hip_runtime.h>

#include <mutex>

#include "../../include/attn.h"
#include "attn_internal.h"

namespace attn {
namespace {

constexpr size_t kScratchBytes = (size_t)16 << 20;  // per device
static __device__ __align__(256) float scratch[kScratchBytes / sizeof(float)];

constexpr int kMaxDevices = 64;
std::mutex g_scratch_mu;
void* g_scratch_ptr[kMaxDevices];  // device address of `scratch`, per device

// The device address of `scratch` on the current device.
int scratch_address(void** out) {
  int dev = -1;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDevices) return ATTN_E_LAUNCH;
  std::lock_guard<std::mutex> lock(g_scratch_mu);
  if (!g_scratch_ptr[dev]) {
    void* p = nullptr;
    if (hipGetSymbolAddress(&p, HIP_SYMBOL(scratch)) != hipSuccess || !p) return ATTN_E_LAUNCH;
    g_scratch_ptr[dev] = p;
  }
  *out = g_scratch_ptr[dev];
  return ATTN_OK;
}

}  // namespace
}  // namespace attn

extern "C" {

ATTN_API int attn_bwd_noalloc(const attn_tensor_t* q, const attn_tensor_t* k, const attn_tensor_t* v,
                              const attn_tensor_t* dout, const attn_bias_desc_t* bias_desc,
                              const attn_mask_desc_t* mask_desc, const attn_tensor_t* dq,
                              const attn_tensor_t* dk, const attn_tensor_t* dv, float* dtable,
                              int32_t dtype, void* stream) {
  attn::AttnBwdArgs ba;
  size_t need = 0;
  int st = attn::validate_bwd(q, k, v, dout, bias_desc, mask_desc, dq, dk, dv, dtable, dtype, &ba, &need,
                              nullptr);
  if (st != ATTN_OK) return st;
  if (need > attn::kScratchBytes) return ATTN_E_UNSUPPORTED;  // beyond the fixed array
  void* ws = nullptr;
  if ((st = attn::scratch_address(&ws)) != ATTN_OK) return st;
  ba.ws = (float*)ws;
  return attn::launch_bwd(ba, stream);
}

}  // extern "C"
