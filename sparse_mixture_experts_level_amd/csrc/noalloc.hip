// moe_forward_noalloc: the forward pass with its workspace in a fixed device array of the
// library, for callers that cannot allocate device memory (code under HIP graph capture,
// tight serving loops, harnesses that forbid allocation).  Declared in include/moe.h.
#include <hip/hip_runtime.h>

#include <mutex>

#include "moe.h"

namespace {

// Per-GPU scratch of MOE_NOALLOC_WORKSPACE_BYTES.  In host code `scratch` only names the
// symbol: its device address comes from hipGetSymbolAddress, once per device.
__device__ __align__(256) uint8_t scratch[MOE_NOALLOC_WORKSPACE_BYTES];

constexpr int kMaxDevices = 64;
std::mutex g_mu;
void *g_scratch[kMaxDevices];  // device address of `scratch` on each device, once resolved

// The current device's copy of `scratch`, resolved on the first call on that device with
// the device current.
moe_status scratch_of_current_device(void **out, const char **why) {
  int dev = -1;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) {
    *why = hipGetErrorString(e);
    return MOE_ERR_HIP;
  }
  if (dev < 0 || dev >= kMaxDevices) {
    *why = "device index beyond the library's table of scratch arrays";
    return MOE_ERR_UNSUPPORTED;
  }
  std::lock_guard<std::mutex> lock(g_mu);
  if (!g_scratch[dev]) {
    void *p = nullptr;
    e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    if (e != hipSuccess || !p) {
      *why = e != hipSuccess ? hipGetErrorString(e) : "hipGetSymbolAddress returned NULL";
      return MOE_ERR_HIP;
    }
    g_scratch[dev] = p;
  }
  *out = g_scratch[dev];
  return MOE_OK;
}

}  // namespace

namespace moe {
moe_status api_fail(moe_status st, const char *what, const char *detail);
}

extern "C" moe_status moe_forward_noalloc(const moe_desc *desc, const moe_weights *weights, const void *x,
                                          const float *logit_offset, void *out, moe_routing *routing,
                                          hipStream_t stream) {
  const size_t need = moe_workspace_size(desc);
  if (need == 0)  // invalid descriptor: moe_forward reports why, before any HIP call
    return moe_forward(desc, weights, x, logit_offset, out, routing, nullptr, 0, stream);
  if (need > (size_t)MOE_NOALLOC_WORKSPACE_BYTES)
    return moe::api_fail(MOE_ERR_WORKSPACE, "moe_forward_noalloc",
                         "the layer needs more workspace than the library's fixed scratch array "
                         "(MOE_NOALLOC_WORKSPACE_BYTES); use moe_forward with a caller workspace");
  void *ws = nullptr;
  const char *why = "";
  const moe_status st = scratch_of_current_device(&ws, &why);
  if (st != MOE_OK) return moe::api_fail(st, "moe_forward_noalloc: scratch array", why);
  return moe_forward(desc, weights, x, logit_offset, out, routing, ws, MOE_NOALLOC_WORKSPACE_BYTES, stream);
}
