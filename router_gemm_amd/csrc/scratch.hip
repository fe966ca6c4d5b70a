// scratch.hip -- moe_forward_noalloc: moe_forward for callers that cannot
// allocate (code under HIP graph capture, tight serving loops), with its
// scratch memory in a library-owned device array instead of a caller
// workspace.
//
// The array is a file-scope __device__ variable: every GPU the library runs on
// holds its own copy, at its own address, until the process ends.  Its name in
// host code is only a stand-in for the symbol, so the device address is looked
// up with hipGetSymbolAddress, once per device with that device current, and
// only that address is ever handed to kernels.  The forward reads nothing from
// its workspace that it has not written in the same call, so nothing needs
// clearing between calls; calls that overlap on one GPU share the array and
// race.

#include <hip/hip_runtime.h>

#include <cstdio>
#include <mutex>

#include "../../include/moe.h"
#include "moe_kernels.h"

namespace {

constexpr size_t kScratchBytes = size_t(64) << 20;   // MOE_NOALLOC_SCRATCH_BYTES
static_assert(kScratchBytes == MOE_NOALLOC_SCRATCH_BYTES, "header and library disagree on the scratch size");

__device__ __align__(256) uint8_t scratch[kScratchBytes];

constexpr int kMaxDevices = 64;
std::mutex g_mu;
void *g_scratch_ptr[kMaxDevices];   // device address of `scratch` on each device (null: not looked up yet)

// The current device's address of `scratch` (looked up on the first call on
// that device), or null with the failure recorded.
void *device_scratch(moe_status *st) {
  int dev = -1;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) {
    *st = moe::api_error(MOE_EHIP, "moe_forward_noalloc: hipGetDevice failed");
    return nullptr;
  }
  if (dev < 0 || dev >= kMaxDevices) {
    *st = moe::api_error(MOE_EUNSUPPORTED, "moe_forward_noalloc: device index beyond the 64 the library tracks");
    return nullptr;
  }
  std::lock_guard<std::mutex> g(g_mu);
  if (!g_scratch_ptr[dev]) {
    void *p = nullptr;
    e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    if (e != hipSuccess || !p) {
      char msg[160];
      snprintf(msg, sizeof msg, "moe_forward_noalloc: hipGetSymbolAddress of the scratch array failed: %s",
               hipGetErrorString(e));
      *st = moe::api_error(MOE_EHIP, msg);
      return nullptr;
    }
    g_scratch_ptr[dev] = p;
  }
  return g_scratch_ptr[dev];
}

}  // namespace

extern "C" moe_status moe_forward_noalloc(const moe_layer *layer, const void *x, int64_t T, void *y,
                                          int32_t out_dtype, int32_t *topk_ids, float *topk_gates, void *stream) {
  // sizes first, on the host: a call too large for the array is refused
  // before the device is touched
  const size_t need = moe::forward_ws_bytes(layer, T);
  if (need > kScratchBytes) {
    char msg[200];
    snprintf(msg, sizeof msg,
             "moe_forward_noalloc: T=%lld needs %zu bytes of scratch, the library's array holds %zu "
             "(use moe_forward with a workspace)", (long long)T, need, kScratchBytes);
    return moe::api_error(MOE_EWORKSPACE, msg);
  }
  // invalid arguments (need 0) and T == 0 are settled by the host-side checks
  if (need == 0 || T == 0)
    return moe::forward_with_ws(layer, x, T, y, out_dtype, topk_ids, topk_gates, nullptr, 0, stream);
  moe_status st = MOE_OK;
  void *ws = device_scratch(&st);
  if (!ws) return st;
  return moe::forward_with_ws(layer, x, T, y, out_dtype, topk_ids, topk_gates, ws, kScratchBytes, stream);
}
