// moe_forward_noalloc: moe_forward with its workspace in a static device
// array instead of a caller buffer, for callers that cannot allocate device
// memory (code under graph capture, tight serving loops).
//
// The array lives in this library's code object: every GPU the library runs
// on holds its own copy from the first call on that device until the process
// ends.  In host code `scratch` names a host-side stand-in, not a device
// address, so its address is fetched once per device with hipGetSymbolAddress
// (with that device current) and only that pointer is handed to the kernels.
// The forward needs no initial contents in its workspace (every kernel clears
// what it accumulates into), so nothing is cleared here.  Calls on one GPU
// share the array: calls that overlap in time on one GPU race.
#include "moe.h"

#include <hip/hip_runtime.h>

#include <mutex>

namespace {

constexpr size_t kScratchBytes = size_t(MOE_NOALLOC_SCRATCH_BYTES);
constexpr int kMaxDevices = 64;

static __device__ __align__(256) uint8_t scratch[kScratchBytes];

std::once_flag g_once[kMaxDevices];
void* g_scratch[kMaxDevices];
hipError_t g_status[kMaxDevices];

}  // namespace

namespace moe {
void set_last_hip_error(int e);   // api.cpp
}

extern "C" int moe_forward_noalloc(const moe_shape_t* s, const void* x, const void* router_w, const float* router_b,
                                   const void* w_gate, const void* w_up, const void* w_down,
                                   const void* ws_gate, const void* ws_up, const void* ws_down, void* out,
                                   void* stream) {
  size_t need = 0;
  if (int rc = moe_workspace_size(s, &need)) return rc;
  if (need > kScratchBytes) return MOE_ERR_TOO_LARGE;
  if (s->T == 0) return MOE_OK;
  int dev = -1;
  if (hipError_t e = hipGetDevice(&dev); e != hipSuccess) {
    moe::set_last_hip_error(int(e));
    return MOE_ERR_HIP;
  }
  if (dev < 0 || dev >= kMaxDevices) {
    moe::set_last_hip_error(int(hipErrorInvalidDevice));
    return MOE_ERR_HIP;
  }
  std::call_once(g_once[dev], [dev] {
    g_status[dev] = hipGetSymbolAddress(&g_scratch[dev], HIP_SYMBOL(scratch));
    if (g_status[dev] == hipSuccess && !g_scratch[dev]) g_status[dev] = hipErrorInvalidSymbol;
  });
  if (g_status[dev] != hipSuccess) {
    moe::set_last_hip_error(int(g_status[dev]));
    return MOE_ERR_HIP;
  }
  return moe_forward(s, x, router_w, router_b, w_gate, w_up, w_down, ws_gate, ws_up, ws_down, out, g_scratch[dev],
                     kScratchBytes, stream);
}
