// moe_ffn_forward_static: the whole forward with its scratch memory in a
// file-scope device array instead of a caller-provided workspace, for
// callers that cannot allocate device memory (code under graph capture, tight
// serving loops, harnesses that forbid allocation).
//
// The array `scratch` holds MOE_STATIC_SCRATCH_BYTES on every device the
// library runs on (the code object of this file is loaded, and the array
// allocated, on a device's first call), until the process ends.  Its device
// address is looked up once per device with hipGetSymbolAddress while that
// device is current; host code only ever passes that address on (the array's
// own name is a host-side stand-in, not a device address).  The forward's
// kernels start from no scratch contents (nothing in the workspace needs to be
// zero), so consecutive calls need no clearing; calls that overlap on one
// device share the array and race.
#include <mutex>

#include "moe_internal.h"

namespace {

static __device__ __align__(256) unsigned char scratch[MOE_STATIC_SCRATCH_BYTES];

constexpr int kMaxDevices = 64;
std::mutex g_scratch_mu;
void* g_scratch_ptr[kMaxDevices];   // device address of `scratch`, per device

// The current device's address of `scratch` (looked up on the first call on
// that device).
hipError_t scratch_address(void** out) {
  int dev = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return e;
  if (dev < 0 || dev >= kMaxDevices) return hipErrorInvalidDevice;
  std::lock_guard<std::mutex> lock(g_scratch_mu);
  if (!g_scratch_ptr[dev]) {
    void* p = nullptr;
    e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    if (e != hipSuccess) return e;
    g_scratch_ptr[dev] = p;
  }
  *out = g_scratch_ptr[dev];
  return hipSuccess;
}

}  // namespace

extern "C" moe_status moe_ffn_forward_static(const moe_problem* p, const moe_weights* w,
                                             const void* x, float* y, const moe_routing* out,
                                             hipStream_t stream) {
  size_t need = 0;
  moe_status st = moe_workspace_size(p, &need);
  if (st != MOE_OK) return st;
  if (need > (size_t)MOE_STATIC_SCRATCH_BYTES) return MOE_ERR_WORKSPACE;
  void* ptr = nullptr;
  const hipError_t e = scratch_address(&ptr);
  if (e != hipSuccess) return moe::hip_failure(e);
  return moe_ffn_forward(p, w, x, y, out, ptr, (size_t)MOE_STATIC_SCRATCH_BYTES, stream);
}
