// The library-held scratch memory of kda_prefill_noalloc: the segment-parallel prefill's
// workspace (the per-segment states B, M and start states) in a file-scope device array,
// for callers that cannot allocate device memory.
//
// In host code `scratch` names a host-side stand-in, not a device address.  The device
// address of each GPU's copy comes from hipGetSymbolAddress, taken once per device (with
// that device current) on the entry point's first call there, and kept; kernels receive
// that address as an argument like any workspace.  Every call on one GPU shares that GPU's
// array, so calls that overlap on one GPU race (the API contract says so).  Nothing in it
// has to start at zero: the three passes write every plane before reading it.
#include <hip/hip_runtime.h>

#include <mutex>

#include "kda_internal.h"

namespace kda {

static __device__ __align__(256) unsigned char scratch[kNoAllocScratchBytes];

namespace {

constexpr int kMaxDevices = 64;
std::mutex g_mu;
void* g_scratch[kMaxDevices] = {};

}  // namespace

hipError_t noalloc_scratch(hipStream_t stream, void** ptr) {
  *ptr = nullptr;
  int dev = 0;
  hipError_t e = hipStreamGetDevice(stream, &dev);
  if (e != hipSuccess) return e;
  if (dev < 0 || dev >= kMaxDevices) return hipErrorInvalidDevice;
  std::lock_guard<std::mutex> lock(g_mu);
  if (!g_scratch[dev]) {
    int cur = 0;
    e = hipGetDevice(&cur);
    if (e != hipSuccess) return e;
    if (cur != dev && (e = hipSetDevice(dev)) != hipSuccess) return e;
    void* p = nullptr;
    e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    if (cur != dev) {
      const hipError_t e2 = hipSetDevice(cur);
      if (e == hipSuccess) e = e2;
    }
    if (e != hipSuccess) return e;
    if (!p) return hipErrorInvalidSymbol;
    g_scratch[dev] = p;
  }
  *ptr = g_scratch[dev];
  return hipSuccess;
}

}  // namespace kda
