// attn_noalloc.hip -- the fixed device scratch behind attn_bwd_noalloc.
//
// A file-scope device array of ATTN_NOALLOC_SCRATCH_BYTES serves as the
// backward's workspace for callers that cannot allocate.  In host code the
// array's name only stands in for the symbol; its device address (one per
// GPU: each device holds its own copy once the module is loaded there) is
// looked up with hipGetSymbolAddress the first time a device asks for it,
// with that device current, and kept per device.  Only that address is ever
// handed to kernels.
#include <hip/hip_runtime.h>

#include <mutex>

#include "../../include/attn.h"

namespace {

static __device__ __align__(256) char scratch[ATTN_NOALLOC_SCRATCH_BYTES];

constexpr int MAX_DEVICES = 64;
std::mutex g_mu;
void* g_ptr[MAX_DEVICES] = {};

}  // namespace

namespace attn {

// Device address of the scratch array on the current device (looked up once
// per device).  Returns the HIP error of the lookup, or hipErrorInvalidDevice
// for a device index past the table.
hipError_t noalloc_scratch(void** out) {
  int dev = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return e;
  if (dev < 0 || dev >= MAX_DEVICES) return hipErrorInvalidDevice;
  std::lock_guard<std::mutex> lock(g_mu);
  if (!g_ptr[dev]) {
    void* p = nullptr;
    e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    if (e != hipSuccess) return e;
    g_ptr[dev] = p;
  }
  *out = g_ptr[dev];
  return hipSuccess;
}

}  // namespace attn
