// Fixed device scratch for callers that cannot allocate (code under stream capture, tight
// serving loops, harnesses that forbid hipMalloc): one file-scope device array per GPU, whose
// address is looked up once per device and then passed to kernels like any other workspace.
#include <hip/hip_runtime.h>

#include <mutex>

#include "kernels.h"

namespace sa {
namespace {

constexpr int kMaxDevices = 64;

// Every GPU the library runs on holds its own copy of this array until the process ends.
__device__ __align__(256) unsigned char scratch[kNoAllocScratchBytes];

std::mutex g_scratch_mu;
void* g_scratch_ptr[kMaxDevices] = {};

}  // namespace

hipError_t noalloc_scratch(void** ptr) {
  *ptr = nullptr;
  int dev = -1;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return e;
  if (dev < 0 || dev >= kMaxDevices) return hipErrorInvalidDevice;
  std::lock_guard<std::mutex> lock(g_scratch_mu);
  if (!g_scratch_ptr[dev]) {
    // the device address of this GPU's copy (the name `scratch` is a host-side stand-in)
    void* p = nullptr;
    e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    if (e != hipSuccess) return e;
    if (!p) return hipErrorInvalidSymbol;
    g_scratch_ptr[dev] = p;
  }
  *ptr = g_scratch_ptr[dev];
  return hipSuccess;
}

}  // namespace sa
