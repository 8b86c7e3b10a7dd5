// Device-resident scratch of the no-allocation entry point.
//
// moe_fused_forward_noalloc runs the layer with this file-scope array as its
// workspace instead of a caller buffer, for callers that cannot allocate
// device memory.  Every GPU the library runs on holds its own copy of the
// array at its own address until the process ends; host code never passes
// the array's name (a host-side stand-in) to a kernel, only the device
// address hipGetSymbolAddress returns for the current device, cached per
// device here.
#include <hip/hip_runtime.h>

#include <atomic>

#include "moe_internal.h"

namespace moe {

static __device__ __align__(256) unsigned char scratch[kNoAllocScratchBytes];

namespace {
constexpr int kMaxDev = 64;
std::atomic<void*> g_scratch[kMaxDev];
}  // namespace

hipError_t noalloc_scratch(void** ptr) {
  *ptr = nullptr;
  int dev = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return e;
  if (dev < 0 || dev >= kMaxDev) return hipErrorInvalidDevice;
  void* p = g_scratch[dev].load(std::memory_order_acquire);
  if (!p) {
    // first use on this device (it is current): its copy's address; two host
    // threads racing here store the same value
    e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    if (e != hipSuccess) return e;
    if (!p) return hipErrorInvalidSymbol;
    g_scratch[dev].store(p, std::memory_order_release);
  }
  *ptr = p;
  return hipSuccess;
}

}  // namespace moe
