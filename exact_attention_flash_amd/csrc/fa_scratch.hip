// Library-owned device scratch for callers that cannot allocate device
// memory (code under stream capture, tight serving loops, harnesses that
// forbid hipMalloc): flash_attn_bwd_noalloc keeps the backward pass's row
// vectors here instead of in a caller workspace.
//
// The buffer is a file-scope device array, so every GPU the library runs on
// holds its own copy for the life of the process.  In host code the array's
// name is only a host-side stand-in, not a device address; the device
// address is looked up once per device with hipGetSymbolAddress (with that
// device current) and cached, and only that address is ever handed to a
// kernel.  Every call on one device shares that device's copy: calls that
// overlap in time on one device race on it.
#include <hip/hip_runtime.h>

#include <atomic>

#include "fa_launch.h"

namespace fa {

static __device__ __align__(256) unsigned char scratch[kNoallocScratchBytes];

hipError_t noalloc_scratch(void** out) {
  static std::atomic<void*> addr[kMaxDevices];
  int dev = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return e;
  if (dev < 0 || dev >= kMaxDevices) return hipErrorInvalidDevice;
  void* p = addr[dev].load(std::memory_order_acquire);
  if (p == nullptr) {
    // first call on this device, which is current: its copy's address
    e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    if (e != hipSuccess) return e;
    if (p == nullptr) return hipErrorInvalidSymbol;
    addr[dev].store(p, std::memory_order_release);
  }
  *out = p;
  return hipSuccess;
}

}  // namespace fa
