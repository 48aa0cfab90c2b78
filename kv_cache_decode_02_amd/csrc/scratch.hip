// Device scratch of the allocation-free entry point.
//
// One file-scope device array per GPU, sized kvd::kNoAllocScratchBytes.  The
// code object's loader places it in device memory when the library is first
// used on a device, and it stays there until the process ends.  In host code
// the name `scratch` is only a host-side stand-in: its device address comes
// from hipGetSymbolAddress, looked up once per device with that device
// current, and that address is what the kernels receive.
#include <hip/hip_runtime.h>

#include <mutex>

#include "kvd_internal.h"

namespace kvd {
namespace {

__device__ __align__(256) unsigned char scratch[kNoAllocScratchBytes];

constexpr int kMaxDevices = 64;
std::mutex g_lock;
void* g_addr[kMaxDevices];  // device address of `scratch`, per device

}  // namespace

void* noalloc_scratch(hipError_t* err) {
  int dev = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e == hipSuccess && (dev < 0 || dev >= kMaxDevices)) e = hipErrorInvalidDevice;
  if (e != hipSuccess) {
    *err = e;
    return nullptr;
  }
  std::lock_guard<std::mutex> hold(g_lock);
  if (!g_addr[dev]) {
    void* p = nullptr;
    e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    if (e != hipSuccess || !p) {
      *err = e != hipSuccess ? e : hipErrorInvalidSymbol;
      return nullptr;
    }
    g_addr[dev] = p;
  }
  *err = hipSuccess;
  return g_addr[dev];
}

}  // namespace kvd
