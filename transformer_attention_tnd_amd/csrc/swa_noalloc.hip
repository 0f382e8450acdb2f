// Library-owned device scratch for the backward entry point that allocates
// nothing (swa_backward_noalloc in include/swa.h).
//
// `scratch` is one fixed array per GPU, part of this file's code object: it is
// placed in device memory when the code object is loaded on a device and held
// until the process ends.  Host code never passes the array's name to a
// kernel or a copy (on the host that name is only a stand-in, not a device
// address); it looks up each device's address once, with that device current,
// and uses that pointer from then on.

#include <hip/hip_runtime.h>

#include <mutex>

#include "swa_internal.hpp"

static __device__ __align__(256) unsigned char scratch[swa::kNoAllocScratchBytes];

namespace swa {
namespace {

constexpr int kMaxDevices = 64;
std::mutex g_mu;
void* g_ptr[kMaxDevices];  // device address of `scratch`, per device (null: not looked up)

}  // namespace

int noalloc_scratch(void* stream, void** ptr, int* device) {
  int dev = 0;
  hipError_t e = stream ? hipStreamGetDevice(static_cast<hipStream_t>(stream), &dev)
                        : hipGetDevice(&dev);
  if (e != hipSuccess) return (int)e;
  if (dev < 0 || dev >= kMaxDevices) return (int)hipErrorInvalidDevice;
  std::lock_guard<std::mutex> lock(g_mu);
  if (!g_ptr[dev]) {
    int cur = 0;
    if ((e = hipGetDevice(&cur)) != hipSuccess) return (int)e;
    if (cur != dev && (e = hipSetDevice(dev)) != hipSuccess) return (int)e;
    void* p = nullptr;
    e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    if (cur != dev) {
      const hipError_t r = hipSetDevice(cur);
      if (e == hipSuccess) e = r;
    }
    if (e != hipSuccess) return (int)e;
    if (!p) return (int)hipErrorInvalidSymbol;
    g_ptr[dev] = p;
  }
  *ptr = g_ptr[dev];
  *device = dev;
  return 0;
}

}  // namespace swa
