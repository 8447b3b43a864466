// noalloc.hip -- the device scratch of hyena_fftconv_fwd_noalloc, the
// single-pass entry point for callers that cannot allocate.
//
// The array below is part of the library's code object: every GPU the library
// is loaded on holds its own copy, from the load until the process ends.  Host
// code must not use the array's name as a device address (in host code it is
// only a stand-in symbol); its address on the current device comes from
// hipGetSymbolAddress, looked up once per device and kept.
#include <hip/hip_runtime.h>

#include <mutex>

#include "launch.hpp"

namespace hyena {

namespace {

static __device__ __align__(256) unsigned char scratch[NOALLOC_SCRATCH_BYTES];

constexpr int kMaxDevices = 256;
std::mutex g_mu;
void* g_ptr[kMaxDevices] = {};

}  // namespace

hipError_t noalloc_scratch(void** ptr, size_t* bytes) {
  int dev = -1;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return e;
  if (dev < 0 || dev >= kMaxDevices) return hipErrorInvalidDevice;
  std::lock_guard<std::mutex> lock(g_mu);
  if (g_ptr[dev] == nullptr) {
    void* p = nullptr;
    e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    if (e != hipSuccess) return e;
    if (p == nullptr) return hipErrorInvalidSymbol;
    g_ptr[dev] = p;
  }
  *ptr = g_ptr[dev];
  *bytes = NOALLOC_SCRATCH_BYTES;
  return hipSuccess;
}

}  // namespace hyena
