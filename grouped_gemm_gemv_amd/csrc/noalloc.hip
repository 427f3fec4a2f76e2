// Device scratch memory of moe_forward_noalloc: a file-scope device array
// that every call on one GPU reuses in place of a caller's workspace.
//
// In host code the name `scratch` is a host-side stand-in, not a device
// address.  Its device address is taken once per device, with that device
// current, through hipGetSymbolAddress, and only that address is ever handed
// to kernels.  Each GPU holds its own copy of the array, at its own address,
// from the first call on it until the process ends.
#include <mutex>

#include "launch.hpp"

namespace moe {
namespace {

static __device__ __align__(256) unsigned char scratch[kNoallocScratchBytes];

constexpr int kMaxDevices = 64;
std::mutex g_mu;
void* g_ptr[kMaxDevices] = {};

}  // namespace

hipError_t noalloc_scratch(void** out) {
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
  *out = g_ptr[dev];
  return hipSuccess;
}

}  // namespace moe
