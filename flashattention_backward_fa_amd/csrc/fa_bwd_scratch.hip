// Library-owned device scratch for fa_bwd_run_noalloc: a file-scope device
// array that the HIP runtime places on each GPU when the library's code
// object is loaded there, so that the entry point itself allocates nothing.
//
// In host code the array's name is only a host-side stand-in; its device
// address on the current device comes from hipGetSymbolAddress, looked up
// once per device (with that device current) and kept in a per-device table.
// Only that address is ever passed to kernels.

#include <hip/hip_runtime.h>

#include <mutex>

#include "fa_bwd_internal.h"

namespace fabwd {
namespace {

__device__ __align__(256) unsigned char scratch[SCRATCH_BYTES];

constexpr int kMaxDevices = 64;
std::mutex g_mu;
void* g_ptr[kMaxDevices] = {};

}  // namespace

int scratch_ptr(void** ptr) {
  int dev = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return (int)e;
  if (dev < 0 || dev >= kMaxDevices) return (int)hipErrorInvalidDevice;
  std::lock_guard<std::mutex> lock(g_mu);
  if (!g_ptr[dev]) {
    void* p = nullptr;
    e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    if (e != hipSuccess) return (int)e;
    if (!p) return (int)hipErrorInvalidSymbol;
    g_ptr[dev] = p;
  }
  *ptr = g_ptr[dev];
  return 0;
}

}  // namespace fabwd
