// Static scratch of the allocation-free forward (mlora_forward_noalloc): one
// file-scope device array, so callers that cannot allocate (graph capture,
// tight serving loops) still get the forward's work buffers.  Each GPU the
// library runs on holds its own copy at its own address until the process
// ends.  The array's name is a host-side stand-in in host code, never a
// device address: the address is looked up with hipGetSymbolAddress once
// per device, with that device current, and cached here; every use goes
// through the cached address.
#include <hip/hip_runtime.h>

#include <mutex>

#include "kernels.hpp"

namespace mlora {

namespace {

__device__ __align__(256) uint8_t scratch[kNoallocScratchBytes];

constexpr int kMaxDevices = 64;
std::mutex g_mu;
void* g_addr[kMaxDevices] = {};

}  // namespace

hipError_t noalloc_scratch(void** out, int* dev) {
  hipError_t e = hipGetDevice(dev);
  if (e != hipSuccess) return e;
  if (*dev < 0 || *dev >= kMaxDevices) return hipErrorInvalidDevice;
  std::lock_guard<std::mutex> lock(g_mu);
  if (!g_addr[*dev]) {
    void* p = nullptr;
    e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    if (e != hipSuccess) return e;
    if (!p) return hipErrorInvalidSymbol;
    g_addr[*dev] = p;
  }
  *out = g_addr[*dev];
  return hipSuccess;
}

}  // namespace mlora
