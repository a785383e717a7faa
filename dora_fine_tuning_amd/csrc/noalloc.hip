// Scratch memory of the entry point that allocates nothing
// (dora_compose_bwd_noalloc): a file-scope device array that each GPU holds
// from the library's load until the process ends, and its per-device address.
//
// In host code the array's name stands for a host-side symbol, not a device
// address, so kernels are given the address hipGetSymbolAddress returns, taken
// once per device with that device current and kept in a per-device table.
#include <hip/hip_runtime.h>

#include <mutex>

#include "noalloc_kernels.hpp"

namespace dora {

namespace {

static __device__ __align__(256) unsigned char scratch[kNoAllocScratchBytes];

constexpr int kMaxDevices = 64;
void* g_scratch[kMaxDevices];
hipError_t g_status[kMaxDevices];
std::once_flag g_once[kMaxDevices];

}  // namespace

hipError_t noalloc_scratch(hipStream_t stream, void** ptr) {
  int dev = -1;
  hipError_t e = hipStreamGetDevice(stream, &dev);
  if (e != hipSuccess) return e;
  if (dev < 0 || dev >= kMaxDevices) return hipErrorInvalidDevice;
  std::call_once(g_once[dev], [dev] {
    int cur = -1;
    hipError_t st = hipGetDevice(&cur);
    if (st == hipSuccess && cur != dev) st = hipSetDevice(dev);
    if (st == hipSuccess) st = hipGetSymbolAddress(&g_scratch[dev], HIP_SYMBOL(scratch));
    if (cur >= 0 && cur != dev) {
      const hipError_t back = hipSetDevice(cur);
      if (st == hipSuccess) st = back;
    }
    g_status[dev] = st;
  });
  if (g_status[dev] != hipSuccess) return g_status[dev];
  *ptr = g_scratch[dev];
  return hipSuccess;
}

}  // namespace dora
