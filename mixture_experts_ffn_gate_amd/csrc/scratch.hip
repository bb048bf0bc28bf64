// Static device scratch of the allocation-free entry points.
//
// `scratch` is a file-scope device array that each GPU the library runs on
// holds until the process ends. Host code never uses its name as a device
// address (in host code the name is a host-side stand-in): the first call on
// each device resolves the device address with hipGetSymbolAddress, with that
// device current, and every later call on the device reuses it.
#include <atomic>
#include <mutex>

#include "kernels.h"

static __device__ __align__(256) int scratch[MOE_STATIC_SCRATCH_INTS];

namespace {
constexpr int kMaxDevices = 64;
std::atomic<int*> g_scratch[kMaxDevices];
std::mutex g_scratch_mu;
}  // namespace

hipError_t static_scratch(int** out) {
  *out = nullptr;
  int dev = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return e;
  if (dev < 0 || dev >= kMaxDevices) return hipErrorInvalidDevice;
  int* p = g_scratch[dev].load(std::memory_order_acquire);
  if (!p) {
    std::lock_guard<std::mutex> lock(g_scratch_mu);
    p = g_scratch[dev].load(std::memory_order_relaxed);
    if (!p) {
      void* addr = nullptr;
      e = hipGetSymbolAddress(&addr, HIP_SYMBOL(scratch));
      if (e != hipSuccess) return e;
      if (!addr) return hipErrorInvalidSymbol;
      p = (int*)addr;
      g_scratch[dev].store(p, std::memory_order_release);
    }
  }
  *out = p;
  return hipSuccess;
}
