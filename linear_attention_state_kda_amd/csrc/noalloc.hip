// Library-owned scratch for the allocation-free prefill entry point
// (kda_chunk_prefill_noalloc): a static device array, one copy per GPU the
// library runs on, held until the process ends.  Host code never passes the
// array's own name to a kernel (on the host it is only a stand-in for the
// symbol): the device address is resolved once per device with
// hipGetSymbolAddress, with that device current, and cached.
#include <mutex>

#include <hip/hip_runtime.h>

#include "kda_launch.hpp"

namespace kda {

__device__ __align__(256) uint8_t scratch[kNoallocScratchBytes];

namespace {
constexpr int kMaxDevices = 64;
std::mutex g_mu;
void* g_scratch[kMaxDevices] = {};
}  // namespace

hipError_t noalloc_scratch(void** out) {
  int dev = -1;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return e;
  if (dev < 0 || dev >= kMaxDevices) return hipErrorInvalidDevice;
  std::lock_guard<std::mutex> lock(g_mu);
  if (g_scratch[dev] == nullptr) {
    void* p = nullptr;
    e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    if (e != hipSuccess) return e;
    if (p == nullptr) return hipErrorInvalidSymbol;
    g_scratch[dev] = p;
  }
  *out = g_scratch[dev];
  return hipSuccess;
}

}  // namespace kda
