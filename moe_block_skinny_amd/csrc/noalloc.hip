// noalloc.hip -- the device-resident scratch of moe_block_noalloc, for
// callers that cannot allocate device memory (code under HIP graph capture,
// tight serving loops, harnesses that forbid hipMalloc).
//
// One file-scope device array per GPU the library runs on, held until the
// process ends.  In host code the array's name stands for a host-side
// symbol, not a device address: its device address is looked up once per
// device with hipGetSymbolAddress (with that device current) and kept; only
// that address is ever handed to kernels.

#include <hip/hip_runtime.h>

#include <mutex>

#include "internal.hpp"

namespace moe {

static __device__ __align__(256) unsigned char scratch[kNoallocScratchBytes];

namespace {
constexpr int kMaxDevices = 64;
std::mutex g_lock;
void* g_addr[kMaxDevices];   // device address of `scratch` on each device (null: not looked up yet)
}  // namespace

hipError_t noalloc_scratch(void** ptr) {
  int dev = -1;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return e;
  if (dev < 0 || dev >= kMaxDevices) return hipErrorInvalidDevice;
  std::lock_guard<std::mutex> g(g_lock);
  if (!g_addr[dev]) {
    void* p = nullptr;
    e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    if (e != hipSuccess) return e;
    if (!p) return hipErrorInvalidSymbol;
    g_addr[dev] = p;
  }
  *ptr = g_addr[dev];
  return hipSuccess;
}

}  // namespace moe
