// Device scratch of dmuon_muon_step_noalloc: a file-scope array that every
// GPU the library runs on holds from module load until the process ends, so
// that a step needs no allocation at all (for callers that cannot allocate:
// code under HIP graph capture, tight serving loops, harnesses that forbid
// hipMalloc).
//
// In host code the array's name is only a stand-in for the symbol, not a
// device address: the address of this device's copy comes from
// hipGetSymbolAddress, looked up once per device and kept.

#include <hip/hip_runtime.h>

#include <mutex>

#include "internal.h"

namespace dmuon {

static __device__ __align__(256) char scratch[kNoAllocScratchBytes];

namespace {
constexpr int kMaxDevices = 64;
std::mutex g_scratch_mu;
void *g_scratch_ptr[kMaxDevices] = {};
}  // namespace

hipError_t noalloc_scratch(void **ptr) {
  int dev = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return e;
  if (dev < 0 || dev >= kMaxDevices) return hipErrorInvalidDevice;
  std::lock_guard<std::mutex> lock(g_scratch_mu);
  if (!g_scratch_ptr[dev]) {
    void *p = nullptr;
    // with this device current: the address of its own copy of the array
    e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    if (e != hipSuccess) return e;
    g_scratch_ptr[dev] = p;
  }
  *ptr = g_scratch_ptr[dev];
  return hipSuccess;
}

}  // namespace dmuon
