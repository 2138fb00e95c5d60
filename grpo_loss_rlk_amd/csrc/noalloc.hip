// Scratch memory for the entry point that allocates nothing
// (rlk_logprob_from_logits_noalloc): for callers that cannot call hipMalloc --
// code under HIP graph capture, tight serving loops, harnesses that forbid
// allocation. It is one file-scope device array, so every GPU the library
// runs on holds its own copy (at its own address) until the process ends.
//
// In host code the array's name is only a host-side stand-in: its device
// address comes from hipGetSymbolAddress, looked up once per device with that
// device current, and only that address is ever handed to a kernel.
#include <hip/hip_runtime.h>

#include <mutex>

#include "kernels.h"

namespace rlk {

namespace {

__device__ __align__(256) uint8_t scratch[kNoAllocScratchBytes];

constexpr int kMaxDevices = 64;
std::mutex g_mutex;
void* g_scratch_ptr[kMaxDevices] = {};

}  // namespace

hipError_t noalloc_scratch(void** out) {
  *out = nullptr;
  int dev = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return e;
  if (dev < 0 || dev >= kMaxDevices) return hipErrorInvalidDevice;
  std::lock_guard<std::mutex> lock(g_mutex);
  if (g_scratch_ptr[dev] == nullptr) {
    void* p = nullptr;
    e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    if (e != hipSuccess) return e;
    if (p == nullptr) return hipErrorInvalidSymbol;
    g_scratch_ptr[dev] = p;
  }
  *out = g_scratch_ptr[dev];
  return hipSuccess;
}

}  // namespace rlk
