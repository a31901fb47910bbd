// Fixed device scratch for the entry point that allocates nothing.
//
// Callers that cannot allocate device memory (code under HIP graph capture,
// tight serving loops, harnesses that forbid it) get the split-KV decode's
// partials workspace from this file-scope array instead of a buffer of their
// own.  Every GPU the library runs on holds its own copy until the process
// ends, at its own address; in host code the array's name is only a stand-in,
// so the device address is looked up once per device with hipGetSymbolAddress
// and only that address is ever handed to kernels.
#include <hip/hip_runtime.h>

#include <mutex>

#include "internal.h"

namespace cpattn {
namespace {

static __device__ __align__(256) uint8_t scratch[kScratchBytes];

constexpr int kMaxDevices = 64;
std::mutex g_scratch_mu;
void* g_scratch_ptr[kMaxDevices] = {};

}  // namespace

hipError_t scratch_address(void** out) {
  int dev = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return e;
  if (dev < 0 || dev >= kMaxDevices) return hipErrorInvalidDevice;
  std::lock_guard<std::mutex> lock(g_scratch_mu);
  if (g_scratch_ptr[dev] == nullptr) {
    void* p = nullptr;
    e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));  // this device is current
    if (e != hipSuccess) return e;
    if (p == nullptr) return hipErrorInvalidSymbol;
    g_scratch_ptr[dev] = p;
  }
  *out = g_scratch_ptr[dev];
  return hipSuccess;
}

}  // namespace cpattn
