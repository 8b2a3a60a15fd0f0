// Device scratch for the entry point that allocates nothing
// (attn_fwd_splitkv_noalloc): the split partials of the split-key forward
// live in a file-scope device array instead of a caller workspace.
//
// In host code `scratch` names a host-side stand-in, not device memory: its
// device address is taken once per device with hipGetSymbolAddress (the
// calling thread's current device being that device), kept in a per-device
// table, and only that address is ever handed to kernels. Each device holds
// its own copy of the array for the life of the process; every call on one
// device shares it, so calls that overlap on one device race.

#include <hip/hip_runtime.h>
#include <stdint.h>

#include <mutex>

#include "fwd_params.h"

namespace attn {
namespace {

static __device__ __align__(256) uint8_t scratch[kNoallocScratchBytes];

constexpr int kMaxDevices = 64;
std::mutex g_scratch_mu;
void* g_scratch_ptr[kMaxDevices] = {};

}  // namespace

int noalloc_scratch(void** ptr) {
  int dev = -1;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return (int)e;
  if (dev < 0 || dev >= kMaxDevices) return (int)hipErrorInvalidDevice;
  std::lock_guard<std::mutex> lock(g_scratch_mu);
  if (g_scratch_ptr[dev] == nullptr) {
    void* p = nullptr;
    e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    if (e != hipSuccess) return (int)e;
    if (p == nullptr) return (int)hipErrorInvalidSymbol;
    g_scratch_ptr[dev] = p;
  }
  *ptr = g_scratch_ptr[dev];
  return (int)hipSuccess;
}

}  // namespace attn
