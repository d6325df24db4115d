// The library's own device scratch memory, for callers that cannot allocate.
//
// One file-scope array per GPU (each device holds its own copy, for the life of the
// process).  In host code the array's name is only a host-side stand-in; its device
// address comes from hipGetSymbolAddress, looked up once per device with that device
// current, and only that address is ever handed to kernels.
#include <hip/hip_runtime.h>

#include <mutex>

#include "kernels.h"

namespace pkv {

static __device__ __align__(256) unsigned char scratch[kScratchBytes];

namespace {
constexpr int kMaxScratchDevices = 64;
std::mutex g_scratch_mu;
void* g_scratch_ptr[kMaxScratchDevices] = {};
}  // namespace

hipError_t scratch_device_pointer(void** out) {
  *out = nullptr;
  int dev = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return e;
  if (dev < 0 || dev >= kMaxScratchDevices) return hipErrorInvalidDevice;
  std::lock_guard<std::mutex> lk(g_scratch_mu);
  if (!g_scratch_ptr[dev]) {
    void* p = nullptr;
    e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    if (e != hipSuccess) return e;
    if (!p || (reinterpret_cast<uintptr_t>(p) & 255u)) return hipErrorInvalidValue;
    g_scratch_ptr[dev] = p;
  }
  *out = g_scratch_ptr[dev];
  return hipSuccess;
}

}  // namespace pkv
