// The fixed device scratch array behind muon_plan_step_noalloc: the
// workspace of steps whose callers cannot allocate device memory.
//
// One array per GPU (a file-scope __device__ variable has its own copy on
// every device the library's code object is loaded on), held until the
// process ends. In host code the array's name is only a host-side stand-in,
// so its device address is looked up once per device, with that device
// current, and kept; every host use (kernel arguments) takes that address.
#include <hip/hip_runtime.h>

#include <mutex>

#include "launch.hpp"

namespace muon {

static __device__ __align__(256) char scratch[kScratchBytes];

namespace {
constexpr int kMaxDevices = 64;
std::mutex g_scratch_mu;
void* g_scratch_ptr[kMaxDevices] = {};
}  // namespace

hipError_t scratch_address(void** out) {
  int dev = -1;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return e;
  if (dev < 0 || dev >= kMaxDevices) return hipErrorInvalidDevice;
  std::lock_guard<std::mutex> lock(g_scratch_mu);
  if (g_scratch_ptr[dev] == nullptr) {
    void* p = nullptr;
    e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    if (e != hipSuccess) return e;
    g_scratch_ptr[dev] = p;
  }
  *out = g_scratch_ptr[dev];
  return hipSuccess;
}

}  // namespace muon
