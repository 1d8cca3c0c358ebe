// Static device scratch for the entry point that allocates nothing
// (mx_quantize_noalloc): the per-workgroup partial maxima of the tensor-wide
// max |x| pass live in a file-scope device array instead of a caller
// workspace.  Each device holds its own copy of the array until the process
// ends; its device address is looked up once per device with the device
// current and kept here, and only that address is ever handed to kernels
// (in host code the array's name is not a device address).
#include <hip/hip_runtime.h>

#include <mutex>

#include "mx_kernels.h"

namespace mxk {

namespace {
constexpr int kMaxDevices = 64;
static __device__ __align__(256) uint32_t scratch[kNoallocScratchBytes / sizeof(uint32_t)];
std::mutex g_mu;
void* g_ptr[kMaxDevices] = {};
}  // namespace

hipError_t noalloc_scratch(void** ptr) {
  *ptr = nullptr;
  int dev = -1;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return e;
  if (dev < 0 || dev >= kMaxDevices) return hipErrorInvalidDevice;
  std::lock_guard<std::mutex> lock(g_mu);
  if (!g_ptr[dev]) {
    void* p = nullptr;
    e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    if (e != hipSuccess) return e;
    if (!p) return hipErrorInvalidSymbol;
    g_ptr[dev] = p;
  }
  *ptr = g_ptr[dev];
  return hipSuccess;
}

}  // namespace mxk
