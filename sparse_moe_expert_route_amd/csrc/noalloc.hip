// Static device scratch for the allocation-free layer entry point.
//
// Callers that cannot allocate (code under HIP graph capture, tight serving
// loops, harnesses that forbid hipMalloc) get the layer's workspace from this
// file-scope array instead of a caller buffer.  Each GPU holds its own copy
// of the array at its own address until the process ends.  In host code the
// array's name is only a stand-in for the symbol, so its device address is
// looked up once per device with hipGetSymbolAddress (with that device
// current) and only that address is ever passed to kernels.
#include <hip/hip_runtime.h>

#include <mutex>

#include "internal.h"
#include "moe_mi355x.h"

namespace moe {

static __device__ __align__(256) unsigned char scratch[MOE_NOALLOC_SCRATCH_BYTES];

namespace {
constexpr int kMaxDevices = 64;
std::mutex g_mu;
void *g_scratch[kMaxDevices];  // device address of `scratch` on each device, once looked up
}  // namespace

hipError_t noalloc_scratch(void **out) {
  *out = nullptr;
  int dev = -1;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return e;
  if (dev < 0 || dev >= kMaxDevices) return hipErrorInvalidDevice;
  std::lock_guard<std::mutex> lock(g_mu);
  if (!g_scratch[dev]) {
    void *p = nullptr;
    e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    if (e != hipSuccess) return e;
    if (!p) return hipErrorInvalidSymbol;
    g_scratch[dev] = p;
  }
  *out = g_scratch[dev];
  return hipSuccess;
}

}  // namespace moe
