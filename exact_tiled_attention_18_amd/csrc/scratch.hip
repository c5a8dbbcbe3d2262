// fa_bwd_noalloc's workspace: one static array per GPU (each device holds its own
// copy, at its own address, until the process ends).  In host code `scratch`
// names a host-side stand-in, not device memory, so the kernels only ever get the
// device address looked up below, once per device.
#include <hip/hip_runtime.h>

#include <mutex>

#include "fa.h"
#include "launch.h"

static __device__ __align__(256) float scratch[FA_BWD_NOALLOC_MAX_ROWS];

namespace fa {
namespace {
constexpr int kMaxDevices = 64;
std::mutex g_mu;
void* g_ptr[kMaxDevices] = {};
}  // namespace

hipError_t scratch_address(void** out) {
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
  *out = g_ptr[dev];
  return hipSuccess;
}

}  // namespace fa
