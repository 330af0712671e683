// Device scratch of pkd_run_static, the run for callers that cannot allocate
// device memory: a plan's work list, merge records, fold counters and
// partial states live here instead of in a caller-allocated workspace.
//
// The array is a static device variable, so every device the library runs
// on holds its own copy from the library's load until the process ends. On
// the host `scratch` names only a stand-in for the device symbol; its device
// address is looked up once per device, with that device current, and only
// that address is given to copies and kernels.
#include <hip/hip_runtime.h>

#include <mutex>

#include "launch.h"

static __device__ __align__(256) unsigned char scratch[pkd::kStaticScratchBytes];

namespace pkd {

namespace {

constexpr int kMaxDevices = 64;
std::mutex g_scratch_mu;
void* g_scratch_ptr[kMaxDevices] = {};

}  // namespace

hipError_t static_scratch_address(void** ptr, int* device) {
  int dev = -1;
  hipError_t e = hipGetDevice(&dev);
  *device = dev;
  if (e != hipSuccess) return e;
  if (dev < 0 || dev >= kMaxDevices) return hipErrorInvalidDevice;
  std::lock_guard<std::mutex> lk(g_scratch_mu);
  if (!g_scratch_ptr[dev]) {
    void* p = nullptr;
    e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    if (e != hipSuccess) return e;
    if (!p) return hipErrorInvalidSymbol;
    g_scratch_ptr[dev] = p;
  }
  *ptr = g_scratch_ptr[dev];
  return hipSuccess;
}

}  // namespace pkd
