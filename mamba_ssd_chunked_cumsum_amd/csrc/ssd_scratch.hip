// Static device scratch for the no-allocation forward (ssd_forward_noalloc): its workspace (run
// states and decays of the fused path; the unfused path's intermediates when they
// fit) lives in this file-scope array instead of stream-ordered allocations. Each device the
// library runs on holds its own copy from the module's load until the process ends.
//
// In host code `scratch` names a host-side stand-in, not device memory: the device address of each
// device's copy comes from hipGetSymbolAddress, called once per device with that device current,
// and only that address is handed to kernels.
#include <hip/hip_runtime.h>

#include <mutex>

#include "ssd_launch.h"

namespace ssd {

static __device__ __align__(256) char scratch[kScratchBytes];

namespace {
constexpr int kMaxDevices = 64;
std::mutex g_mu;
void* g_addr[kMaxDevices] = {};
}  // namespace

hipError_t scratch_address(void** out) {
  int dev = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return e;
  if (dev < 0 || dev >= kMaxDevices) return hipErrorInvalidDevice;
  std::lock_guard<std::mutex> lock(g_mu);
  if (!g_addr[dev]) {
    void* p = nullptr;
    e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    if (e != hipSuccess) return e;
    g_addr[dev] = p;
  }
  *out = g_addr[dev];
  return hipSuccess;
}

}  // namespace ssd
