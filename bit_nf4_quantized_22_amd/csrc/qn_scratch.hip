// Library-owned device scratch for callers that cannot allocate device
// memory (code under graph capture, serving loops, allocation-free hosts).
//
// One fixed array per GPU, loaded with this code object the first time the
// process touches it on that device and held until the process ends.  Host
// code never passes the array's name to a kernel: on the host that name is
// only a stand-in, not a device address.  The address of each device's
// copy comes from hipGetSymbolAddress, resolved once per device (with that
// device current) and cached here.
#include <hip/hip_runtime.h>

#include <mutex>

#include "qn_launch.h"

namespace qn {
namespace {

static __device__ __align__(256) unsigned char scratch[kScratchBytes];

constexpr int kMaxDevices = 64;
std::mutex g_mu;
void* g_addr[kMaxDevices] = {};

}  // namespace

hipError_t scratch_address(hipStream_t stream, void** out) {
  int cur = 0;
  hipError_t e = hipGetDevice(&cur);
  if (e != hipSuccess) return e;
  // the stream's device (the null stream belongs to the current one)
  int dev = cur;
  if (stream && (e = hipStreamGetDevice(stream, &dev)) != hipSuccess) return e;
  if (dev < 0 || dev >= kMaxDevices) return hipErrorInvalidDevice;
  std::lock_guard<std::mutex> lock(g_mu);
  if (!g_addr[dev]) {
    // resolved with that device current, then the caller's device restored
    if (dev != cur && (e = hipSetDevice(dev)) != hipSuccess) return e;
    void* p = nullptr;
    e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    if (dev != cur) {
      const hipError_t e2 = hipSetDevice(cur);
      if (e == hipSuccess) e = e2;
    }
    if (e != hipSuccess) return e;
    if (!p) return hipErrorInvalidSymbol;
    g_addr[dev] = p;
  }
  *out = g_addr[dev];
  return hipSuccess;
}

}  // namespace qn
