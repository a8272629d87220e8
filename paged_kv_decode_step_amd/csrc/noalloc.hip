// noalloc.hip -- a fixed device array that stands in for a pool's split-K
// workspace, for callers that cannot allocate device memory at step time.
//
// The array is a file-scope device variable: each GPU the library runs on
// holds its own copy from the moment the code object is loaded until the
// process ends.  In host code its name is only a stand-in for the symbol,
// not a device address, so its address on each device is looked up once,
// with that device current, and kept; kernels get that address as an
// argument like any workspace.
#include <hip/hip_runtime.h>

#include <mutex>

#include "kernels.h"

namespace pkv {
namespace {

static __device__ __align__(256) char scratch[kScratchBytes];

constexpr int kMaxDevices = 64;

std::mutex g_lock;
void* g_addr[kMaxDevices] = {};

}  // namespace

hipError_t scratch_address(int device, void** addr) {
  *addr = nullptr;
  if (device < 0 || device >= kMaxDevices) return hipErrorInvalidDevice;
  std::lock_guard<std::mutex> hold(g_lock);
  if (!g_addr[device]) {
    int prev = -1;
    hipError_t e = hipGetDevice(&prev);
    if (e != hipSuccess) return e;
    if (prev != device) {
      e = hipSetDevice(device);
      if (e != hipSuccess) return e;
    }
    void* p = nullptr;
    e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    if (prev != device) (void)hipSetDevice(prev);
    if (e != hipSuccess) return e;
    if (!p) return hipErrorInvalidSymbol;
    g_addr[device] = p;
  }
  *addr = g_addr[device];
  return hipSuccess;
}

}  // namespace pkv
