// static_workspace.hip -- the workspace that gdn_prefill_static_workspace
// hands to the two-pass chunked prefill: a file-scope device array, one copy
// per device, so that its callers allocate nothing.
//
// Host code never passes `scratch` itself to a kernel: in host code the name
// is a host-side stand-in, not the array's device address.  The address is
// asked for once per device, with that device current, through
// hipGetSymbolAddress, and kept per device; kernels receive that pointer as
// their workspace argument, as they receive a caller's workspace.
#include <hip/hip_runtime.h>

#include <mutex>

#include "gdn.h"
#include "gdn_launch.hpp"

namespace gdn {

namespace {

constexpr int kMaxDevices = 64;

// Every call on a device shares this array and finds in it whatever the last
// call left: the chunk table and the per-chunk records are written in full
// before they are read, so nothing needs clearing.
__device__ __align__(256) unsigned char scratch[GDN_STATIC_WORKSPACE_BYTES];

std::mutex g_mutex;
void* g_ptr[kMaxDevices] = {};

}  // namespace

hipError_t static_workspace(void** ptr, size_t* bytes) {
  *ptr = nullptr;
  *bytes = 0;
  int dev = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return e;
  if (dev < 0 || dev >= kMaxDevices) return hipErrorInvalidDevice;
  std::lock_guard<std::mutex> lock(g_mutex);
  if (g_ptr[dev] == nullptr) {
    void* p = nullptr;
    e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    if (e != hipSuccess) return e;
    if (p == nullptr || (reinterpret_cast<uintptr_t>(p) & 255u) != 0) return hipErrorInvalidSymbol;
    g_ptr[dev] = p;
  }
  *ptr = g_ptr[dev];
  *bytes = GDN_STATIC_WORKSPACE_BYTES;
  return hipSuccess;
}

}  // namespace gdn
