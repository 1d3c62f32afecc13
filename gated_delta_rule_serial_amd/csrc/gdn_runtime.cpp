// gdn_runtime.cpp -- per-device launch state of libgdn: the dynamic-LDS
// limit of the kernels that need more than the default 64 KiB, and the
// compute-unit count that sizes persistent grids.  Both are kept per device
// (HIP applies a function attribute, and reports attributes, for the device
// that is current on the calling thread) and guarded for concurrent callers.
#include <hip/hip_runtime.h>

#include <atomic>
#include <mutex>
#include <vector>

#include "gdn_launch.hpp"

namespace gdn {

namespace {

constexpr int kMaxDevices = 64;

struct LdsEntry {
  const void* kernel;
  int device;
  int bytes;
};

std::mutex g_lds_mutex;
std::vector<LdsEntry> g_lds_done;  // (kernel, device) pairs already configured

std::atomic<int> g_cus[kMaxDevices];  // 0: not queried yet

int current_device() {
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0) dev = 0;
  return dev;
}

}  // namespace

hipError_t ensure_dynamic_lds(const void* kernel, int bytes) {
  const int dev = current_device();
  std::lock_guard<std::mutex> lock(g_lds_mutex);
  for (const LdsEntry& e : g_lds_done)
    if (e.kernel == kernel && e.device == dev && e.bytes >= bytes) return hipSuccess;
  const hipError_t e = hipFuncSetAttribute(kernel, hipFuncAttributeMaxDynamicSharedMemorySize, bytes);
  if (e == hipSuccess) g_lds_done.push_back(LdsEntry{kernel, dev, bytes});
  return e;
}

int device_compute_units() {
  int dev = 0;
  const bool have = hipGetDevice(&dev) == hipSuccess && dev >= 0;
  if (have && dev < kMaxDevices) {
    const int cached = g_cus[dev].load(std::memory_order_relaxed);
    if (cached > 0) return cached;
  }
  int n = 0;
  if (!have || hipDeviceGetAttribute(&n, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || n <= 0)
    return 256;  // no device to ask (a host-only query): the MI355X's count
  if (dev < kMaxDevices) g_cus[dev].store(n, std::memory_order_relaxed);
  return n;
}

}  // namespace gdn
