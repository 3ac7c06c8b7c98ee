// Per-device kernel attributes (host code): the dynamic-LDS limit of a kernel is raised once per
// (kernel, device), on the device of the stream the kernel is launched on.

#include <hip/hip_runtime.h>

#include <mutex>
#include <vector>

#include "rba_internal.h"

namespace rba {

namespace {
struct LdsLimit {
  const void* fn;
  int device;
  int bytes;
};
std::mutex g_mu;
std::vector<LdsLimit> g_set;   // (kernel, device) pairs raised so far, with the limit set

// Device the stream's work runs on (the current device for the null stream).
hipError_t stream_device(hipStream_t s, int* dev) {
  if (s == nullptr) return hipGetDevice(dev);
  return hipStreamGetDevice(s, dev);
}
}  // namespace

hipError_t set_max_lds(const void* fn, int bytes, hipStream_t s) {
  if (bytes <= 64 * 1024) return hipSuccess;   // within the default limit
  int dev = 0;
  hipError_t e = stream_device(s, &dev);
  if (e != hipSuccess) return e;
  std::lock_guard<std::mutex> lock(g_mu);
  for (const LdsLimit& x : g_set)
    if (x.fn == fn && x.device == dev && x.bytes >= bytes) return hipSuccess;
  int cur = 0;
  e = hipGetDevice(&cur);
  if (e != hipSuccess) return e;
  if (cur != dev && (e = hipSetDevice(dev)) != hipSuccess) return e;
  e = hipFuncSetAttribute(fn, hipFuncAttributeMaxDynamicSharedMemorySize, bytes);
  if (cur != dev) {
    const hipError_t e2 = hipSetDevice(cur);
    if (e == hipSuccess) e = e2;
  }
  if (e != hipSuccess) return e;
  for (LdsLimit& x : g_set)
    if (x.fn == fn && x.device == dev) {
      x.bytes = bytes;
      return hipSuccess;
    }
  g_set.push_back({fn, dev, bytes});
  return hipSuccess;
}

}  // namespace rba
