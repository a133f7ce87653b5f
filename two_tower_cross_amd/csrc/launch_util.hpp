// Host helpers of the kernel launchers: per-device settings and queries, cached once per device
// and safe to call from several host threads at once.
#pragma once

#include <hip/hip_runtime.h>

#include <map>
#include <mutex>
#include <utility>

namespace tt {

// Lets `func` launch with up to `bytes` of dynamic LDS on the current device: the attribute is set
// once per (kernel, device) and the outcome remembered, so that later launches skip the call.
inline hipError_t allow_dynamic_lds(const void *func, int bytes) {
  static std::mutex mu;
  static std::map<std::pair<const void *, int>, hipError_t> done;
  int dev = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return e;
  std::lock_guard<std::mutex> lock(mu);
  const auto key = std::make_pair(func, dev);
  const auto it = done.find(key);
  if (it != done.end()) return it->second;
  e = hipFuncSetAttribute(func, hipFuncAttributeMaxDynamicSharedMemorySize, bytes);
  done.emplace(key, e);
  return e;
}

// Compute units of the current device, queried once per device; 0 when the query fails.
inline int current_device_cus() {
  static std::mutex mu;
  static std::map<int, int> cus;
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess) return 0;
  std::lock_guard<std::mutex> lock(mu);
  const auto it = cus.find(dev);
  if (it != cus.end()) return it->second;
  int n = 0;
  if (hipDeviceGetAttribute(&n, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess) n = 0;
  cus.emplace(dev, n);
  return n;
}

}  // namespace tt
