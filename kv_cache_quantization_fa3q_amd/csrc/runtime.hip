// Library-wide host pieces: status strings, version, device queries.
#include <mutex>
#include <unordered_map>

#include "fa3q_internal.hpp"

namespace fa3q {

int device_cu_count() {
  static std::mutex mu;
  static std::unordered_map<int, int> cache;
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess) return 256;
  std::lock_guard<std::mutex> lock(mu);
  auto it = cache.find(dev);
  if (it != cache.end()) return it->second;
  int cus = 0;
  if (hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || cus <= 0)
    cus = 256;
  cache[dev] = cus;
  return cus;
}

int device_max_lds_per_block() {
  static std::mutex mu;
  static std::unordered_map<int, int> cache;
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess) return 64 * 1024;
  std::lock_guard<std::mutex> lock(mu);
  auto it = cache.find(dev);
  if (it != cache.end()) return it->second;
  int lds = 0;
  if (hipDeviceGetAttribute(&lds, hipDeviceAttributeMaxSharedMemoryPerBlock, dev) != hipSuccess || lds <= 0)
    lds = 64 * 1024;
  cache[dev] = lds;
  return lds;
}

int allow_dynamic_lds(const void* kernel, size_t bytes) {
  if (bytes <= 64 * 1024) return FA3Q_OK;
  if (bytes > kLdsLimit || bytes > static_cast<size_t>(device_max_lds_per_block()))
    return FA3Q_ERR_UNSUPPORTED;
  static std::mutex mu;
  static std::unordered_map<const void*, size_t> done;
  std::lock_guard<std::mutex> lock(mu);
  auto it = done.find(kernel);
  if (it != done.end() && it->second >= bytes) return FA3Q_OK;
  if (hipFuncSetAttribute(kernel, hipFuncAttributeMaxDynamicSharedMemorySize,
                          static_cast<int>(kLdsLimit)) != hipSuccess)
    return FA3Q_ERR_HIP;
  done[kernel] = kLdsLimit;
  return FA3Q_OK;
}

}  // namespace fa3q

extern "C" const char* fa3q_status_string(int status) {
  switch (status) {
    case FA3Q_OK: return "FA3Q_OK";
    case FA3Q_ERR_NULL: return "FA3Q_ERR_NULL: a required pointer is NULL";
    case FA3Q_ERR_DTYPE: return "FA3Q_ERR_DTYPE: unknown dtype code";
    case FA3Q_ERR_SHAPE: return "FA3Q_ERR_SHAPE: invalid size";
    case FA3Q_ERR_RATIO: return "FA3Q_ERR_RATIO: ratio outside (0, 1] or int(ratio*N) < 1";
    case FA3Q_ERR_ALIGN: return "FA3Q_ERR_ALIGN: pointer not aligned as required";
    case FA3Q_ERR_WORKSPACE: return "FA3Q_ERR_WORKSPACE: workspace missing or too small";
    case FA3Q_ERR_HIP: return "FA3Q_ERR_HIP: HIP runtime rejected a launch";
    case FA3Q_ERR_UNSUPPORTED: return "FA3Q_ERR_UNSUPPORTED: arguments outside what this build handles";
    case FA3Q_ERR_ALIAS: return "FA3Q_ERR_ALIAS: an output partly overlaps an input";
    case FA3Q_ERR_SCRATCH: return "FA3Q_ERR_SCRATCH: the call needs more scratch than the static array holds";
    case FA3Q_ERR_LAYOUT: return "FA3Q_ERR_LAYOUT: unknown layout code";
    default: return "FA3Q_ERR_UNKNOWN";
  }
}

extern "C" int fa3q_version(void) { return (1 << 16) | 0; }
