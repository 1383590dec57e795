// Per-device launch facts shared by every kernel launcher: the compute-unit
// count, the resident-workgroup count of each kernel instance at each
// dynamic-LDS size, and whether a kernel's dynamic-LDS limit has been raised.
//
// The launchers run on the caller's threads, several at a time when one plan
// is used from several threads or on several devices. Every entry here is
// looked up and filled under one mutex and keyed by the current device, so a
// first use from two threads at once neither races nor mixes the answers of
// two devices. The queries themselves (hipDeviceGetAttribute,
// hipFuncSetAttribute, hipOccupancyMaxActiveBlocksPerMultiprocessor) enqueue
// nothing on a stream, so a first use inside stream capture is also fine.
#include <hip/hip_runtime.h>

#include <map>
#include <mutex>
#include <tuple>

#include "internal.h"

namespace qg {

namespace {

struct Registry {
  std::mutex mu;
  std::map<int, int> cus;                                          // device -> CUs
  std::map<std::tuple<int, const void*, int, size_t>, int> per_cu;  // (device, kernel, threads, lds) -> WGs per CU
  std::map<std::pair<int, const void*>, bool> lds_raised;          // (device, kernel)
};

Registry& registry() {
  static Registry r;  // constructed once, thread-safely (C++11 static initialization)
  return r;
}

int current_device() {
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess) dev = 0;
  return dev;
}

int cus_locked(Registry& r, int dev) {
  auto it = r.cus.find(dev);
  if (it != r.cus.end()) return it->second;
  int c = 0;
  if (hipDeviceGetAttribute(&c, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || c <= 0) c = 256;
  r.cus[dev] = c;
  return c;
}

}  // namespace

int device_cus() {
  Registry& r = registry();
  const int dev = current_device();
  std::lock_guard<std::mutex> g(r.mu);
  return cus_locked(r, dev);
}

hipError_t kernel_residency(const void* kern, int threads, size_t lds, bool raise_lds, int* per_cu, int* cus) {
  Registry& r = registry();
  const int dev = current_device();
  std::lock_guard<std::mutex> g(r.mu);
  if (cus) *cus = cus_locked(r, dev);
  if (raise_lds) {
    auto key = std::make_pair(dev, kern);
    if (!r.lds_raised.count(key)) {
      hipError_t e = hipFuncSetAttribute(kern, hipFuncAttributeMaxDynamicSharedMemorySize, kLdsBytes);
      if (e != hipSuccess) return e;
      r.lds_raised[key] = true;
    }
  }
  auto key = std::make_tuple(dev, kern, threads, lds);
  auto it = r.per_cu.find(key);
  if (it != r.per_cu.end()) {
    *per_cu = it->second;
    return hipSuccess;
  }
  int nb = 0;
  if (hipOccupancyMaxActiveBlocksPerMultiprocessor(&nb, kern, threads, lds) != hipSuccess || nb < 1) nb = 1;
  r.per_cu[key] = nb;
  *per_cu = nb;
  return hipSuccess;
}

void clear_launch_cache() {
  Registry& r = registry();
  std::lock_guard<std::mutex> g(r.mu);
  r.cus.clear();
  r.per_cu.clear();
  r.lds_raised.clear();
}

}  // namespace qg
