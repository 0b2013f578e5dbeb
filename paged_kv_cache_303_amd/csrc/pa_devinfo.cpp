// Per-device facts that stay fixed while the process runs (compute-unit
// count, resident workgroups of a kernel instance), queried once and cached
// so that repeated launches of small batches make no runtime queries.
#include <hip/hip_runtime.h>

#include <map>
#include <mutex>
#include <tuple>

#include "pa_launch.h"

namespace pa {
namespace {
std::mutex g_mu;
std::map<int, int> g_cus;
std::map<std::tuple<int, const void*, size_t, int>, int> g_occ;
}  // namespace

pa_status current_device(int* dev) {
  return hipGetDevice(dev) == hipSuccess ? PA_OK : PA_ERR_HIP;
}

pa_status device_cus(int dev, int* cus) {
  std::lock_guard<std::mutex> lock(g_mu);
  auto it = g_cus.find(dev);
  if (it == g_cus.end()) {
    int n = 0;
    if (hipDeviceGetAttribute(&n, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess ||
        n < 1)
      return PA_ERR_HIP;
    it = g_cus.emplace(dev, n).first;
  }
  *cus = it->second;
  return PA_OK;
}

pa_status resident_per_cu(int dev, const void* kernel, int threads, size_t lds, int* per_cu) {
  std::lock_guard<std::mutex> lock(g_mu);
  const auto key = std::make_tuple(dev, kernel, lds, threads);
  auto it = g_occ.find(key);
  if (it == g_occ.end()) {
    int n = 0;
    if (hipOccupancyMaxActiveBlocksPerMultiprocessor(&n, kernel, threads, lds) != hipSuccess)
      return PA_ERR_HIP;
    it = g_occ.emplace(key, n).first;
  }
  *per_cu = it->second;
  return PA_OK;
}

}  // namespace pa
