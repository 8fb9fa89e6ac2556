// Per-device facts the launchers need, looked up once per device and kept
// for the life of the process: the compute-unit count (persistent kernels
// size their grids by it) and each kernel's dynamic-LDS limit (raised with
// hipFuncSetAttribute before the first launch that needs more than 64 KiB).
// Both tables are guarded by one mutex, so launchers may run on several
// host threads and devices at once.

#include <hip/hip_runtime_api.h>

#include <mutex>
#include <vector>

#include "msa_kernels.h"

namespace msa {
namespace {

struct LdsAttr {
  int dev;
  const void* fn;
  int bytes;  // the largest limit set so far for (dev, fn)
};

std::mutex g_mu;
std::vector<int> g_cu;  // by device ordinal; 0 = not yet queried
std::vector<LdsAttr> g_lds;

}  // namespace

hipError_t current_cu_count(int* n_cu) {
  int dev = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return e;
  std::lock_guard<std::mutex> g(g_mu);
  if ((int)g_cu.size() <= dev) g_cu.resize(dev + 1, 0);
  if (g_cu[dev] == 0) {
    int n = 0;
    e = hipDeviceGetAttribute(&n, hipDeviceAttributeMultiprocessorCount, dev);
    if (e != hipSuccess) return e;
    g_cu[dev] = n > 0 ? n : 1;
  }
  *n_cu = g_cu[dev];
  return hipSuccess;
}

hipError_t ensure_dynamic_lds(const void* fn, int bytes) {
  int dev = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return e;
  std::lock_guard<std::mutex> g(g_mu);
  for (LdsAttr& a : g_lds) {
    if (a.dev != dev || a.fn != fn) continue;
    if (a.bytes >= bytes) return hipSuccess;
    e = hipFuncSetAttribute(fn, hipFuncAttributeMaxDynamicSharedMemorySize, bytes);
    if (e == hipSuccess) a.bytes = bytes;
    return e;
  }
  e = hipFuncSetAttribute(fn, hipFuncAttributeMaxDynamicSharedMemorySize, bytes);
  if (e == hipSuccess) g_lds.push_back({dev, fn, bytes});
  return e;
}

}  // namespace msa
