// Per-device properties the launchers size their grids from, cached once per
// device under a lock (calls may come from several host threads, each with its
// own current device).

#include <map>
#include <mutex>

#include "qn_internal.h"

namespace qn {

int device_cus() {
  static std::mutex mu;
  static std::map<int, int> cache;
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess) dev = 0;
  std::lock_guard<std::mutex> lk(mu);
  auto it = cache.find(dev);
  if (it != cache.end()) return it->second;
  int cus = 0;
  hipDeviceProp_t p;
  if (hipGetDeviceProperties(&p, dev) == hipSuccess) cus = p.multiProcessorCount;
  if (cus <= 0) cus = 256;
  cache[dev] = cus;
  return cus;
}

}  // namespace qn
