// Library-owned device scratch, one buffer per device, grown on demand and
// kept until the process ends.  Kernels of one call use it in stream order;
// calls that use it must therefore be ordered on one device (one stream).
#include <mutex>

#include "kernels.hpp"

namespace dfa {

void* device_workspace(size_t bytes) {
  static std::mutex mu;
  static void* ptr[64] = {};
  static size_t cap[64] = {};
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= 64) return nullptr;
  std::lock_guard<std::mutex> lock(mu);
  if (cap[dev] >= bytes) return ptr[dev];
  if (ptr[dev] != nullptr) {  // work queued with the old buffer must finish first
    if (hipDeviceSynchronize() != hipSuccess || hipFree(ptr[dev]) != hipSuccess) return nullptr;
    ptr[dev] = nullptr;
    cap[dev] = 0;
  }
  void* p = nullptr;
  if (hipMalloc(&p, bytes) != hipSuccess) {
    (void)hipGetLastError();
    return nullptr;
  }
  ptr[dev] = p;
  cap[dev] = bytes;
  return p;
}

}  // namespace dfa
