// Library-owned device scratch: one buffer per (device, stream), grown on
// demand and kept until the process ends.  The kernels of one call use it in
// stream order, and calls on one stream are ordered, so a stream's buffer is
// never in use by two calls at once; calls on different streams get
// different buffers and may overlap.
#include <map>
#include <mutex>
#include <utility>

#include "kernels.hpp"

namespace dfa {

void* device_workspace(size_t bytes, hipStream_t stream) {
  struct Buf {
    void* ptr = nullptr;
    size_t cap = 0;
  };
  static std::mutex mu;
  static std::map<std::pair<int, hipStream_t>, Buf> bufs;
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess) return nullptr;
  std::lock_guard<std::mutex> lock(mu);
  Buf& b = bufs[{dev, stream}];
  if (b.cap >= bytes) return b.ptr;
  if (b.ptr != nullptr) {  // work queued on this stream with the old buffer must finish first
    if (hipStreamSynchronize(stream) != hipSuccess || hipFree(b.ptr) != hipSuccess) return nullptr;
    b.ptr = nullptr;
    b.cap = 0;
  }
  void* p = nullptr;
  if (hipMalloc(&p, bytes) != hipSuccess) {
    (void)hipGetLastError();
    return nullptr;
  }
  b.ptr = p;
  b.cap = bytes;
  return p;
}

}  // namespace dfa
