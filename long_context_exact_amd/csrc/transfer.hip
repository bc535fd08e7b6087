// Emulated exchange of a chunk between two workers on one device: a copy
// on a DMA (system DMA) engine, which takes no compute units, standing in
// for the peer-to-peer send / receive of one schedule step.
#include <string>

#include "kernels.hpp"

using namespace dfa;

extern "C" dfa_status dfa_chunk_transfer(void* dst, const void* src, int64_t bytes,
                                         void* hip_stream) {
  try {
    const std::string f("dfa_chunk_transfer");
    if (bytes < 0) return fail(DFA_ERR_INVALID, f + ": bytes must be >= 0");
    if (bytes == 0) return DFA_OK;
    if (dst == nullptr || src == nullptr) return fail(DFA_ERR_INVALID, f + ": dst / src is null");
    const uintptr_t d = reinterpret_cast<uintptr_t>(dst), s = reinterpret_cast<uintptr_t>(src);
    if (d < s + uint64_t(bytes) && s < d + uint64_t(bytes))
      return fail(DFA_ERR_INVALID, f + ": dst and src overlap");
    const hipError_t e = hipMemcpyAsync(dst, src, size_t(bytes), hipMemcpyDeviceToDeviceNoCU,
                                        static_cast<hipStream_t>(hip_stream));
    if (e != hipSuccess) return fail(DFA_ERR_HIP, f + ": " + hipGetErrorString(e));
    return DFA_OK;
  } catch (...) {
    return fail(DFA_ERR_INVALID, "dfa_chunk_transfer: internal error");
  }
}
