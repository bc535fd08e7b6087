// dfa_attn_fwd_partial_noalloc: the forward of dfa_attn_fwd_partial with its
// scratch (the transposed V) in a fixed device array of this library instead
// of a caller workspace, for callers that cannot allocate device memory.
#include <mutex>
#include <string>

#include "kernels.hpp"

namespace dfa {
namespace {

// Largest transposed V the array holds: 64 MiB, the V^T of a 32768-key chunk
// of 8 key/value heads of 128 (the grouped-query 32K-chunk pair).
constexpr int64_t kNoAllocScratchBytes = int64_t(64) << 20;

// One copy per device, loaded with the library's code object and kept until
// the process ends.  In host code this name is not a device address: host
// code uses only the per-device address hipGetSymbolAddress returns.
__device__ __align__(256) unsigned char scratch[kNoAllocScratchBytes];

constexpr int kMaxDevices = 64;

struct DeviceScratch {
  std::once_flag once;
  void* ptr = nullptr;
  hipError_t err = hipSuccess;
};
DeviceScratch g_scratch[kMaxDevices];

// The address of `scratch` on the current device, resolved once per device
// with that device current.
dfa_status scratch_on_current_device(void** out) {
  int dev = -1;
  const hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess)
    return fail(DFA_ERR_HIP, std::string("dfa_attn_fwd_partial_noalloc: ") + hipGetErrorString(e));
  if (dev < 0 || dev >= kMaxDevices)
    return fail(DFA_ERR_UNSUPPORTED, "dfa_attn_fwd_partial_noalloc: device index past " +
                                         std::to_string(kMaxDevices));
  DeviceScratch& s = g_scratch[dev];
  std::call_once(s.once, [&s] {
    void* p = nullptr;
    s.err = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    if (s.err == hipSuccess) s.ptr = p;
  });
  if (s.err != hipSuccess || s.ptr == nullptr)
    return fail(DFA_ERR_HIP, std::string("dfa_attn_fwd_partial_noalloc: scratch address: ") +
                                 hipGetErrorString(s.err));
  *out = s.ptr;
  return DFA_OK;
}

}  // namespace
}  // namespace dfa

using namespace dfa;

extern "C" dfa_status dfa_attn_fwd_partial_noalloc(const dfa_attn_desc* desc, const void* q,
                                                   const void* k, const void* v, float* o_part,
                                                   float* lse, void* hip_stream) {
  try {
    if (desc == nullptr) return fail(DFA_ERR_INVALID, "dfa_attn_fwd_partial_noalloc: desc is null");
    dfa_attn_desc d = *desc;
    d.workspace = nullptr;
    d.workspace_bytes = 0;
    int64_t need = 0;
    const dfa_status st = dfa_attn_workspace_size(&d, DFA_OP_FWD, &need);
    if (st != DFA_OK) return st;
    if (need > kNoAllocScratchBytes)
      return fail(DFA_ERR_CAPACITY,
                  "dfa_attn_fwd_partial_noalloc: the transposed V needs " + std::to_string(need) +
                      " bytes; the library's fixed scratch holds " +
                      std::to_string(kNoAllocScratchBytes) + " (use dfa_attn_fwd_partial)");
    if (need > 0) {
      void* p = nullptr;
      const dfa_status sst = scratch_on_current_device(&p);
      if (sst != DFA_OK) return sst;
      d.workspace = p;
      d.workspace_bytes = kNoAllocScratchBytes;
    }
    return dfa_attn_fwd_partial(&d, q, k, v, o_part, lse, hip_stream);
  } catch (...) {
    return fail(DFA_ERR_INVALID, "dfa_attn_fwd_partial_noalloc: internal error");
  }
}
