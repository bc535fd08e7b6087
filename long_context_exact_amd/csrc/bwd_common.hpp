// Arguments shared by the two bf16 backward kernels (dK/dV and dQ), each
// built from its own source file so that each gets its own compiler options.
#pragma once

#include <cfloat>

#include "kernels.hpp"

namespace dfa {

struct BwdArgs {
  const uint16_t* q;
  const uint16_t* k;
  const uint16_t* v;
  const uint16_t* d_o;
  const float* lse;
  const float* delta;
  float* dq;
  float* dk;
  float* dv;
  int64_t len_q, len_kv, q_start, kv_start;
  int32_t hq, hkv, group, causal;
  int32_t n_tiles, n_hgroups, n_ktiles;
  float c;      // scale * log2(e), > 0
  float scale;
  int64_t win;  // sliding window in tokens; a huge value when there is none
};

// LSE in base 2 for the exp2 form; a row without keys (LSE = -inf) gets +inf
// so that its P is exactly 0.
__device__ __forceinline__ float lse2_of(float lse) {
  return lse > -INFINITY ? lse * kLog2e : INFINITY;
}

#ifndef DFA_BWD_OCC
#define DFA_BWD_OCC 2  // waves per SIMD the register budget is sized for
#endif

// Launchers of the two kernels (head_dim 64 or 128, bf16 operands).
dfa_status launch_dkdv_bf16(const dfa_attn_desc& d, const BwdArgs& a, hipStream_t s);
dfa_status launch_dq_bf16(const dfa_attn_desc& d, const BwdArgs& a, hipStream_t s);

}  // namespace dfa
