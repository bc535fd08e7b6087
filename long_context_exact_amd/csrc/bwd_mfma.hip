// Backward of one chunk pair on gfx950 bf16 MFMA, from the saved final O
// and LSE ([DistFlashAttn §3.3]: checkpointing the attention output lets the
// attention backward reuse it, so the forward is never recomputed).  P is
// rebuilt from the saved LSE inside the kernels; nothing re-runs the forward
// kernel.
//
// Two deterministic kernels, each owning its outputs (no atomics):
//  dkdv_bf16_kernel  key-outer.  A workgroup owns 32*NW keys of one
//    key/value head (their K and V rows resident in LDS); wave w owns 32 of
//    them and accumulates dK^T, dV^T in VGPRs over every query head of the
//    group and every query row that sees the keys.  Per step of 32 query
//    rows (Q, dO staged straight from HBM into swizzled LDS, double-buffered):
//      S  = Q K^T,  dP = dO V^T            (lane = key, registers = rows)
//      P  = exp2(S*c - LSE2),  dS = P (dP - delta)
//      dV^T += dO^T P,  dK^T += Q^T dS     (A operand via transpose reads,
//                                           B straight from the accumulators)
//  dq_bf16_kernel    query-outer, shaped like the forward.  Per key tile:
//      S^T = K Q^T, dP^T = V dO^T          (lane = query row)
//      dS^T = P^T (dP^T - delta),  dQ^T += K^T dS^T
// Both add into the caller's fp32 accumulators (dq, dk, dv +=).  Pairs in
// which every query sees every key run mask-free instantiations (in dQ the
// key loop is also software-pipelined: the next block's S and dP are issued
// next to the current block's vector work).
#include <algorithm>
#include <cfloat>
#include <climits>

#include "bwd_common.hpp"

namespace dfa {

dfa_status launch_bwd_f32(const dfa_attn_desc& d, const void* q, const void* k, const void* v,
                          const float* lse, const void* d_o, const float* delta, float* dq,
                          float* dk, float* dv, hipStream_t s, int parts);

BwdArgs bwd_args_of(const dfa_attn_desc& d) {
  BwdArgs a{};
  a.len_q = d.len_q;
  a.len_kv = d.len_kv;
  a.q_start = d.q_start;
  a.kv_start = d.kv_start;
  a.hq = d.heads_q;
  a.hkv = d.heads_kv;
  a.group = d.heads_q / d.heads_kv;
  a.causal = d.causal;
  // c > 0 keeps exp2(fma(-inf, c, -lse2)) == 0 for hidden scores; a zero
  // scale runs as the smallest normal one (scores * 1.2e-38 round away in
  // fp32), and dQ, dK carry the true scale.
  a.c = std::max(d.scale * kLog2e, FLT_MIN);
  a.scale = d.scale;
  a.win = d.window > 0 ? d.window : kNoWindow;
  a.rsplit = 1;  // the dK/dV launcher may split rows
  a.ws = nullptr;
  a.band_lo = 0;  // and may run a pair as row bands
  a.band_hi = INT32_MAX;
  a.pair_wt = 0;
  a.rows_up = 0;
  a.keys_down = 0;
  return a;
}

int64_t bwd_workspace_bytes(const dfa_attn_desc& d) {
  if (d.dtype != DFA_BF16) return 0;
  return dkdv_workspace_bytes(d);
}

dfa_status launch_bwd(const dfa_attn_desc& d, const void* q, const void* k, const void* v,
                      const float* lse, const void* d_o, const float* delta, float* dq,
                      float* dk, float* dv, hipStream_t s, int parts) {
  if (d.dtype == DFA_F32)
    return launch_bwd_f32(d, q, k, v, lse, d_o, delta, dq, dk, dv, s, parts);
  BwdArgs a = bwd_args_of(d);
  a.q = static_cast<const uint16_t*>(q);
  a.k = static_cast<const uint16_t*>(k);
  a.v = static_cast<const uint16_t*>(v);
  a.d_o = static_cast<const uint16_t*>(d_o);
  a.lse = lse;
  a.delta = delta;
  a.dq = dq;
  a.dk = dk;
  a.dv = dv;
  if (parts & 1) {
    const dfa_status st = launch_dkdv_bf16(d, a, s);
    if (st != DFA_OK) return st;
  }
  return (parts & 2) ? launch_dq_bf16(d, a, s) : DFA_OK;
}

}  // namespace dfa
