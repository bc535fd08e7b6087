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
  // dK/dV row split: each key block's steps are cut into rsplit slices run
  // by separate workgroups, which store their partial dK, dV to ws
  // ([2][rsplit][B][len_kv][Hkv][d] float32) for a fixed-order reduction;
  // rsplit = 1 adds straight into dk, dv.
  int32_t rsplit;
  float* ws;
  // dK/dV row band: of each key block's row tiles (its span below, from its
  // first visible row), only tiles [band_lo, band_hi) run in this launch, so
  // that one pair can run as bands of different kernels (0, INT32_MAX: all).
  int32_t band_lo, band_hi;
  // Paired launch of a windowed diagonal pair's two masked bands: the
  // window-edge rows start pair_wt row tiles past each key block's first row
  // (0 for every other launch).
  int32_t pair_wt;
  // Work order: dQ takes row tiles first to last (rows_up) instead of last to
  // first, dK/dV key blocks last to first (keys_down) instead of first to
  // last, when that puts the longest workgroups first.
  int32_t rows_up, keys_down;
};

// The query-row steps of the dK/dV workgroup owning keys [k_lo, k_lo + bk):
// rows from the first one at or after its first key to the last one whose
// window still reaches its last key, in blocks of bq rows (cut to the
// launch's row band), times the group's query heads.  Shared by the
// launcher, the kernel and the split reduction, so all three agree on which
// slices exist.
struct DkvSpan {
  int qt0, nq, steps;
};
__host__ __device__ inline DkvSpan dkdv_span(const BwdArgs& a, int64_t k_lo, int bk, int bq) {
  int64_t i_begin = 0;
  if (a.causal) i_begin = a.kv_start + k_lo - a.q_start > 0 ? a.kv_start + k_lo - a.q_start : 0;
  const int64_t k_last = (k_lo + bk < a.len_kv ? k_lo + bk : a.len_kv) - 1;
  int64_t i_end = a.kv_start + k_last + a.win - a.q_start;
  if (i_end > a.len_q) i_end = a.len_q;
  if (i_begin >= i_end) return {0, 0, 0};
  const int qt0 = int(i_begin / bq);
  const int nq = int((i_end + bq - 1) / bq) - qt0;
  const int lo = a.band_lo < nq ? a.band_lo : nq;
  const int hi = a.band_hi < nq ? a.band_hi : nq;
  if (lo >= hi) return {0, 0, 0};
  return {qt0 + lo, hi - lo, a.group * (hi - lo)};
}

// LSE in base 2 for the exp2 form; a row without keys (LSE = -inf) gets +inf
// so that its P is exactly 0.
__device__ __forceinline__ float lse2_of(float lse) {
  return lse > -INFINITY ? lse * kLog2e : INFINITY;
}

#ifndef DFA_BWD_OCC
#define DFA_BWD_OCC 2  // waves per SIMD the register budget is sized for
#endif

// The kernels' arguments for a descriptor (pointers left null).
BwdArgs bwd_args_of(const dfa_attn_desc& d);

// Row-split workspace of the dK/dV kernel: bytes of one slice's fp32 dK and
// dV partials, and the whole workspace the descriptor's split needs (0 when
// it does not split).
int64_t dkdv_split_bytes_per_slice(const dfa_attn_desc& d);
int64_t dkdv_workspace_bytes(const dfa_attn_desc& d);
// Launches of the dK/dV kernel for a descriptor (row bands make a diagonal
// pair's dK/dV two launches; 0 for an empty pair).  Host only.
int dkdv_launches(const dfa_attn_desc& d);
// Whether the dK/dV kernel takes the descriptor's key blocks last to first
// (its last block has more row steps than its first).  Host only.
bool dkdv_keys_down(const dfa_attn_desc& d);

// Launchers of the two kernels (head_dim 64 or 128, bf16 operands).
dfa_status launch_dkdv_bf16(const dfa_attn_desc& d, const BwdArgs& a, hipStream_t s);
dfa_status launch_dq_bf16(const dfa_attn_desc& d, const BwdArgs& a, hipStream_t s);

}  // namespace dfa
