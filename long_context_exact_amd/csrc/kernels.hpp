// Internal launch interface between the C ABI (api.hip) and the kernels.
#pragma once

#include "common.hpp"

namespace dfa {

// Forward of one chunk pair (bf16 -> MFMA kernel, f32 -> exact fp32 kernel).
// visits: optional tile-visit record (test support), else nullptr.
dfa_status launch_fwd(const dfa_attn_desc& d, const void* q, const void* k,
                      const void* v, float* o, float* lse, uint8_t* visits,
                      hipStream_t s);
void fwd_tile_shape(const dfa_attn_desc& d, int32_t* bm, int32_t* bn);

dfa_status launch_merge(int32_t n, const float* const* o_parts,
                        const float* const* lse_parts, int32_t batch,
                        int32_t heads, int64_t len_q, int32_t head_dim,
                        int32_t out_dtype, void* o_out, float* lse_out,
                        hipStream_t s);

dfa_status launch_delta(const dfa_attn_desc& d, const void* o, const void* d_o,
                        float* delta, hipStream_t s);

// parts: bit 0 = dK/dV kernel, bit 1 = dQ kernel (3 = the whole backward).
dfa_status launch_bwd(const dfa_attn_desc& d, const void* q, const void* k,
                      const void* v, const float* lse, const void* d_o,
                      const float* delta, float* dq, float* dk, float* dv,
                      hipStream_t s, int parts = 3);

// Opt a kernel into more than 64 KiB of dynamic LDS (gfx950 has 160 KiB).
template <typename K>
dfa_status allow_lds(K kernel, int bytes, const char* what) {
  if (bytes <= 65536) return DFA_OK;
  const hipError_t e = hipFuncSetAttribute(reinterpret_cast<const void*>(kernel),
                                           hipFuncAttributeMaxDynamicSharedMemorySize, bytes);
  if (e != hipSuccess) return fail(DFA_ERR_HIP, std::string(what) + ": " + hipGetErrorString(e));
  return DFA_OK;
}

// Sliding window in the kernels' arguments when the descriptor has none:
// larger than any token distance (positions are < 2^41), small enough that
// position arithmetic with it cannot overflow.
constexpr int64_t kNoWindow = int64_t(1) << 60;

// True when every query row of the pair sees every key (non-causal, or the
// key chunk ends at or before the first query) and the key chunk is a whole
// number of `tile` keys: such pairs need no mask anywhere.
inline bool pair_is_full(const dfa_attn_desc& d, int64_t tile) {
  const bool all_visible = !d.causal || d.kv_start + d.len_kv - 1 <= d.q_start;
  // a window must also reach from the last query back to the first key
  const bool in_window = d.window <= 0 || (d.q_start + d.len_q - 1) - d.kv_start < d.window;
  return all_visible && in_window && d.len_kv % tile == 0;
}

// Whether the pair's first query row sees more keys than its last one (a
// sliding window whose edge leaves the key chunk behind the later rows): the
// forward and dQ then hand out row tiles first to last instead of last to
// first, so that in either case the longest workgroups start first and the
// short ones fill the end of the launch.
inline bool rows_heaviest_first(const dfa_attn_desc& d) {
  if (d.len_q <= 0 || d.len_kv <= 0) return false;
  auto seen = [&](int64_t r) {  // keys visible to local query row r
    const int64_t q = d.q_start + r;
    int64_t hi = d.kv_start + d.len_kv - 1, lo = d.kv_start;
    if (d.causal && q < hi) hi = q;
    if (d.window > 0 && q - d.window + 1 > lo) lo = q - d.window + 1;
    return hi >= lo ? hi - lo + 1 : int64_t(0);
  };
  return seen(0) > seen(d.len_q - 1);
}

// Device workspace (bytes) the forward / backward of a descriptor needs:
// host arithmetic only (no HIP call), so the size query works anywhere.
int64_t fwd_workspace_bytes(const dfa_attn_desc& d);
int64_t bwd_workspace_bytes(const dfa_attn_desc& d);

// X [B][len][H][d] bf16 -> X^T [B][H][d][ld] (ld a multiple of 64, >= len):
// keys permuted within 16-key groups (index bits 2 and 3 swapped), keys past
// len zero.  The layout the forward reads V^T from for O^T += V^T P^T.
dfa_status launch_kv_transpose(const uint16_t* x, uint16_t* xt, int32_t batch, int64_t len,
                               int32_t heads, int32_t head_dim, int64_t ld, hipStream_t s);

// o = 0, lse = -inf for every row (a chunk pair with no keys).
dfa_status launch_fill_empty(int64_t n_o, float* o, int64_t n_lse, float* lse,
                             hipStream_t s);

}  // namespace dfa
