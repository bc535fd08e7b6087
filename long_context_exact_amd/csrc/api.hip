// C ABI entry points of libdfa: argument checks (no HIP call before they
// pass), then dispatch to the kernels on the caller's stream.
#include <cstring>
#include <string>

#include "bwd_common.hpp"
#include "kernels.hpp"

namespace dfa {

dfa_status check_launch(const char* what) {
  const hipError_t e = hipGetLastError();
  if (e != hipSuccess)
    return fail(DFA_ERR_HIP, std::string(what) + ": " + hipGetErrorString(e));
  return DFA_OK;
}

namespace {

bool aligned16(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }

// Checks shared by every call that takes a descriptor.
dfa_status check_desc(const char* fn, const dfa_attn_desc* d) {
  const std::string f(fn);
  if (d == nullptr) return fail(DFA_ERR_INVALID, f + ": desc is null");
  if (d->batch < 0 || d->batch > 65535)
    return fail(DFA_ERR_INVALID, f + ": batch must be in [0, 65535]");
  if (d->heads_q < 1 || d->heads_kv < 1 || d->heads_q % d->heads_kv != 0)
    return fail(DFA_ERR_INVALID, f + ": heads_q must be a positive multiple of heads_kv >= 1");
  if (d->len_q < 0 || d->len_kv < 0 || d->q_start < 0 || d->kv_start < 0)
    return fail(DFA_ERR_INVALID, f + ": lengths and starts must be >= 0");
  if (d->causal != 0 && d->causal != 1) return fail(DFA_ERR_INVALID, f + ": causal must be 0 or 1");
  if (d->window < 0) return fail(DFA_ERR_INVALID, f + ": window must be >= 0");
  if (d->window > 0 && d->causal != 1)
    return fail(DFA_ERR_INVALID, f + ": a sliding window needs causal = 1");
  if (!std::isfinite(d->scale) || d->scale < 0.f)
    return fail(DFA_ERR_INVALID, f + ": scale must be finite and >= 0");
  if (d->dtype != DFA_F32 && d->dtype != DFA_BF16)
    return fail(DFA_ERR_INVALID, f + ": unknown dtype");
  if (d->head_dim != 64 && d->head_dim != 128)
    return fail(DFA_ERR_UNSUPPORTED,
                f + ": head_dim " + std::to_string(d->head_dim) + " unsupported (64 or 128)");
  // Kernels stage tiles of at most 256 rows through 32-bit byte offsets from
  // a tile base: 256 rows of heads_q * head_dim elements of up to 4 bytes
  // must stay below 2^31 bytes.
  if (int64_t(d->heads_q) * d->head_dim >= (int64_t(1) << 21))
    return fail(DFA_ERR_UNSUPPORTED,
                f + ": heads_q * head_dim must be below 2^21 (32-bit tile offsets)");
  if (d->len_q > (int64_t(1) << 40) || d->len_kv > (int64_t(1) << 40))
    return fail(DFA_ERR_INVALID, f + ": chunk length too large");
  // grid extents: row tiles x heads (with a margin) must fit a 32-bit grid
  if (cdiv(d->len_q, 4) * d->heads_q > INT32_MAX || cdiv(d->len_kv, 4) * d->heads_kv > INT32_MAX)
    return fail(DFA_ERR_INVALID, f + ": problem exceeds the launch grid");
  return DFA_OK;
}

dfa_status need(const std::string& fn, const void* p, const char* name, bool vec) {
  if (p == nullptr) return fail(DFA_ERR_INVALID, fn + ": " + name + " is null");
  if (vec && !aligned16(p))
    return fail(DFA_ERR_INVALID, fn + ": " + name + " must be 16-byte aligned");
  return DFA_OK;
}

// The caller's workspace must hold what the call needs (checked before any
// enqueue): DFA_ERR_CAPACITY names the required size.
dfa_status check_workspace(const std::string& fn, const dfa_attn_desc& d, int64_t need_bytes) {
  if (need_bytes <= 0) return DFA_OK;
  if (d.workspace_bytes < need_bytes || d.workspace == nullptr)
    return fail(DFA_ERR_CAPACITY, fn + ": workspace of " + std::to_string(need_bytes) +
                                      " bytes required (dfa_attn_workspace_size), " +
                                      std::to_string(d.workspace == nullptr ? 0 : d.workspace_bytes) +
                                      " given");
  if (!aligned16(d.workspace)) return fail(DFA_ERR_INVALID, fn + ": workspace must be 16-byte aligned");
  return DFA_OK;
}

#define DFA_TRY(expr)                    \
  do {                                   \
    const dfa_status _st = (expr);       \
    if (_st != DFA_OK) return _st;       \
  } while (0)

dfa_status fwd_common(const char* fn, const dfa_attn_desc* desc, const void* q, const void* k,
                      const void* v, float* o_part, float* lse, uint8_t* visits,
                      void* hip_stream) {
  DFA_TRY(check_desc(fn, desc));
  const dfa_attn_desc& d = *desc;
  const std::string f(fn);
  if (d.batch == 0 || d.len_q == 0) return DFA_OK;
  DFA_TRY(need(f, q, "q", true));
  DFA_TRY(need(f, o_part, "o_part", true));
  DFA_TRY(need(f, lse, "lse", false));
  const hipStream_t s = static_cast<hipStream_t>(hip_stream);
  if (d.len_kv == 0) {
    if (visits != nullptr) return DFA_OK;  // no key tiles: nothing visited
    return launch_fill_empty(int64_t(d.batch) * d.len_q * d.heads_q * d.head_dim, o_part,
                             int64_t(d.batch) * d.heads_q * d.len_q, lse, s);
  }
  DFA_TRY(need(f, k, "k", true));
  DFA_TRY(need(f, v, "v", true));
  DFA_TRY(check_workspace(f, d, fwd_workspace_bytes(d)));
  return launch_fwd(d, q, k, v, o_part, lse, visits, s);
}

}  // namespace
}  // namespace dfa

using namespace dfa;

extern "C" dfa_status dfa_attn_fwd_partial(const dfa_attn_desc* desc, const void* q,
                                           const void* k, const void* v, float* o_part,
                                           float* lse, void* hip_stream) {
  try {
    return fwd_common("dfa_attn_fwd_partial", desc, q, k, v, o_part, lse, nullptr, hip_stream);
  } catch (...) {
    return fail(DFA_ERR_INVALID, "dfa_attn_fwd_partial: internal error");
  }
}

extern "C" dfa_status dfa_lse_merge(int32_t n, const float* const* o_parts,
                                    const float* const* lse_parts, int32_t batch, int32_t heads,
                                    int64_t len_q, int32_t head_dim, int32_t out_dtype,
                                    void* o_out, float* lse_out, void* hip_stream) {
  try {
    const std::string f("dfa_lse_merge");
    if (n < 1 || n > 64) return fail(DFA_ERR_INVALID, f + ": n must be in [1, 64]");
    if (o_parts == nullptr || lse_parts == nullptr)
      return fail(DFA_ERR_INVALID, f + ": o_parts / lse_parts arrays are null");
    if (batch < 0 || heads < 1 || len_q < 0)
      return fail(DFA_ERR_INVALID, f + ": batch >= 0, heads >= 1, len_q >= 0 required");
    if (out_dtype != DFA_F32 && out_dtype != DFA_BF16)
      return fail(DFA_ERR_INVALID, f + ": unknown out_dtype");
    if (head_dim != 64 && head_dim != 128)
      return fail(DFA_ERR_UNSUPPORTED, f + ": head_dim must be 64 or 128");
    if (int64_t(batch) * len_q * heads * (head_dim / 4) > (int64_t(INT32_MAX) * 256))
      return fail(DFA_ERR_INVALID, f + ": problem exceeds the launch grid");
    if (batch == 0 || len_q == 0) return DFA_OK;
    for (int r = 0; r < n; ++r) {
      DFA_TRY(need(f, o_parts[r], "o_parts[r]", true));
      DFA_TRY(need(f, lse_parts[r], "lse_parts[r]", false));
      if (static_cast<const void*>(o_parts[r]) == o_out && (r > 0 || out_dtype != DFA_F32))
        return fail(DFA_ERR_INVALID,
                    f + ": o_out may alias only o_parts[0], and only with DFA_F32 output");
      if (r > 0 && lse_parts[r] == lse_out)
        return fail(DFA_ERR_INVALID, f + ": lse_out may alias only lse_parts[0]");
    }
    DFA_TRY(need(f, o_out, "o_out", out_dtype == DFA_F32));
    if (out_dtype == DFA_BF16 && (reinterpret_cast<uintptr_t>(o_out) & 7u))
      return fail(DFA_ERR_INVALID, f + ": o_out must be 8-byte aligned");
    DFA_TRY(need(f, lse_out, "lse_out", false));
    return launch_merge(n, o_parts, lse_parts, batch, heads, len_q, head_dim, out_dtype, o_out,
                        lse_out, static_cast<hipStream_t>(hip_stream));
  } catch (...) {
    return fail(DFA_ERR_INVALID, "dfa_lse_merge: internal error");
  }
}

namespace dfa {
namespace {
dfa_status bwd_common(const char* fn, const dfa_attn_desc* desc, const void* q, const void* k,
                      const void* v, const void* o, const float* lse, const void* d_o,
                      float* delta, int32_t compute_delta, float* dq, float* dk, float* dv,
                      void* hip_stream, int parts) {
  const std::string f(fn);
  DFA_TRY(check_desc(fn, desc));
  const dfa_attn_desc& d = *desc;
  if (compute_delta != 0 && compute_delta != 1)
    return fail(DFA_ERR_INVALID, f + ": compute_delta must be 0 or 1");
  if (d.batch == 0 || d.len_q == 0) return DFA_OK;  // no query rows: nothing to write
  DFA_TRY(need(f, d_o, "d_o", true));
  DFA_TRY(need(f, delta, "delta", false));
  if (compute_delta) DFA_TRY(need(f, o, "o", true));
  const hipStream_t s = static_cast<hipStream_t>(hip_stream);
  if (d.len_kv == 0) {
    // No keys: nothing to add to dq, dk, dv, but delta (which later pairs of
    // the query chunk read) is still written when asked for.
    return compute_delta ? launch_delta(d, o, d_o, delta, s) : DFA_OK;
  }
  DFA_TRY(need(f, q, "q", true));
  DFA_TRY(need(f, k, "k", true));
  DFA_TRY(need(f, v, "v", true));
  DFA_TRY(need(f, lse, "lse", false));
  if (parts & 2) DFA_TRY(need(f, dq, "dq", true));
  if (parts & 1) DFA_TRY(need(f, dk, "dk", true));
  if (parts & 1) DFA_TRY(need(f, dv, "dv", true));
  if (parts & 1) DFA_TRY(check_workspace(f, d, bwd_workspace_bytes(d)));
  if (compute_delta) DFA_TRY(launch_delta(d, o, d_o, delta, s));
  return launch_bwd(d, q, k, v, lse, d_o, delta, dq, dk, dv, s, parts);
}
}  // namespace
}  // namespace dfa

extern "C" dfa_status dfa_attn_bwd(const dfa_attn_desc* desc, const void* q, const void* k,
                                   const void* v, const void* o, const float* lse,
                                   const void* d_o, float* delta, int32_t compute_delta,
                                   float* dq, float* dk, float* dv, void* hip_stream) {
  try {
    return bwd_common("dfa_attn_bwd", desc, q, k, v, o, lse, d_o, delta, compute_delta, dq, dk,
                      dv, hip_stream, 3);
  } catch (...) {
    return fail(DFA_ERR_INVALID, "dfa_attn_bwd: internal error");
  }
}

extern "C" dfa_status dfa_test_bwd_part(const dfa_attn_desc* desc, const void* q, const void* k,
                                        const void* v, const float* lse, const void* d_o,
                                        const float* delta, float* dq, float* dk, float* dv,
                                        int32_t part, void* hip_stream) {
  try {
    if (part != 1 && part != 2)
      return fail(DFA_ERR_INVALID, "dfa_test_bwd_part: part must be 1 or 2");
    return bwd_common("dfa_test_bwd_part", desc, q, k, v, nullptr, lse, d_o,
                      const_cast<float*>(delta), 0, dq, dk, dv, hip_stream, part);
  } catch (...) {
    return fail(DFA_ERR_INVALID, "dfa_test_bwd_part: internal error");
  }
}

extern "C" dfa_status dfa_test_bwd_launches(const dfa_attn_desc* desc, int32_t part,
                                            int32_t* launches) {
  try {
    DFA_TRY(check_desc("dfa_test_bwd_launches", desc));
    if (part != 1 && part != 2)
      return fail(DFA_ERR_INVALID, "dfa_test_bwd_launches: part must be 1 or 2");
    if (launches == nullptr) return fail(DFA_ERR_INVALID, "dfa_test_bwd_launches: launches is null");
    const dfa_attn_desc& d = *desc;
    const bool empty = d.batch == 0 || d.len_q == 0 || d.len_kv == 0;
    *launches = part == 1 ? dkdv_launches(d) : (empty ? 0 : 1);
    return DFA_OK;
  } catch (...) {
    return fail(DFA_ERR_INVALID, "dfa_test_bwd_launches: internal error");
  }
}

extern "C" dfa_status dfa_test_work_order(const dfa_attn_desc* desc, int32_t* rows_first_to_last,
                                          int32_t* keys_last_to_first) {
  try {
    DFA_TRY(check_desc("dfa_test_work_order", desc));
    if (rows_first_to_last == nullptr || keys_last_to_first == nullptr)
      return fail(DFA_ERR_INVALID, "dfa_test_work_order: output pointer is null");
    *rows_first_to_last = rows_heaviest_first(*desc) ? 1 : 0;
    *keys_last_to_first = dkdv_keys_down(*desc) ? 1 : 0;
    return DFA_OK;
  } catch (...) {
    return fail(DFA_ERR_INVALID, "dfa_test_work_order: internal error");
  }
}

extern "C" dfa_status dfa_attn_workspace_size(const dfa_attn_desc* desc, int32_t op,
                                              int64_t* bytes) {
  try {
    DFA_TRY(check_desc("dfa_attn_workspace_size", desc));
    if (bytes == nullptr) return fail(DFA_ERR_INVALID, "dfa_attn_workspace_size: bytes is null");
    if (op == DFA_OP_FWD)
      *bytes = fwd_workspace_bytes(*desc);
    else if (op == DFA_OP_BWD)
      *bytes = bwd_workspace_bytes(*desc);
    else
      return fail(DFA_ERR_INVALID, "dfa_attn_workspace_size: op must be DFA_OP_FWD or DFA_OP_BWD");
    return DFA_OK;
  } catch (...) {
    return fail(DFA_ERR_INVALID, "dfa_attn_workspace_size: internal error");
  }
}

extern "C" int32_t dfa_version(void) { return 10100; }

extern "C" dfa_status dfa_test_tile_shape(const dfa_attn_desc* desc, int32_t* bm, int32_t* bn) {
  DFA_TRY(check_desc("dfa_test_tile_shape", desc));
  if (bm == nullptr || bn == nullptr)
    return fail(DFA_ERR_INVALID, "dfa_test_tile_shape: bm / bn are null");
  fwd_tile_shape(*desc, bm, bn);
  return DFA_OK;
}

extern "C" dfa_status dfa_test_fwd_tile_visits(const dfa_attn_desc* desc, const void* q,
                                               const void* k, const void* v, float* o_part,
                                               float* lse, uint8_t* visits, void* hip_stream) {
  try {
    DFA_TRY(check_desc("dfa_test_fwd_tile_visits", desc));
    if (desc->dtype != DFA_BF16)
      return fail(DFA_ERR_UNSUPPORTED, "dfa_test_fwd_tile_visits: bf16 (tiled) path only");
    if (visits == nullptr) return fail(DFA_ERR_INVALID, "dfa_test_fwd_tile_visits: visits is null");
    return fwd_common("dfa_test_fwd_tile_visits", desc, q, k, v, o_part, lse, visits,
                      hip_stream);
  } catch (...) {
    return fail(DFA_ERR_INVALID, "dfa_test_fwd_tile_visits: internal error");
  }
}
