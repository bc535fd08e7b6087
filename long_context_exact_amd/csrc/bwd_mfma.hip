// Backward of one chunk pair on gfx950 bf16 MFMA, from the saved final O
// and LSE ([DistFlashAttn §3.3]: checkpointing the attention output lets the
// attention backward reuse it, so the forward is never recomputed).  P is
// rebuilt from the saved LSE inside the kernels; nothing re-runs the forward
// kernel.
//
// Two deterministic kernels, each owning its outputs (no atomics):
//  dkdv_bf16_kernel  key-outer.  A workgroup owns 32*NW keys of one
//    key/value head; wave w owns 32 of them with K, V held as MFMA operands
//    in VGPRs and dK^T, dV^T accumulated in VGPRs over every query head of
//    the group and every query row that sees the keys.  Per step of BQ
//    query rows (Q, dO row-major and swizzled in LDS, double-buffered):
//      S  = Q K^T,  dP = dO V^T            (lane = key, registers = rows)
//      P  = exp2(S*c - LSE2),  dS = P (dP - delta)
//      dV^T += dO^T P,  dK^T += Q^T dS     (A operand via transpose reads,
//                                           B straight from the accumulators)
//  dq_bf16_kernel    query-outer, shaped like the forward.  Per key tile:
//      S^T = K Q^T, dP^T = V dO^T          (lane = query row)
//      dS^T = P^T (dP^T - delta),  dQ^T += K^T dS^T
// Both add into the caller's fp32 accumulators (dq, dk, dv +=).
#include <algorithm>
#include <cfloat>

#include "kernels.hpp"

namespace dfa {
namespace {

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
};

// LSE in base 2 for the exp2 form; a row without keys (LSE = -inf) gets +inf
// so that its P is exactly 0.
__device__ __forceinline__ float lse2_of(float lse) {
  return lse > -INFINITY ? lse * kLog2e : INFINITY;
}

// ---------------------------------------------------------------- dK, dV
template <int D, int NW, int BQ>
struct DkvCfg {
  static constexpr int NT = NW * 64;
  static constexpr int BK = 32 * NW;   // keys per workgroup
  static constexpr int CH = BQ * D / 8;
  static constexpr int CPT = CH / NT;
  static constexpr int TILE = BQ * D;  // elements of one Q (or dO) tile
  // stage: Q tile, dO tile, then BQ floats of LSE2 and BQ floats of delta
  static constexpr int STAGE_BYTES = 2 * TILE * 2 + 2 * BQ * 4;
  static constexpr int LDS_BYTES = 2 * STAGE_BYTES;
  static_assert(CH % NT == 0, "query tile chunks must divide evenly");
  static_assert(2 * BQ <= NT, "one thread per LSE / delta value");
};

template <int D, int NW, int BQ>
__global__ __launch_bounds__(NW * 64) void dkdv_bf16_kernel(BwdArgs a) {
  using C = DkvCfg<D, NW, BQ>;
  extern __shared__ __align__(16) uint16_t smem_generic[];
  lds_u16* smem = lds_base(smem_generic);

  const int tid = threadIdx.x;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);  // wave-uniform (scalar)
  const int lane = tid & 63;
  const int l32 = lane & 31, hi = lane >> 5;
  const int half16 = (lane >> 4) & 1;
  const int kt = blockIdx.x / a.hkv;
  const int g = blockIdx.x % a.hkv;
  const int64_t b = blockIdx.y;
  const int64_t k_lo = int64_t(kt) * C::BK;
  const int64_t wk_lo = k_lo + wave * 32;
  const int64_t wk_hi = min(wk_lo + 32, a.len_kv);
  const bool wave_active = wk_lo < a.len_kv;
  const int64_t key = wk_lo + l32;

  const int64_t q_rs = int64_t(a.hq) * D;
  const int64_t kv_rs = int64_t(a.hkv) * D;

  bf16x8 kf[D / 16], vf[D / 16];
  {
    const uint16_t* kp = a.k + (b * a.len_kv + key) * kv_rs + int64_t(g) * D;
    const uint16_t* vp = a.v + (b * a.len_kv + key) * kv_rs + int64_t(g) * D;
#pragma unroll
    for (int st = 0; st < D / 16; ++st) {
      if (key < a.len_kv) {
        kf[st] = ld_bf16x8(kp + 16 * st + 8 * hi);
        vf[st] = ld_bf16x8(vp + 16 * st + 8 * hi);
      } else {
        kf[st] = bf16x8{};
        vf[st] = bf16x8{};
      }
    }
  }

  // Query rows that see at least one key of this workgroup.
  int64_t i_begin = 0;
  if (a.causal) i_begin = max<int64_t>(0, a.kv_start + k_lo - a.q_start);
  if (i_begin >= a.len_q) return;  // uniform over the workgroup
  const int qt0 = int(i_begin / BQ);
  const int nq = int(cdiv(a.len_q, BQ)) - qt0;
  const int steps = a.group * nq;

  f32x16 dk_acc[D / 32], dv_acc[D / 32];
#pragma unroll
  for (int db = 0; db < D / 32; ++db) {
    dk_acc[db] = f32x16{};
    dv_acc[db] = f32x16{};
  }

  uint4 qreg[C::CPT], dreg[C::CPT];
  float sreg = 0.f;
  auto gload = [&](int it) {
    const int h = g * a.group + it / nq;
    const int64_t i0 = int64_t(qt0 + it % nq) * BQ;
    const uint16_t* qb = a.q + b * a.len_q * q_rs + int64_t(h) * D;
    const uint16_t* db_ = a.d_o + b * a.len_q * q_rs + int64_t(h) * D;
#pragma unroll
    for (int i = 0; i < C::CPT; ++i) {
      const int c = tid + i * C::NT;
      const int r = c / (D / 8), dc = c % (D / 8);
      const int64_t row = i0 + r;
      if (row < a.len_q) {
        qreg[i] = ld_u4(qb + row * q_rs + 8 * dc);
        dreg[i] = ld_u4(db_ + row * q_rs + 8 * dc);
      } else {
        qreg[i] = make_uint4(0, 0, 0, 0);
        dreg[i] = make_uint4(0, 0, 0, 0);
      }
    }
    if (tid < 2 * BQ) {
      const int64_t row = i0 + (tid % BQ);
      const int64_t li = (b * a.hq + h) * a.len_q + row;
      if (tid < BQ) sreg = row < a.len_q ? lse2_of(a.lse[li]) : INFINITY;
      else sreg = row < a.len_q ? a.delta[li] : 0.f;
    }
  };
  auto stage_ptr = [&](int stage) {
    return smem + stage * (C::STAGE_BYTES / 2);
  };
  auto sstore = [&](int stage) {
    lds_u16* Qs = stage_ptr(stage);
    lds_u16* dOs = Qs + C::TILE;
    lds_f32* sv = (lds_f32*)(dOs + C::TILE);
#pragma unroll
    for (int i = 0; i < C::CPT; ++i) {
      const int c = tid + i * C::NT;
      const int r = c / (D / 8), dc = c % (D / 8);
      tile_store16<D>(Qs, r, dc, qreg[i]);
      tile_store16<D>(dOs, r, dc, dreg[i]);
    }
    if (tid < 2 * BQ) sv[tid] = sreg;
  };

  gload(0);
  sstore(0);
  __syncthreads();

  for (int it = 0; it < steps; ++it) {
    if (it + 1 < steps) gload(it + 1);
    const lds_u16* Qs = stage_ptr(it & 1);
    const lds_u16* dOs = Qs + C::TILE;
    const lds_f32* lse2s = (const lds_f32*)(dOs + C::TILE);
    const lds_f32* dls = lse2s + BQ;
    const int64_t i0 = int64_t(qt0 + it % nq) * BQ;
#pragma unroll 1
    for (int qb = 0; qb < BQ / 32; ++qb) {
      const int64_t r0 = i0 + 32 * qb;  // first row of this 32-row block
      bool any = wave_active && r0 < a.len_q;
      if (any && a.causal) any = a.q_start + min(r0 + 32, a.len_q) - 1 >= a.kv_start + wk_lo;
      if (!any) continue;
      const bool need_mask = (a.causal && a.q_start + r0 < a.kv_start + wk_hi - 1) ||
                             (r0 + 32 > a.len_q) || (wk_lo + 32 > a.len_kv);
      f32x16 s = f32x16{}, dp = f32x16{};
#pragma unroll
      for (int st = 0; st < D / 16; ++st) {
        s = mfma32(tile_row8<D>(Qs, 32 * qb + l32, 2 * st + hi), kf[st], s);
        dp = mfma32(tile_row8<D>(dOs, 32 * qb + l32, 2 * st + hi), vf[st], dp);
      }
      // row (local to the block) of register r: 8 * (r / 4) + 4 * hi + r % 4
      const int64_t rmin = a.causal ? a.kv_start + key - a.q_start - r0 : INT64_MIN / 2;
      const int64_t rmax = a.len_q - 1 - r0;
      const bool key_ok = key < a.len_kv;
      if (need_mask) {  // hidden scores -> -inf, so P = exp2(-inf) = 0 (c > 0)
#pragma unroll
        for (int r = 0; r < 16; ++r) {
          const int ri = 8 * (r >> 2) + 4 * hi + (r & 3);
          if (!key_ok || ri < rmin || ri > rmax) s[r] = -INFINITY;
        }
      }
#pragma unroll
      for (int r4 = 0; r4 < 4; ++r4) {
        const f32x4 x = *(const DFA_LDS f32x4*)(lse2s + 32 * qb + 8 * r4 + 4 * hi);
        const f32x4 y = *(const DFA_LDS f32x4*)(dls + 32 * qb + 8 * r4 + 4 * hi);
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          const int r = 4 * r4 + e;
          const float p = exp2_fast(fmaf(s[r], a.c, -x[e]));
          s[r] = p;
          dp[r] = p * (dp[r] - y[e]);
        }
      }
#pragma unroll
      for (int j = 0; j < 2; ++j) {
        bf16x8 pb, sb;
#pragma unroll
        for (int e = 0; e < 8; ++e) {
          pb[e] = static_cast<__bf16>(s[8 * j + e]);
          sb[e] = static_cast<__bf16>(dp[8 * j + e]);
        }
        const int t0 = 32 * qb + 16 * j + 4 * hi;
#pragma unroll
        for (int db = 0; db < D / 32; ++db) {
          const int c0 = 32 * db + 16 * half16;
          const bf16x8 ta =
              cat4(tile_tr4<D>(dOs, t0, c0, lane), tile_tr4<D>(dOs, t0 + 8, c0, lane));
          dv_acc[db] = mfma32(ta, pb, dv_acc[db]);
          const bf16x8 ua = cat4(tile_tr4<D>(Qs, t0, c0, lane), tile_tr4<D>(Qs, t0 + 8, c0, lane));
          dk_acc[db] = mfma32(ua, sb, dk_acc[db]);
        }
      }
    }
    if (it + 1 < steps) sstore((it + 1) & 1);
    __syncthreads();
  }

  if (!wave_active || key >= a.len_kv) return;
  float* dkr = a.dk + (b * a.len_kv + key) * kv_rs + int64_t(g) * D;
  float* dvr = a.dv + (b * a.len_kv + key) * kv_rs + int64_t(g) * D;
#pragma unroll
  for (int db = 0; db < D / 32; ++db)
#pragma unroll
    for (int r4 = 0; r4 < 4; ++r4) {
      const int d = 32 * db + 8 * r4 + 4 * hi;
      f32x4 xk = *reinterpret_cast<f32x4*>(dkr + d);
      f32x4 xv = *reinterpret_cast<f32x4*>(dvr + d);
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        xk[e] += a.scale * dk_acc[db][4 * r4 + e];
        xv[e] += dv_acc[db][4 * r4 + e];
      }
      *reinterpret_cast<f32x4*>(dkr + d) = xk;
      *reinterpret_cast<f32x4*>(dvr + d) = xv;
    }
}

// Variant of the key-outer kernel for two waves per SIMD: the workgroup's
// K and V rows live in LDS (read as MFMA operands) instead of VGPRs, which
// leaves the register budget to the dK^T / dV^T accumulators.  NW waves own
// 32*NW keys; steps of 32 query rows, single-buffered with a register
// prefetch of the next step.
template <int D, int NW>
struct DkvLdsCfg {
  static constexpr int NT = NW * 64;
  static constexpr int BK = 32 * NW;
  static constexpr int BQ = 32;
  static constexpr int KV_TILE = BK * D;   // elements of the K (or V) tile
  static constexpr int Q_TILE = BQ * D;
  static constexpr int LDS_BYTES = (2 * KV_TILE + 2 * Q_TILE) * 2 + 2 * BQ * 4;
  static constexpr int QCPT = Q_TILE / 8 / NT;   // 16-byte chunks per thread (Q or dO)
  static constexpr int KCPT = KV_TILE / 8 / NT;  // chunks per thread (K or V)
  static_assert(QCPT >= 1 && Q_TILE / 8 % NT == 0, "query chunks must divide evenly");
  static_assert(KV_TILE / 8 % NT == 0, "key chunks must divide evenly");
};

#ifndef DFA_DKDV_OCC
#define DFA_DKDV_OCC 2
#endif

template <int D, int NW>
__global__ __launch_bounds__(NW * 64) __attribute__((amdgpu_waves_per_eu(DFA_DKDV_OCC, DFA_DKDV_OCC)))
void dkdv_lds_bf16_kernel(BwdArgs a) {
  using C = DkvLdsCfg<D, NW>;
  extern __shared__ __align__(16) uint16_t smem_generic[];
  lds_u16* smem = lds_base(smem_generic);
  lds_u16* Ks = smem;
  lds_u16* Vs = Ks + C::KV_TILE;
  lds_u16* Qs = Vs + C::KV_TILE;
  lds_u16* dOs = Qs + C::Q_TILE;
  lds_f32* lse2s = (lds_f32*)(dOs + C::Q_TILE);
  lds_f32* dls = lse2s + C::BQ;

  const int tid = threadIdx.x;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);  // wave-uniform (scalar)
  const int lane = tid & 63;
  const int l32 = lane & 31, hi = lane >> 5;
  const int half16 = (lane >> 4) & 1;
  const int kt = blockIdx.x / a.hkv;
  const int g = blockIdx.x % a.hkv;
  const int64_t b = blockIdx.y;
  const int64_t k_lo = int64_t(kt) * C::BK;
  const int64_t wk_lo = k_lo + wave * 32;
  const int64_t wk_hi = min(wk_lo + 32, a.len_kv);
  const bool wave_active = wk_lo < a.len_kv;
  const int64_t key = wk_lo + l32;

  const int64_t q_rs = int64_t(a.hq) * D;
  const int64_t kv_rs = int64_t(a.hkv) * D;

  int64_t i_begin = 0;
  if (a.causal) i_begin = max<int64_t>(0, a.kv_start + k_lo - a.q_start);
  if (i_begin >= a.len_q) return;  // uniform over the workgroup
  const int qt0 = int(i_begin / C::BQ);
  const int nq = int(cdiv(a.len_q, C::BQ)) - qt0;
  const int steps = a.group * nq;

  // The workgroup's K and V rows, once.
  {
    const uint16_t* kb = a.k + b * a.len_kv * kv_rs + int64_t(g) * D;
    const uint16_t* vb = a.v + b * a.len_kv * kv_rs + int64_t(g) * D;
#pragma unroll 1
    for (int i = 0; i < C::KCPT; ++i) {
      const int c = tid + i * C::NT;
      const int r = c / (D / 8), dc = c % (D / 8);
      const int64_t kk = k_lo + r;
      uint4 x = make_uint4(0, 0, 0, 0), y = make_uint4(0, 0, 0, 0);
      if (kk < a.len_kv) {
        x = ld_u4(kb + kk * kv_rs + 8 * dc);
        y = ld_u4(vb + kk * kv_rs + 8 * dc);
      }
      tile_store16<D>(Ks, r, dc, x);
      tile_store16<D>(Vs, r, dc, y);
    }
  }

  f32x16 dk_acc[D / 32], dv_acc[D / 32];
#pragma unroll
  for (int db = 0; db < D / 32; ++db) {
    dk_acc[db] = f32x16{};
    dv_acc[db] = f32x16{};
  }

  uint4 qreg[C::QCPT], dreg[C::QCPT];
  float sreg = 0.f;
  auto gload = [&](int it) {
    const int h = g * a.group + it / nq;
    const int64_t i0 = int64_t(qt0 + it % nq) * C::BQ;
    const uint16_t* qb = a.q + b * a.len_q * q_rs + int64_t(h) * D;
    const uint16_t* db_ = a.d_o + b * a.len_q * q_rs + int64_t(h) * D;
#pragma unroll
    for (int i = 0; i < C::QCPT; ++i) {
      const int c = tid + i * C::NT;
      const int r = c / (D / 8), dc = c % (D / 8);
      const int64_t row = i0 + r;
      if (row < a.len_q) {
        qreg[i] = ld_u4(qb + row * q_rs + 8 * dc);
        dreg[i] = ld_u4(db_ + row * q_rs + 8 * dc);
      } else {
        qreg[i] = make_uint4(0, 0, 0, 0);
        dreg[i] = make_uint4(0, 0, 0, 0);
      }
    }
    if (tid < 2 * C::BQ) {
      const int64_t row = i0 + (tid % C::BQ);
      const int64_t li = (b * a.hq + h) * a.len_q + row;
      if (tid < C::BQ) sreg = row < a.len_q ? lse2_of(a.lse[li]) : INFINITY;
      else sreg = row < a.len_q ? a.delta[li] : 0.f;
    }
  };
  auto sstore = [&]() {
#pragma unroll
    for (int i = 0; i < C::QCPT; ++i) {
      const int c = tid + i * C::NT;
      const int r = c / (D / 8), dc = c % (D / 8);
      tile_store16<D>(Qs, r, dc, qreg[i]);
      tile_store16<D>(dOs, r, dc, dreg[i]);
    }
    if (tid < C::BQ) lse2s[tid] = sreg;
    else if (tid < 2 * C::BQ) dls[tid - C::BQ] = sreg;
  };

  gload(0);
  sstore();
  __syncthreads();

#pragma unroll 1
  for (int it = 0; it < steps; ++it) {
    if (it + 1 < steps) gload(it + 1);
    const int64_t r0 = int64_t(qt0 + it % nq) * C::BQ;
    bool any = wave_active;
    if (any && a.causal) any = a.q_start + min(r0 + C::BQ, a.len_q) - 1 >= a.kv_start + wk_lo;
    if (any) {
      const bool need_mask = (a.causal && a.q_start + r0 < a.kv_start + wk_hi - 1) ||
                             (r0 + C::BQ > a.len_q) || (wk_lo + 32 > a.len_kv);
      f32x16 s = f32x16{}, dp = f32x16{};
#pragma unroll
      for (int st = 0; st < D / 16; ++st) {
        s = mfma32(tile_row8<D>(Qs, l32, 2 * st + hi), tile_row8<D>(Ks, wave * 32 + l32, 2 * st + hi), s);
        dp = mfma32(tile_row8<D>(dOs, l32, 2 * st + hi), tile_row8<D>(Vs, wave * 32 + l32, 2 * st + hi), dp);
      }
      const int64_t rmin = a.causal ? a.kv_start + key - a.q_start - r0 : INT64_MIN / 2;
      const int64_t rmax = a.len_q - 1 - r0;
      const bool key_ok = key < a.len_kv;
      if (need_mask) {  // hidden scores -> -inf, so P = exp2(-inf) = 0 (c > 0)
#pragma unroll
        for (int r = 0; r < 16; ++r) {
          const int ri = 8 * (r >> 2) + 4 * hi + (r & 3);
          if (!key_ok || ri < rmin || ri > rmax) s[r] = -INFINITY;
        }
      }
#pragma unroll
      for (int r4 = 0; r4 < 4; ++r4) {
        const f32x4 x = *(const DFA_LDS f32x4*)(lse2s + 8 * r4 + 4 * hi);
        const f32x4 y = *(const DFA_LDS f32x4*)(dls + 8 * r4 + 4 * hi);
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          const int r = 4 * r4 + e;
          const float p = exp2_fast(fmaf(s[r], a.c, -x[e]));
          s[r] = p;
          dp[r] = p * (dp[r] - y[e]);
        }
      }
#pragma unroll 1
      for (int j = 0; j < 2; ++j) {
        bf16x8 pb, sb;
#pragma unroll
        for (int e = 0; e < 8; ++e) {
          pb[e] = static_cast<__bf16>(s[8 * j + e]);
          sb[e] = static_cast<__bf16>(dp[8 * j + e]);
        }
        const int t0 = 16 * j + 4 * hi;
#pragma unroll
        for (int db = 0; db < D / 32; ++db) {
          const int c0 = 32 * db + 16 * half16;
          const bf16x8 ta =
              cat4(tile_tr4<D>(dOs, t0, c0, lane), tile_tr4<D>(dOs, t0 + 8, c0, lane));
          dv_acc[db] = mfma32(ta, pb, dv_acc[db]);
          const bf16x8 ua = cat4(tile_tr4<D>(Qs, t0, c0, lane), tile_tr4<D>(Qs, t0 + 8, c0, lane));
          dk_acc[db] = mfma32(ua, sb, dk_acc[db]);
        }
      }
    }
    __syncthreads();
    if (it + 1 < steps) sstore();
    __syncthreads();
  }

  if (!wave_active || key >= a.len_kv) return;
  float* dkr = a.dk + (b * a.len_kv + key) * kv_rs + int64_t(g) * D;
  float* dvr = a.dv + (b * a.len_kv + key) * kv_rs + int64_t(g) * D;
#pragma unroll
  for (int db = 0; db < D / 32; ++db)
#pragma unroll
    for (int r4 = 0; r4 < 4; ++r4) {
      const int d = 32 * db + 8 * r4 + 4 * hi;
      f32x4 xk = *reinterpret_cast<f32x4*>(dkr + d);
      f32x4 xv = *reinterpret_cast<f32x4*>(dvr + d);
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        xk[e] += a.scale * dk_acc[db][4 * r4 + e];
        xv[e] += dv_acc[db][4 * r4 + e];
      }
      *reinterpret_cast<f32x4*>(dkr + d) = xk;
      *reinterpret_cast<f32x4*>(dvr + d) = xv;
    }
}

// ---------------------------------------------------------------- dQ
template <int D, int NW, int HPW, int BN>
struct DqCfg {
  static constexpr int NT = NW * 64;
  static constexpr int BM = 32 * (NW / HPW);
  static constexpr int CH = BN * D / 8;
  static constexpr int CPT = CH / NT;
  static constexpr int STAGE = 2 * BN * D;  // K tile + V tile (elements)
  static constexpr int LDS_BYTES = 2 * STAGE * 2;
  static_assert(CH % NT == 0, "key tile chunks must divide evenly");
};

#ifndef DFA_DQ_OCC
#define DFA_DQ_OCC 2  // waves per SIMD the register budget is sized for
#endif

template <int D, int NW, int HPW, int BN>
__global__ __launch_bounds__(NW * 64) __attribute__((amdgpu_waves_per_eu(DFA_DQ_OCC, DFA_DQ_OCC)))
void dq_bf16_kernel(BwdArgs a) {
  using C = DqCfg<D, NW, HPW, BN>;
  extern __shared__ __align__(16) uint16_t smem_generic[];
  lds_u16* smem = lds_base(smem_generic);

  const int tid = threadIdx.x;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);  // wave-uniform (scalar)
  const int lane = tid & 63;
  const int l32 = lane & 31, hi = lane >> 5;
  const int half16 = (lane >> 4) & 1;
  const int bid = blockIdx.x;
  const int qt = a.n_tiles - 1 - bid / a.n_hgroups;
  const int hg = bid % a.n_hgroups;
  const int64_t b = blockIdx.y;
  const int h = hg * HPW + wave % HPW;
  const int g = (hg * HPW) / a.group;
  const int64_t q_lo = int64_t(qt) * C::BM;
  const int64_t w_lo = q_lo + (wave / HPW) * 32;
  const int64_t q_hi = min(q_lo + C::BM, a.len_q);
  const int64_t w_hi = min(w_lo + 32, a.len_q);
  const bool wave_active = w_lo < a.len_q;
  const int64_t row = w_lo + l32;

  const int64_t q_rs = int64_t(a.hq) * D;
  const int64_t kv_rs = int64_t(a.hkv) * D;
  const uint16_t* kbase = a.k + b * a.len_kv * kv_rs + int64_t(g) * D;
  const uint16_t* vbase = a.v + b * a.len_kv * kv_rs + int64_t(g) * D;

  bf16x8 qf[D / 16], df[D / 16];
  float lse2 = INFINITY, dl = 0.f;
  {
    const int64_t off = (b * a.len_q + row) * q_rs + int64_t(h) * D;
#pragma unroll
    for (int st = 0; st < D / 16; ++st) {
      if (row < a.len_q) {
        qf[st] = ld_bf16x8(a.q + off + 16 * st + 8 * hi);
        df[st] = ld_bf16x8(a.d_o + off + 16 * st + 8 * hi);
      } else {
        qf[st] = bf16x8{};
        df[st] = bf16x8{};
      }
    }
    if (row < a.len_q) {
      const int64_t li = (b * a.hq + h) * a.len_q + row;
      lse2 = lse2_of(a.lse[li]);
      dl = a.delta[li];
    }
  }

  int kt_end = a.n_ktiles;
  if (a.causal) {
    const int64_t lim = a.q_start + (q_hi - 1) - a.kv_start;
    kt_end = lim < 0 ? 0 : int(min<int64_t>(a.n_ktiles, lim / BN + 1));
  }
  if (kt_end == 0) return;  // uniform: no key visible to any row here

  f32x16 acc[D / 32];
#pragma unroll
  for (int db = 0; db < D / 32; ++db) acc[db] = f32x16{};

  uint4 kreg[C::CPT], vreg[C::CPT];
  auto gload = [&](int kt) {
#pragma unroll
    for (int i = 0; i < C::CPT; ++i) {
      const int c = tid + i * C::NT;
      const int key = c / (D / 8), dc = c % (D / 8);
      const int64_t kk = int64_t(kt) * BN + key;
      if (kk < a.len_kv) {
        kreg[i] = ld_u4(kbase + kk * kv_rs + 8 * dc);
        vreg[i] = ld_u4(vbase + kk * kv_rs + 8 * dc);
      } else {
        kreg[i] = make_uint4(0, 0, 0, 0);
        vreg[i] = make_uint4(0, 0, 0, 0);
      }
    }
  };
  auto sstore = [&](int stage) {
    lds_u16* Ks = smem + stage * C::STAGE;
    lds_u16* Vs = Ks + BN * D;
#pragma unroll
    for (int i = 0; i < C::CPT; ++i) {
      const int c = tid + i * C::NT;
      const int key = c / (D / 8), dc = c % (D / 8);
      tile_store16<D>(Ks, key, dc, kreg[i]);
      tile_store16<D>(Vs, key, dc, vreg[i]);
    }
  };

  gload(0);
  sstore(0);
  __syncthreads();

  for (int kt = 0; kt < kt_end; ++kt) {
    if (kt + 1 < kt_end) gload(kt + 1);
    const lds_u16* Ks = smem + (kt & 1) * C::STAGE;
    const lds_u16* Vs = Ks + BN * D;
    const int64_t key0 = int64_t(kt) * BN;
    int nsb = 0;
    if (wave_active) {
      int64_t vis_last = a.len_kv - 1 - key0;
      if (a.causal) vis_last = min(vis_last, a.q_start + (w_hi - 1) - a.kv_start - key0);
      nsb = vis_last < 0 ? 0 : int(min<int64_t>(BN / 32, vis_last / 32 + 1));
    }
    if (nsb > 0) {
      const bool need_mask =
          (a.causal && a.kv_start + key0 + nsb * 32 - 1 > a.q_start + w_lo) ||
          (key0 + nsb * 32 > a.len_kv);
      int64_t vlim = a.len_kv - 1 - key0;
      if (a.causal) vlim = min(vlim, a.q_start + row - a.kv_start - key0);
#pragma unroll 1
      for (int kb = 0; kb < nsb; ++kb) {
        {
          f32x16 s = f32x16{}, dp = f32x16{};
#pragma unroll
          for (int st = 0; st < D / 16; ++st) {
            s = mfma32(tile_row8<D>(Ks, kb * 32 + l32, 2 * st + hi), qf[st], s);
            dp = mfma32(tile_row8<D>(Vs, kb * 32 + l32, 2 * st + hi), df[st], dp);
          }
          if (need_mask) {  // hidden scores -> -inf, so P = exp2(-inf) = 0 (c > 0)
#pragma unroll
            for (int r = 0; r < 16; ++r) {
              const int off = kb * 32 + 8 * (r >> 2) + 4 * hi + (r & 3);
              if (off > vlim) s[r] = -INFINITY;
            }
          }
#pragma unroll
          for (int r = 0; r < 16; ++r) {
            const float p = exp2_fast(fmaf(s[r], a.c, -lse2));
            dp[r] = p * (dp[r] - dl);
          }
#pragma unroll
          for (int j = 0; j < 2; ++j) {
            bf16x8 sb;
#pragma unroll
            for (int e = 0; e < 8; ++e) sb[e] = static_cast<__bf16>(dp[8 * j + e]);
            const int t0 = kb * 32 + 16 * j + 4 * hi;
#pragma unroll
            for (int db = 0; db < D / 32; ++db) {
              const int c0 = 32 * db + 16 * half16;
              const bf16x8 ta =
                  cat4(tile_tr4<D>(Ks, t0, c0, lane), tile_tr4<D>(Ks, t0 + 8, c0, lane));
              acc[db] = mfma32(ta, sb, acc[db]);
            }
          }
        }
      }
    }
    if (kt + 1 < kt_end) sstore((kt + 1) & 1);
    __syncthreads();
  }

  if (!wave_active || row >= a.len_q) return;
  float* out = a.dq + (b * a.len_q + row) * q_rs + int64_t(h) * D;
#pragma unroll
  for (int db = 0; db < D / 32; ++db)
#pragma unroll
    for (int r4 = 0; r4 < 4; ++r4) {
      const int d = 32 * db + 8 * r4 + 4 * hi;
      f32x4 x = *reinterpret_cast<f32x4*>(out + d);
#pragma unroll
      for (int e = 0; e < 4; ++e) x[e] += a.scale * acc[db][4 * r4 + e];
      *reinterpret_cast<f32x4*>(out + d) = x;
    }
}

struct Plan {
  int nw, hpw;
};
Plan dq_plan(int group) {
  if (group % 4 == 0) return {4, 4};
  if (group % 2 == 0) return {4, 2};
  return {4, 1};
}
constexpr int kDqBN = 64;
constexpr int kDkvNW = 4;
constexpr int kDkvBQ = 64;


template <int D, int NW, int HPW>
dfa_status launch_dq(const dfa_attn_desc& d, BwdArgs a, hipStream_t s) {
  using C = DqCfg<D, NW, HPW, kDqBN>;
  a.n_tiles = int(cdiv(d.len_q, C::BM));
  a.n_hgroups = d.heads_q / HPW;
  a.n_ktiles = int(cdiv(d.len_kv, kDqBN));
  auto kern = dq_bf16_kernel<D, NW, HPW, kDqBN>;
  const dfa_status st = allow_lds(kern, C::LDS_BYTES, "dq_bf16_kernel");
  if (st != DFA_OK) return st;
  dim3 grid(unsigned(a.n_tiles) * unsigned(a.n_hgroups), unsigned(d.batch));
  hipLaunchKernelGGL(kern, grid, dim3(C::NT), C::LDS_BYTES, s, a);
  return check_launch("dq_bf16_kernel");
}

#ifndef DFA_DKDV_KV_LDS
#define DFA_DKDV_KV_LDS 1  // K, V in LDS, two waves per SIMD
#endif

template <int D>
dfa_status launch_bwd_d(const dfa_attn_desc& d, BwdArgs a, hipStream_t s, int parts) {
  using KC = DkvCfg<D, kDkvNW, kDkvBQ>;
  if (!(parts & 1)) {
    // dQ only
  } else if constexpr (DFA_DKDV_KV_LDS && D == 128) {
    using LC = DkvLdsCfg<D, 8>;
    auto kern = dkdv_lds_bf16_kernel<D, 8>;
    const dfa_status st = allow_lds(kern, LC::LDS_BYTES, "dkdv_lds_bf16_kernel");
    if (st != DFA_OK) return st;
    dim3 grid(unsigned(cdiv(d.len_kv, LC::BK)) * unsigned(d.heads_kv), unsigned(d.batch));
    hipLaunchKernelGGL(kern, grid, dim3(LC::NT), LC::LDS_BYTES, s, a);
    const dfa_status st2 = check_launch("dkdv_lds_bf16_kernel");
    if (st2 != DFA_OK) return st2;
  } else {
    auto kern = dkdv_bf16_kernel<D, kDkvNW, kDkvBQ>;
    const dfa_status st = allow_lds(kern, KC::LDS_BYTES, "dkdv_bf16_kernel");
    if (st != DFA_OK) return st;
    dim3 grid(unsigned(cdiv(d.len_kv, KC::BK)) * unsigned(d.heads_kv), unsigned(d.batch));
    hipLaunchKernelGGL(kern, grid, dim3(KC::NT), KC::LDS_BYTES, s, a);
    const dfa_status st2 = check_launch("dkdv_bf16_kernel");
    if (st2 != DFA_OK) return st2;
  }
  if (!(parts & 2)) return DFA_OK;
  const Plan p = dq_plan(a.group);
  if (p.hpw == 4) return launch_dq<D, 4, 4>(d, a, s);
  if (p.hpw == 2) return launch_dq<D, 4, 2>(d, a, s);
  return launch_dq<D, 4, 1>(d, a, s);
}

}  // namespace

dfa_status launch_bwd_f32(const dfa_attn_desc& d, const void* q, const void* k, const void* v,
                          const float* lse, const void* d_o, const float* delta, float* dq,
                          float* dk, float* dv, hipStream_t s, int parts);

dfa_status launch_bwd(const dfa_attn_desc& d, const void* q, const void* k, const void* v,
                      const float* lse, const void* d_o, const float* delta, float* dq,
                      float* dk, float* dv, hipStream_t s, int parts) {
  if (d.dtype == DFA_F32)
    return launch_bwd_f32(d, q, k, v, lse, d_o, delta, dq, dk, dv, s, parts);
  BwdArgs a{};
  a.q = static_cast<const uint16_t*>(q);
  a.k = static_cast<const uint16_t*>(k);
  a.v = static_cast<const uint16_t*>(v);
  a.d_o = static_cast<const uint16_t*>(d_o);
  a.lse = lse;
  a.delta = delta;
  a.dq = dq;
  a.dk = dk;
  a.dv = dv;
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
  if (d.head_dim == 128) return launch_bwd_d<128>(d, a, s, parts);
  return launch_bwd_d<64>(d, a, s, parts);
}

}  // namespace dfa
