// Forward partial attention of one chunk pair on gfx950 bf16 MFMA.
//
// Per chunk pair the kernel returns the normalised output and its natural
// log-sum-exp ([DistFlashAttn App. D]: the forward returns output and
// logsumexp values), computing only the causal prefix (§2, §3.2).  Inside
// the kernel the softmax is the online (running max / running sum) form the
// paper builds on (FlashAttention, cited prior art), in base 2 with
// log2(e) folded into the scale.
//
// Work decomposition
//   workgroup = NW waves; wave w owns QB blocks of 32 query rows of query
//   head hg*HPW + w%HPW (HPW heads of one grouped-query group share each K/V
//   tile); the workgroup's query tile is BM = 32*QB * NW/HPW rows.
//   Grid x enumerates (query tile, head group) with the heaviest (latest)
//   query tiles first and head groups fastest, so that with >= 8 head
//   groups the workgroups of one key/value head stay on one XCD's L2.
// Per key tile of BN keys (row-major, swizzled, double-buffered in LDS):
//   S^T = K Q^T        (A = K rows from LDS, B = Q fragments in VGPRs),
//   so each lane owns one query row and the row max / sum need only its
//   16 accumulator registers plus the lane 32 apart;
//   O^T += V^T P^T     (A = V^T via transpose reads of the row-major V tile,
//   B = P^T straight from the S^T accumulators: the contraction order of the
//   keys is permuted identically on both operands, so no shuffle is needed).
//   Each K / V fragment read from LDS feeds QB matrix instructions.
#include "kernels.hpp"

namespace dfa {
namespace {

struct FwdArgs {
  const uint16_t* q;
  const uint16_t* k;
  const uint16_t* v;
  float* o;
  float* lse;
  uint8_t* visits;
  int64_t len_q, len_kv, q_start, kv_start;
  int32_t hq, hkv, group, causal;
  int32_t n_qtiles, n_ktiles, n_hgroups;
  float c;  // scale * log2(e)
};

template <int D, int NW, int HPW, int BN, int QB>
struct FwdCfg {
  static constexpr int NT = NW * 64;
  static constexpr int RPW = 32 * QB;            // query rows per wave
  static constexpr int BM = RPW * (NW / HPW);    // query rows per workgroup
  static constexpr int CH = BN * D / 8;          // 16-byte chunks per K (or V) tile
  static constexpr int CPT = CH / NT;
  static constexpr int STAGE = 2 * BN * D;       // elements per LDS stage (K + V)
  static constexpr int LDS_BYTES = 2 * STAGE * 2;
  static_assert(CH % NT == 0, "tile chunks must divide evenly");
  static_assert(NW % HPW == 0, "heads per workgroup must divide waves");
};

#ifndef DFA_FWD_OCC
#define DFA_FWD_OCC 2  // waves per SIMD the register budget is sized for
#endif

template <int D, int NW, int HPW, int BN, int QB, bool INSTR>
__global__ __launch_bounds__(NW * 64) __attribute__((amdgpu_waves_per_eu(DFA_FWD_OCC, DFA_FWD_OCC)))
void fwd_bf16_kernel(FwdArgs a) {
  using C = FwdCfg<D, NW, HPW, BN, QB>;
  extern __shared__ __align__(16) uint16_t smem_generic[];
  lds_u16* smem = lds_base(smem_generic);

  const int tid = threadIdx.x;
  const int wave = tid >> 6, lane = tid & 63;
  const int l32 = lane & 31, hi = lane >> 5;
  const int half16 = (lane >> 4) & 1;  // which 16 columns of a 32-wide block
  const int bid = blockIdx.x;
  const int qt = a.n_qtiles - 1 - bid / a.n_hgroups;
  const int hg = bid % a.n_hgroups;
  const int64_t b = blockIdx.y;
  const int h = hg * HPW + wave % HPW;
  const int g = (hg * HPW) / a.group;
  const int64_t q_lo = int64_t(qt) * C::BM;
  const int64_t w_lo = q_lo + (wave / HPW) * C::RPW;
  const int64_t q_hi = min(q_lo + C::BM, a.len_q);
  const int64_t w_hi = min(w_lo + C::RPW, a.len_q);
  const bool wave_active = w_lo < a.len_q;

  const int64_t q_rs = int64_t(a.hq) * D;
  const int64_t kv_rs = int64_t(a.hkv) * D;
  const uint16_t* qbase = a.q + b * a.len_q * q_rs + int64_t(h) * D;
  const uint16_t* kbase = a.k + b * a.len_kv * kv_rs + int64_t(g) * D;
  const uint16_t* vbase = a.v + b * a.len_kv * kv_rs + int64_t(g) * D;

  bf16x8 qf[QB][D / 16];
#pragma unroll
  for (int qb = 0; qb < QB; ++qb) {
    const int64_t row = w_lo + 32 * qb + l32;
#pragma unroll
    for (int st = 0; st < D / 16; ++st) {
      if (row < a.len_q) qf[qb][st] = ld_bf16x8(qbase + row * q_rs + 16 * st + 8 * hi);
      else qf[qb][st] = bf16x8{};
    }
  }

  int kt_end = a.n_ktiles;
  if (a.causal) {
    const int64_t lim = a.q_start + (q_hi - 1) - a.kv_start;
    kt_end = lim < 0 ? 0 : int(min<int64_t>(a.n_ktiles, lim / BN + 1));
  }

  f32x16 oacc[QB][D / 32];
  float m[QB], l[QB];
#pragma unroll
  for (int qb = 0; qb < QB; ++qb) {
    m[qb] = -INFINITY;
    l[qb] = 0.f;
#pragma unroll
    for (int db = 0; db < D / 32; ++db) oacc[qb][db] = f32x16{};
  }

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

  if (kt_end > 0) {
    gload(0);
    sstore(0);
  }
  __syncthreads();

  for (int kt = 0; kt < kt_end; ++kt) {
    if (kt + 1 < kt_end) gload(kt + 1);
    const lds_u16* Ks = smem + (kt & 1) * C::STAGE;
    const lds_u16* Vs = Ks + BN * D;
    const int64_t key0 = int64_t(kt) * BN;
    if (INSTR && b == 0 && hg == 0 && tid == 0) {
      const int64_t last_k = a.kv_start + min(key0 + BN, a.len_kv) - 1;
      const bool straddle = a.causal && last_k > a.q_start + q_lo;
      a.visits[int64_t(qt) * a.n_ktiles + kt] = straddle ? 2 : 1;
    }
    // Visible 32-key sub-blocks of this tile for this wave's rows.
    int nsb = 0;
    if (wave_active) {
      int64_t vis_last = a.len_kv - 1 - key0;  // last key offset inside the chunk
      if (a.causal) vis_last = min(vis_last, a.q_start + (w_hi - 1) - a.kv_start - key0);
      nsb = vis_last < 0 ? 0 : int(min<int64_t>(BN / 32, vis_last / 32 + 1));
    }
    // One 32-key sub-block at a time: S^T, online-softmax update, O^T += V^T P^T.
#pragma unroll 1
    for (int kb = 0; kb < nsb; ++kb) {
      f32x16 s[QB];
#pragma unroll
      for (int qb = 0; qb < QB; ++qb) s[qb] = f32x16{};
#pragma unroll
      for (int st = 0; st < D / 16; ++st) {
        const bf16x8 ka = tile_row8<D>(Ks, kb * 32 + l32, 2 * st + hi);
#pragma unroll
        for (int qb = 0; qb < QB; ++qb) s[qb] = mfma32(ka, qf[qb][st], s[qb]);
      }
      const int64_t kfirst = key0 + kb * 32;  // local index of the sub-block's first key
#pragma unroll
      for (int qb = 0; qb < QB; ++qb) {
        const int64_t rlo = w_lo + 32 * qb;  // first row of this 32-row block
        const bool need_mask = (a.causal && a.kv_start + kfirst + 31 > a.q_start + rlo) ||
                               (kfirst + 32 > a.len_kv);
        if (need_mask) {
          // last visible key offset (inside this sub-block) for this lane's row
          int64_t vlim = a.len_kv - 1 - kfirst;
          if (a.causal) vlim = min(vlim, a.q_start + rlo + l32 - a.kv_start - kfirst);
#pragma unroll
          for (int r = 0; r < 16; ++r) {
            const int off = 8 * (r >> 2) + 4 * hi + (r & 3);
            if (off > vlim) s[qb][r] = -INFINITY;
          }
        }
        float mx = s[qb][0];
#pragma unroll
        for (int r = 1; r < 16; ++r) mx = fmaxf(mx, s[qb][r]);
        mx = fmaxf(mx, xor32(mx));
        const float m_new = (mx == -INFINITY) ? m[qb] : fmaxf(m[qb], mx * a.c);
        const float m_use = (m_new == -INFINITY) ? 0.f : m_new;
        float lsum = 0.f;
#pragma unroll
        for (int r = 0; r < 16; ++r) {
          float t = exp2_fast(fmaf(s[qb][r], a.c, -m_use));
          if (need_mask && s[qb][r] == -INFINITY) t = 0.f;
          s[qb][r] = t;
          lsum += t;
        }
        if (m_new != m[qb]) {  // rescale only when the running max moved
          const float alpha = exp2_fast(m[qb] - m_use);
          l[qb] *= alpha;
#pragma unroll
          for (int db = 0; db < D / 32; ++db) oacc[qb][db] *= alpha;
        }
        l[qb] += lsum;
        m[qb] = m_new;
      }
#pragma unroll
      for (int j = 0; j < 2; ++j) {
        bf16x8 pb[QB];
#pragma unroll
        for (int qb = 0; qb < QB; ++qb)
#pragma unroll
          for (int e = 0; e < 8; ++e) pb[qb][e] = static_cast<__bf16>(s[qb][8 * j + e]);
        const int r0 = kb * 32 + 16 * j + 4 * hi;
#pragma unroll
        for (int db = 0; db < D / 32; ++db) {
          const int c0 = 32 * db + 16 * half16;
          const bf16x8 va = cat4(tile_tr4<D>(Vs, r0, c0, lane), tile_tr4<D>(Vs, r0 + 8, c0, lane));
#pragma unroll
          for (int qb = 0; qb < QB; ++qb) oacc[qb][db] = mfma32(va, pb[qb], oacc[qb][db]);
        }
      }
    }
    if (kt + 1 < kt_end) sstore((kt + 1) & 1);
    __syncthreads();
  }

  if (!wave_active) return;
#pragma unroll
  for (int qb = 0; qb < QB; ++qb) {
    const int64_t row = w_lo + 32 * qb + l32;
    const float l_tot = l[qb] + xor32(l[qb]);
    if (row >= a.len_q) continue;
    const float inv = l_tot > 0.f ? 1.f / l_tot : 0.f;
    float* orow = a.o + (b * a.len_q + row) * q_rs + int64_t(h) * D;
#pragma unroll
    for (int db = 0; db < D / 32; ++db)
#pragma unroll
      for (int r4 = 0; r4 < 4; ++r4) {
        const f32x4 val = {oacc[qb][db][4 * r4] * inv, oacc[qb][db][4 * r4 + 1] * inv,
                           oacc[qb][db][4 * r4 + 2] * inv, oacc[qb][db][4 * r4 + 3] * inv};
        *reinterpret_cast<f32x4*>(orow + 32 * db + 8 * r4 + 4 * hi) = val;
      }
    if (hi == 0)
      a.lse[(b * a.hq + h) * a.len_q + row] =
          l_tot > 0.f ? (m[qb] + __builtin_amdgcn_logf(l_tot)) * kLn2 : -INFINITY;
  }
}

// Waves / heads / query blocks per workgroup for a head grouping.
struct FwdPlan {
  int nw, hpw, qb;
};

#ifndef DFA_FWD_QB
#define DFA_FWD_QB 1
#endif
#ifndef DFA_FWD_WIDE_GQA
#define DFA_FWD_WIDE_GQA 1  // 8 waves x 8 heads per workgroup when the group allows
#endif

FwdPlan plan_for(int group) {
  if (DFA_FWD_QB == 2) {
    if (group % 4 == 0) return {4, 4, 2};
    if (group % 2 == 0) return {4, 2, 2};
    return {4, 1, 2};
  }
  if (DFA_FWD_WIDE_GQA && group % 8 == 0) return {8, 8, 1};
  if (group % 4 == 0) return {4, 4, 1};
  if (group % 2 == 0) return {4, 2, 1};
  return {4, 1, 1};
}

constexpr int kBN = 64;

template <int D, int NW, int HPW, int QB>
dfa_status launch_cfg(const dfa_attn_desc& d, FwdArgs a, bool instr, hipStream_t s) {
  using C = FwdCfg<D, NW, HPW, kBN, QB>;
  a.n_qtiles = int(cdiv(d.len_q, C::BM));
  a.n_ktiles = int(cdiv(d.len_kv, kBN));
  a.n_hgroups = d.heads_q / HPW;
  dim3 grid(unsigned(a.n_qtiles) * unsigned(a.n_hgroups), unsigned(d.batch));
  if (instr)
    hipLaunchKernelGGL((fwd_bf16_kernel<D, NW, HPW, kBN, QB, true>), grid, dim3(C::NT),
                       C::LDS_BYTES, s, a);
  else
    hipLaunchKernelGGL((fwd_bf16_kernel<D, NW, HPW, kBN, QB, false>), grid, dim3(C::NT),
                       C::LDS_BYTES, s, a);
  return check_launch("fwd_bf16_kernel");
}

template <int D>
dfa_status launch_d(const dfa_attn_desc& d, const FwdArgs& a, bool instr, hipStream_t s) {
  const FwdPlan p = plan_for(a.group);
  if (p.qb == 2) {
    if (p.hpw == 4) return launch_cfg<D, 4, 4, 2>(d, a, instr, s);
    if (p.hpw == 2) return launch_cfg<D, 4, 2, 2>(d, a, instr, s);
    return launch_cfg<D, 4, 1, 2>(d, a, instr, s);
  }
  if (p.nw == 8) return launch_cfg<D, 8, 8, 1>(d, a, instr, s);
  if (p.hpw == 4) return launch_cfg<D, 4, 4, 1>(d, a, instr, s);
  if (p.hpw == 2) return launch_cfg<D, 4, 2, 1>(d, a, instr, s);
  return launch_cfg<D, 4, 1, 1>(d, a, instr, s);
}

}  // namespace

dfa_status launch_fwd_f32(const dfa_attn_desc& d, const void* q, const void* k, const void* v,
                          float* o, float* lse, hipStream_t s);

void fwd_tile_shape(const dfa_attn_desc& d, int32_t* bm, int32_t* bn) {
  if (d.dtype == DFA_F32) {  // exact fp32 kernel: one row per wave, all keys
    *bm = 4;
    *bn = 1;
    return;
  }
  const FwdPlan p = plan_for(d.heads_q / d.heads_kv);
  *bm = 32 * p.qb * (p.nw / p.hpw);
  *bn = kBN;
}

dfa_status launch_fwd(const dfa_attn_desc& d, const void* q, const void* k, const void* v,
                      float* o, float* lse, uint8_t* visits, hipStream_t s) {
  if (d.dtype == DFA_F32) return launch_fwd_f32(d, q, k, v, o, lse, s);
  FwdArgs a{};
  a.q = static_cast<const uint16_t*>(q);
  a.k = static_cast<const uint16_t*>(k);
  a.v = static_cast<const uint16_t*>(v);
  a.o = o;
  a.lse = lse;
  a.visits = visits;
  a.len_q = d.len_q;
  a.len_kv = d.len_kv;
  a.q_start = d.q_start;
  a.kv_start = d.kv_start;
  a.hq = d.heads_q;
  a.hkv = d.heads_kv;
  a.group = d.heads_q / d.heads_kv;
  a.causal = d.causal;
  a.c = d.scale * kLog2e;
  if (d.head_dim == 128) return launch_d<128>(d, a, visits != nullptr, s);
  return launch_d<64>(d, a, visits != nullptr, s);
}

}  // namespace dfa
