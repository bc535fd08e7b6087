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
//   workgroup = NW waves; wave w owns 32 query rows of query head
//   hg*HPW + w%HPW (HPW heads of one grouped-query group share each K/V
//   tile); the workgroup's query tile is BM = 32 * NW/HPW rows.
//   Grid x enumerates (query tile, head group) with the heaviest (latest)
//   query tiles first and head groups fastest, so that with >= 8 head
//   groups the workgroups of one key/value head stay on one XCD's L2.
// Per key tile of BN keys (staged in LDS: K row-major, V transposed):
//   S^T = K Q^T        (A = K rows from LDS, B = Q fragments in VGPRs),
//   so each lane owns one query row and the row max / sum need only its
//   16 accumulator registers plus the lane 32 apart;
//   O^T += V^T P^T     (A = V^T from LDS, B = P^T straight from the S^T
//   accumulators: the contraction order of keys is permuted identically
//   on both operands, so no shuffle is needed).
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

template <int D, int NW, int HPW, int BN>
struct FwdCfg {
  static constexpr int NT = NW * 64;
  static constexpr int BM = 32 * (NW / HPW);
  static constexpr int KS = D + 8;   // K row stride in LDS (elements)
  static constexpr int VS = BN + 4;  // V^T row stride in LDS (elements)
  static constexpr int CH = BN * D / 8;  // 16-byte chunks per K (or V) tile
  static constexpr int CPT = CH / NT;
  static constexpr int LDS_BYTES = (BN * KS + D * VS) * 2;
  static_assert(CH % NT == 0, "tile chunks must divide evenly");
  static_assert(NW % HPW == 0, "heads per workgroup must divide waves");
};

template <int D, int NW, int HPW, int BN, bool INSTR>
__global__ __launch_bounds__(NW * 64) void fwd_bf16_kernel(FwdArgs a) {
  using C = FwdCfg<D, NW, HPW, BN>;
  extern __shared__ __align__(16) uint16_t smem[];
  uint16_t* Ks = smem;
  uint16_t* Vt = smem + BN * C::KS;

  const int tid = threadIdx.x;
  const int wave = tid >> 6, lane = tid & 63;
  const int l32 = lane & 31, hi = lane >> 5;
  const int bid = blockIdx.x;
  const int qt = a.n_qtiles - 1 - bid / a.n_hgroups;
  const int hg = bid % a.n_hgroups;
  const int64_t b = blockIdx.y;
  const int h = hg * HPW + wave % HPW;
  const int g = (hg * HPW) / a.group;
  const int64_t q_lo = int64_t(qt) * C::BM;
  const int64_t w_lo = q_lo + (wave / HPW) * 32;
  const int64_t q_hi = min(q_lo + C::BM, a.len_q);
  const int64_t w_hi = min(w_lo + 32, a.len_q);
  const bool wave_active = w_lo < a.len_q;

  const int64_t q_rs = int64_t(a.hq) * D;
  const int64_t kv_rs = int64_t(a.hkv) * D;
  const uint16_t* qbase = a.q + b * a.len_q * q_rs + int64_t(h) * D;
  const uint16_t* kbase = a.k + b * a.len_kv * kv_rs + int64_t(g) * D;
  const uint16_t* vbase = a.v + b * a.len_kv * kv_rs + int64_t(g) * D;
  const int64_t row = w_lo + l32;  // this lane's query row (local index)

  bf16x8 qf[D / 16];
#pragma unroll
  for (int st = 0; st < D / 16; ++st) {
    if (row < a.len_q) qf[st] = ld_bf16x8(qbase + row * q_rs + 16 * st + 8 * hi);
    else qf[st] = bf16x8{};
  }

  int kt_end = a.n_ktiles;
  if (a.causal) {
    const int64_t lim = a.q_start + (q_hi - 1) - a.kv_start;
    kt_end = lim < 0 ? 0 : int(min<int64_t>(a.n_ktiles, lim / BN + 1));
  }

  f32x16 oacc[D / 32];
#pragma unroll
  for (int db = 0; db < D / 32; ++db) oacc[db] = f32x16{};
  float m = -INFINITY, l = 0.f;

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
  auto sstore = [&]() {
#pragma unroll
    for (int i = 0; i < C::CPT; ++i) {
      const int c = tid + i * C::NT;
      const int key = c / (D / 8), dc = c % (D / 8);
      *reinterpret_cast<uint4*>(Ks + key * C::KS + 8 * dc) = kreg[i];
      const uint32_t w[4] = {vreg[i].x, vreg[i].y, vreg[i].z, vreg[i].w};
#pragma unroll
      for (int e = 0; e < 8; ++e)
        Vt[(8 * dc + e) * C::VS + key] = uint16_t(w[e >> 1] >> (16 * (e & 1)));
    }
  };

  if (kt_end > 0) {
    gload(0);
    sstore();
  }
  __syncthreads();

  for (int kt = 0; kt < kt_end; ++kt) {
    if (kt + 1 < kt_end) gload(kt + 1);
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
    if (nsb > 0) {
      const bool need_mask =
          (a.causal && a.kv_start + key0 + nsb * 32 - 1 > a.q_start + w_lo) ||
          (key0 + nsb * 32 > a.len_kv);
      f32x16 s[BN / 32];
#pragma unroll
      for (int kb = 0; kb < BN / 32; ++kb) {
        s[kb] = f32x16{};
        if (kb < nsb) {
#pragma unroll
          for (int st = 0; st < D / 16; ++st)
            s[kb] = mfma32(ld_bf16x8(Ks + (kb * 32 + l32) * C::KS + 16 * st + 8 * hi), qf[st],
                           s[kb]);
        }
      }
      if (need_mask) {
        // last visible key offset (inside this tile) for this lane's row
        int64_t vlim = a.len_kv - 1 - key0;
        if (a.causal) vlim = min(vlim, a.q_start + row - a.kv_start - key0);
#pragma unroll
        for (int kb = 0; kb < BN / 32; ++kb)
#pragma unroll
          for (int r = 0; r < 16; ++r) {
            const int off = kb * 32 + 8 * (r >> 2) + 4 * hi + (r & 3);
            if (off > vlim) s[kb][r] = -INFINITY;
          }
      }
      float mx = -INFINITY;
#pragma unroll
      for (int kb = 0; kb < BN / 32; ++kb)
        if (kb < nsb) {
#pragma unroll
          for (int r = 0; r < 16; ++r) mx = fmaxf(mx, s[kb][r]);
        }
      mx = fmaxf(mx, xor32(mx));
      const float m_new = (mx == -INFINITY) ? m : fmaxf(m, mx * a.c);
      const float m_use = (m_new == -INFINITY) ? 0.f : m_new;
      const float alpha = exp2_fast(m - m_use);
      float lsum = 0.f;
#pragma unroll
      for (int kb = 0; kb < BN / 32; ++kb)
        if (kb < nsb) {
#pragma unroll
          for (int r = 0; r < 16; ++r) {
            float t = exp2_fast(fmaf(s[kb][r], a.c, -m_use));
            if (need_mask && s[kb][r] == -INFINITY) t = 0.f;
            s[kb][r] = t;
            lsum += t;
          }
        }
      l = l * alpha + lsum;
      m = m_new;
#pragma unroll
      for (int db = 0; db < D / 32; ++db) oacc[db] *= alpha;
#pragma unroll
      for (int kb = 0; kb < BN / 32; ++kb)
        if (kb < nsb) {
#pragma unroll
          for (int j = 0; j < 2; ++j) {
            bf16x8 pb;
#pragma unroll
            for (int e = 0; e < 8; ++e) pb[e] = static_cast<__bf16>(s[kb][8 * j + e]);
#pragma unroll
            for (int db = 0; db < D / 32; ++db) {
              const uint16_t* vp = Vt + (32 * db + l32) * C::VS + kb * 32 + 16 * j + 4 * hi;
              const bf16x8 va = cat4(*reinterpret_cast<const bf16x4*>(vp),
                                     *reinterpret_cast<const bf16x4*>(vp + 8));
              oacc[db] = mfma32(va, pb, oacc[db]);
            }
          }
        }
    }
    __syncthreads();
    if (kt + 1 < kt_end) sstore();
    __syncthreads();
  }

  if (!wave_active || row >= a.len_q) return;
  const float l_tot = l + xor32(l);
  const float inv = l_tot > 0.f ? 1.f / l_tot : 0.f;
  float* orow = a.o + (b * a.len_q + row) * q_rs + int64_t(h) * D;
#pragma unroll
  for (int db = 0; db < D / 32; ++db)
#pragma unroll
    for (int r4 = 0; r4 < 4; ++r4) {
      const f32x4 val = {oacc[db][4 * r4] * inv, oacc[db][4 * r4 + 1] * inv,
                         oacc[db][4 * r4 + 2] * inv, oacc[db][4 * r4 + 3] * inv};
      *reinterpret_cast<f32x4*>(orow + 32 * db + 8 * r4 + 4 * hi) = val;
    }
  if (hi == 0)
    a.lse[(b * a.hq + h) * a.len_q + row] =
        l_tot > 0.f ? (m + __builtin_amdgcn_logf(l_tot)) * kLn2 : -INFINITY;
}

// One configuration of waves / heads per workgroup for a head grouping.
struct FwdPlan {
  int nw, hpw;
};

FwdPlan plan_for(int group) {
  if (group % 8 == 0) return {8, 8};
  if (group % 4 == 0) return {4, 4};
  if (group % 2 == 0) return {4, 2};
  return {4, 1};
}

constexpr int kBN = 64;

template <int D, int NW, int HPW>
dfa_status launch_cfg(const dfa_attn_desc& d, FwdArgs a, bool instr, hipStream_t s) {
  using C = FwdCfg<D, NW, HPW, kBN>;
  a.n_qtiles = int(cdiv(d.len_q, C::BM));
  a.n_ktiles = int(cdiv(d.len_kv, kBN));
  a.n_hgroups = d.heads_q / HPW;
  dim3 grid(unsigned(a.n_qtiles) * unsigned(a.n_hgroups), unsigned(d.batch));
  if (instr)
    hipLaunchKernelGGL((fwd_bf16_kernel<D, NW, HPW, kBN, true>), grid, dim3(C::NT),
                       C::LDS_BYTES, s, a);
  else
    hipLaunchKernelGGL((fwd_bf16_kernel<D, NW, HPW, kBN, false>), grid, dim3(C::NT),
                       C::LDS_BYTES, s, a);
  return check_launch("fwd_bf16_kernel");
}

template <int D>
dfa_status launch_d(const dfa_attn_desc& d, const FwdArgs& a, bool instr, hipStream_t s) {
  const FwdPlan p = plan_for(a.group);
  if (p.nw == 8) return launch_cfg<D, 8, 8>(d, a, instr, s);
  if (p.hpw == 4) return launch_cfg<D, 4, 4>(d, a, instr, s);
  if (p.hpw == 2) return launch_cfg<D, 4, 2>(d, a, instr, s);
  return launch_cfg<D, 4, 1>(d, a, instr, s);
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
  *bm = 32 * (p.nw / p.hpw);
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
