// dQ of one chunk pair on gfx950 bf16 MFMA (the query-outer half of the
// backward; see bwd_mfma.hip for the pair of kernels and their contract).
#include <algorithm>
#include <cfloat>

#include "bwd_common.hpp"

// K^T fragments of a sub-block's dQ product read before its exponentials
// (two fit the register budget: 253 of 256; measured 0.8 % faster than none,
// four 0.2 %).
#ifndef DFA_DQ_KT_AHEAD
#define DFA_DQ_KT_AHEAD 2
#endif

namespace dfa {
namespace {

// ---------------------------------------------------------------- dQ
template <int D, int NW, int HPW, int BN>
struct DqCfg {
  static constexpr int NT = NW * 64;
  static constexpr int BM = 32 * (NW / HPW);
  static constexpr int NSB = BN / 32;
  static constexpr int TILE = BN * D;
  static constexpr int SEGS = TILE / 512;
  static constexpr int STAGE = 2 * TILE;  // K tile + V tile (elements)
  static constexpr int LDS_BYTES = 2 * STAGE * 2;
  static_assert(SEGS % NW == 0, "key tile segments must divide over the waves");
};

template <int D, int NW, int HPW, int BN, bool FULL>
__global__ __launch_bounds__(NW * 64) __attribute__((amdgpu_waves_per_eu(DFA_BWD_OCC, DFA_BWD_OCC)))
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
  const int qt = a.rows_up ? bid / a.n_hgroups : a.n_tiles - 1 - bid / a.n_hgroups;
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
  auto load_rows = [&]() {
    const int64_t off = (b * a.len_q + row) * q_rs + int64_t(h) * D;
#pragma unroll
    for (int st = 0; st < D / 16; ++st) {
      qf[st] = row < a.len_q ? ld_bf16x8(a.q + off + 16 * st + 8 * hi) : bf16x8{};
      df[st] = row < a.len_q ? ld_bf16x8(a.d_o + off + 16 * st + 8 * hi) : bf16x8{};
    }
    if (row < a.len_q) {
      const int64_t li = (b * a.hq + h) * a.len_q + row;
      lse2 = lse2_of(a.lse[li]);
      dl = a.delta[li];
    }
  };
  // Every tile of a fully visible pair has keys for every row; elsewhere a
  // workgroup whose rows see no key (nothing to add to dq) leaves before
  // loading them.
  if constexpr (FULL) load_rows();

  int kt_end = a.n_ktiles;
  if (a.causal) {
    const int64_t lim = a.q_start + (q_hi - 1) - a.kv_start;
    kt_end = lim < 0 ? 0 : int(min<int64_t>(a.n_ktiles, lim / BN + 1));
  }
  int kt_begin = 0;  // first key tile inside the window of the tile's first row
  {
    const int64_t lo = a.q_start + q_lo - a.win + 1 - a.kv_start;
    if (lo > 0) kt_begin = lo >= a.len_kv ? a.n_ktiles : int(lo / BN);
  }
  if (kt_begin >= kt_end) return;  // uniform: no key visible to any row here
  if constexpr (!FULL) load_rows();

  f32x16 acc[D / 32];
#pragma unroll
  for (int db = 0; db < D / 32; ++db) acc[db] = f32x16{};

  auto stage_tile = [&](int kt, int stage) {
    lds_u16* Ks = smem + stage * C::STAGE;
    lds_u16* Vs = Ks + C::TILE;
    const int64_t key0 = int64_t(kt) * BN;
    // rows past the chunk re-read its last key (their scores are masked)
    const int last_row = FULL ? BN - 1 : int(min<int64_t>(a.len_kv - 1 - key0, BN - 1));
    const uint16_t* kt_base = kbase + key0 * kv_rs;
    const uint16_t* vt_base = vbase + key0 * kv_rs;
#pragma unroll
    for (int i = 0; i < C::SEGS / NW; ++i) {
      const int seg = wave * (C::SEGS / NW) + i;
      tile_dma_rows<D>(Ks, seg, lane, kt_base, uint32_t(kv_rs * 2), last_row);
      tile_dma_rows<D>(Vs, seg, lane, vt_base, uint32_t(kv_rs * 2), last_row);
    }
  };
  // S^T = K Q^T and dP^T = V dO^T of one 32-key sub-block (lane = query row).
  auto sdp = [&](const lds_u16* Ks, const lds_u16* Vs, int kb, f32x16& s, f32x16& dp) {
    s = f32x16{};
    dp = f32x16{};
#pragma unroll
    for (int st = 0; st < D / 16; ++st) {
      s = mfma32(tile_row8<D>(Ks, kb * 32 + l32, 2 * st + hi), qf[st], s);
      dp = mfma32(tile_row8<D>(Vs, kb * 32 + l32, 2 * st + hi), df[st], dp);
    }
    if constexpr (D == 128) {
      // Each operand's LDS read three products ahead of the product that
      // takes it (0x100: LDS reads, 0x008: MFMA); left to itself, at this
      // register budget, the scheduler issues each read just before its
      // product, which then waits out the LDS latency.
      __builtin_amdgcn_sched_group_barrier(0x100, 3, 0);
#pragma unroll
      for (int k = 0; k < 13; ++k) {
        __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
        __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);
      }
      __builtin_amdgcn_sched_group_barrier(0x008, 3, 0);
    }
  };
  // dS^T = P^T (dP^T - delta) (hidden scores already -inf), dQ^T += K^T dS^T.
  auto update = [&](const lds_u16* Ks, int kb, const f32x16& s, f32x16& dp) {
    auto kt_frag = [&](int j, int db) {
      const int t0 = kb * 32 + 16 * j + 4 * hi;
      const int c0 = 32 * db + 16 * half16;
      return cat4(tile_tr4<D>(Ks, t0, c0, lane), tile_tr4<D>(Ks, t0 + 8, c0, lane));
    };
    // the first K^T fragments are read ahead of the exponentials
    constexpr int AHEAD = DFA_DQ_KT_AHEAD;
    bf16x8 early[AHEAD > 0 ? AHEAD : 1];
#pragma unroll
    for (int i = 0; i < AHEAD; ++i) early[i] = kt_frag(0, i);
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
#pragma unroll
      for (int db = 0; db < D / 32; ++db) {
        const bf16x8 ta = (j == 0 && db < AHEAD) ? early[db] : kt_frag(j, db);
        acc[db] = mfma32(ta, sb, acc[db]);
      }
    }
  };

  stage_tile(kt_begin, kt_begin & 1);
  wait_vmem();
  __syncthreads();

  for (int kt = kt_begin; kt < kt_end; ++kt) {
    if (kt + 1 < kt_end) stage_tile(kt + 1, (kt + 1) & 1);  // lands while this tile computes
    const lds_u16* Ks = smem + (kt & 1) * C::STAGE;
    const lds_u16* Vs = Ks + C::TILE;
    const int64_t key0 = int64_t(kt) * BN;
    // Every tile runs software-pipelined over its 32-key sub-blocks, mask-free
    // when every row of this wave sees it whole (always, in a fully visible
    // pair); otherwise each sub-block's hidden scores become -inf, so P =
    // exp2(-inf) = 0 (c > 0).  Tiles no row of the wave sees are skipped.
    bool run = wave_active, whole = FULL;
    if constexpr (!FULL) {
      whole = key0 + BN <= a.len_kv &&
              (!a.causal || a.kv_start + key0 + BN - 1 <= a.q_start + w_lo) &&
              a.q_start + (w_hi - 1) - (a.kv_start + key0) < a.win;
      run = run && (!a.causal || a.kv_start + key0 <= a.q_start + w_hi - 1) &&
            a.q_start + w_lo - (a.kv_start + min(key0 + BN, a.len_kv) - 1) < a.win;
    }
    auto mask = [&](f32x16& s, int kb) {
      if (whole) return;
      const int64_t kfirst = key0 + kb * 32;
      int64_t vlim64 = a.len_kv - 1 - kfirst;
      if (a.causal) vlim64 = min(vlim64, a.q_start + row - a.kv_start - kfirst);
      const int vlim = clamp_off(vlim64);
      const int vmin = clamp_off(a.q_start + row - a.win + 1 - a.kv_start - kfirst);
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        const int off = 8 * (r >> 2) + 4 * hi + (r & 3);
        if (off > vlim || off < vmin) s[r] = -INFINITY;
      }
    };
    if (run) {
      f32x16 s, dp;
      sdp(Ks, Vs, 0, s, dp);
#pragma unroll 1
      for (int kb = 0; kb < C::NSB - 1; ++kb) {
        f32x16 s2, dp2;
        sdp(Ks, Vs, kb + 1, s2, dp2);  // independent of the vector work below
        mask(s, kb);
        update(Ks, kb, s, dp);
        s = s2;
        dp = dp2;
      }
      mask(s, C::NSB - 1);
      update(Ks, C::NSB - 1, s, dp);
    }
    wait_vmem();  // the next tile's segments this wave staged have landed
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

#ifndef DFA_DQ_BN
#define DFA_DQ_BN 64
#endif
constexpr int kDqBN = DFA_DQ_BN;

int dq_hpw(int group) {
  if (group % 8 == 0) return 8;
  if (group % 4 == 0) return 4;
  if (group % 2 == 0) return 2;
  return 1;
}

template <int D, int HPW>
dfa_status launch_dq(const dfa_attn_desc& d, BwdArgs a, hipStream_t s) {
  constexpr int NW = 8;
  using C = DqCfg<D, NW, HPW, kDqBN>;
  a.n_tiles = int(cdiv(d.len_q, C::BM));
  a.n_hgroups = d.heads_q / HPW;
  a.n_ktiles = int(cdiv(d.len_kv, kDqBN));
  a.rows_up = rows_heaviest_first(d);
  dim3 grid(unsigned(a.n_tiles) * unsigned(a.n_hgroups), unsigned(d.batch));
  auto go = [&](auto kern) {
    const dfa_status st = allow_lds(kern, C::LDS_BYTES, "dq_bf16_kernel");
    if (st != DFA_OK) return st;
    hipLaunchKernelGGL(kern, grid, dim3(C::NT), C::LDS_BYTES, s, a);
    return check_launch("dq_bf16_kernel");
  };
  if (pair_is_full(d, kDqBN)) return go(dq_bf16_kernel<D, NW, HPW, kDqBN, true>);
  return go(dq_bf16_kernel<D, NW, HPW, kDqBN, false>);
}

template <int D>
dfa_status launch_dq_d(const dfa_attn_desc& d, const BwdArgs& a, hipStream_t s) {
  switch (dq_hpw(a.group)) {
    case 8: return launch_dq<D, 8>(d, a, s);
    case 4: return launch_dq<D, 4>(d, a, s);
    case 2: return launch_dq<D, 2>(d, a, s);
    default: return launch_dq<D, 1>(d, a, s);
  }
}

}  // namespace

dfa_status launch_dq_bf16(const dfa_attn_desc& d, const BwdArgs& a, hipStream_t s) {
  if (d.head_dim == 128) return launch_dq_d<128>(d, a, s);
  return launch_dq_d<64>(d, a, s);
}

}  // namespace dfa
