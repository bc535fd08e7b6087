// Forward partial attention of one chunk pair on gfx950 bf16 MFMA.
//
// Per chunk pair the kernel returns the normalised output and its natural
// log-sum-exp (the per-pair state of [DistFlashAttn App. D]), computing
// only the causal prefix (§2, §3.2).  Inside
// the kernel the softmax is the online (running max / running sum) form the
// paper builds on (FlashAttention, cited prior art), in base 2 with
// log2(e) folded into the scale.
//
// Work decomposition
//   workgroup = NW waves; wave w owns 32 query rows of query head
//   hg*HPW + w%HPW (HPW heads of one grouped-query group share each K/V
//   tile); the workgroup's query tile is BM = 32 * NW/HPW rows.
//   Grid x enumerates (query tile, head group) with the heaviest query
//   tiles first (the latest, or with a window whose edge leaves the key
//   chunk behind, the earliest) and head groups fastest, so that with >= 8
//   head groups the workgroups of one key/value head stay on one XCD's L2.
// Per key tile of BN keys, staged straight from HBM into LDS
// (global_load_lds, row-major, swizzled, double-buffered):
//   S^T = K Q^T        (A = K rows from LDS, B = Q fragments in VGPRs),
//   so each lane owns one query row and the row max / sum need only its
//   16 accumulator registers plus the lane 32 apart;
//   O^T += V^T P^T     (A = V^T rows from LDS, B = P^T straight from the S^T
//   accumulators).  Before the kernel, V is transposed once per call into
//   the caller's workspace, V^T [B][Hkv][d][keys], with the keys of every 16-key
//   group stored in the order the accumulator layout hands P^T over (bits 2
//   and 3 of the key index swapped), so each lane's A fragment is 8
//   consecutive elements of a V^T row: a 16-byte read instead of two
//   transposing 8-byte reads (which move half the bytes per LDS cycle).
// Chunk pairs in which every query sees every key (the off-diagonal pairs)
// run a mask-free instantiation whose sub-block loop is software-pipelined:
// the S^T of the next 32 keys is issued next to the softmax of the current
// ones, so matrix and vector instructions can interleave.
#include <algorithm>
#include <cfloat>

#include "kernels.hpp"

namespace dfa {
namespace {

struct FwdArgs {
  const uint16_t* q;
  const uint16_t* k;
  const uint16_t* vt;  // V^T [B][Hkv][d][vt_ld], keys permuted within 16-key groups
  int64_t vt_ld;       // keys per V^T row: len_kv rounded up to a whole key tile
  float* o;
  float* lse;
  uint8_t* visits;
  int64_t len_q, len_kv, q_start, kv_start;
  int32_t hq, hkv, group, causal;
  int32_t n_qtiles, n_ktiles, n_hgroups;
  float c;  // scale * log2(e), > 0
  int64_t win;  // sliding window in tokens; a huge value when there is none
  int32_t rows_up;  // row tiles first to last (the first rows see the most keys)
};

template <int D, int NW, int HPW, int BN>
struct FwdCfg {
  static constexpr int NT = NW * 64;
  static constexpr int BM = 32 * (NW / HPW);   // query rows per workgroup
  static constexpr int NSB = BN / 32;          // 32-key sub-blocks per tile
  static constexpr int TILE = BN * D;          // elements of the K (or V) tile
  static constexpr int SEGS = TILE / 512;      // 1 KiB segments per tile
  static constexpr int STAGE = 2 * TILE;       // elements per LDS stage (K + V)
  static constexpr int LDS_BYTES = 2 * STAGE * 2;
  static_assert(SEGS % NW == 0, "tile segments must divide over the waves");
  static_assert(NW % HPW == 0, "heads per workgroup must divide waves");
};

#ifndef DFA_FWD_OCC
#define DFA_FWD_OCC 2  // waves per SIMD the register budget is sized for
#endif

// FULL: every query row sees every key of the pair and the key chunk is a
// whole number of tiles, so no score is ever masked and the tile loop runs
// software-pipelined; otherwise the general (masked) loop runs.
template <int D, int NW, int HPW, int BN, bool INSTR, bool FULL>
__global__ __launch_bounds__(NW * 64) __attribute__((amdgpu_waves_per_eu(DFA_FWD_OCC, DFA_FWD_OCC)))
void fwd_bf16_kernel(FwdArgs a) {
  using C = FwdCfg<D, NW, HPW, BN>;
  extern __shared__ __align__(16) uint16_t smem_generic[];
  lds_u16* smem = lds_base(smem_generic);

  const int tid = threadIdx.x;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);  // wave-uniform (scalar)
  const int lane = tid & 63;
  const int l32 = lane & 31, hi = lane >> 5;
  const int half16 = (lane >> 4) & 1;  // which 16 columns of a 32-wide block
  const int bid = blockIdx.x;
  const int qt = a.rows_up ? bid / a.n_hgroups : a.n_qtiles - 1 - bid / a.n_hgroups;
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
  const uint16_t* kbase = a.k + b * a.len_kv * kv_rs + int64_t(g) * D;
  const uint16_t* vtb = a.vt + (b * a.hkv + g) * D * a.vt_ld;  // this head's V^T rows
  const int64_t row = w_lo + l32;  // this lane's query row (local index)

  int kt_end = a.n_ktiles;
  if (a.causal) {
    const int64_t lim = a.q_start + (q_hi - 1) - a.kv_start;
    kt_end = lim < 0 ? 0 : int(min<int64_t>(a.n_ktiles, lim / BN + 1));
  }
  // First key tile inside the window of the tile's first row (App. F).
  int kt_begin = 0;
  {
    const int64_t lo = a.q_start + q_lo - a.win + 1 - a.kv_start;  // lowest visible key
    if (lo > 0) kt_begin = lo >= a.len_kv ? a.n_ktiles : int(lo / BN);
  }

  // Q of this lane's row as the B operand of S^T, in VGPRs for the whole
  // loop; not loaded by a workgroup whose rows see no key tile (it only
  // writes O = 0, LSE = -inf)
  bf16x8 qf[D / 16];
  if (FULL || kt_begin < kt_end) {
    const uint16_t* qp = a.q + (b * a.len_q + row) * q_rs + int64_t(h) * D;
#pragma unroll
    for (int st = 0; st < D / 16; ++st)
      qf[st] = row < a.len_q ? ld_bf16x8(qp + 16 * st + 8 * hi) : bf16x8{};
  }

  f32x16 oacc[D / 32];
#pragma unroll
  for (int db = 0; db < D / 32; ++db) oacc[db] = f32x16{};
  float m = -INFINITY, l = 0.f;

  // Each wave stages SEGS/NW 1 KiB segments of the K and of the V tile.
  auto stage_tile = [&](int kt, int stage) {
    lds_u16* Ks = smem + stage * C::STAGE;
    lds_u16* Vs = Ks + C::TILE;
    const int64_t key0 = int64_t(kt) * BN;
    // rows past the chunk re-read its last key (their scores are masked)
    const int last_row = FULL ? BN - 1 : int(min<int64_t>(a.len_kv - 1 - key0, BN - 1));
    const uint16_t* kt_base = kbase + key0 * kv_rs;
#pragma unroll
    for (int i = 0; i < C::SEGS / NW; ++i) {
      const int seg = wave * (C::SEGS / NW) + i;
      tile_dma_rows<D>(Ks, seg, lane, kt_base, uint32_t(kv_rs * 2), last_row);
      // V^T tile: D rows of BN keys (zero past the chunk's end)
      tile_dma_rows<BN>(Vs, seg, lane, vtb + key0, uint32_t(a.vt_ld * 2), D - 1);
    }
  };

  // S^T of one 32-key sub-block.
  auto qk = [&](const lds_u16* Ks, int kb) {
    f32x16 s = f32x16{};
#pragma unroll
    for (int st = 0; st < D / 16; ++st)
      s = mfma32(tile_row8<D>(Ks, kb * 32 + l32, 2 * st + hi), qf[st], s);
    if constexpr (D == 128) {
      // Each K read three products ahead of the product that takes it
      // (0x100: LDS reads, 0x008: MFMA); left to itself, at this register
      // budget, the scheduler issues each read just before its product.
      __builtin_amdgcn_sched_group_barrier(0x100, 3, 0);
#pragma unroll
      for (int k = 0; k < 5; ++k) {
        __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
        __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);
      }
      __builtin_amdgcn_sched_group_barrier(0x008, 3, 0);
    }
    return s;
  };
  // Online-softmax update with the sub-block's scores (hidden ones -inf);
  // leaves P in s.  The reference point m (log2 units) moves only when the
  // row max exceeds it by more than 8, so P <= 2^8 and rescaling the
  // accumulators is rare; O and the LSE do not depend on m.
  auto softmax = [&](f32x16& s) {
    float mx = s[0];
#pragma unroll
    for (int r = 1; r < 16; ++r) mx = fmaxf(mx, s[r]);
    mx = max_xor32(mx);
    const float m_new = (mx * a.c > m + 8.f) ? mx * a.c : m;
    const float m_use = (m_new == -INFINITY) ? 0.f : m_new;
    float lsum = 0.f;
#pragma unroll
    for (int r = 0; r < 16; ++r) {
      const float t = exp2_fast(fmaf(s[r], a.c, -m_use));
      s[r] = t;
      lsum += t;
    }
    if (m_new != m) {  // rescale only when the running max moved
      const float alpha = exp2_fast(m - m_use);
      l *= alpha;
#pragma unroll
      for (int db = 0; db < D / 32; ++db) oacc[db] *= alpha;
    }
    l += lsum;
    m = m_new;
  };
  // O^T += V^T P^T for one sub-block.
  // V^T fragments of one sub-block, read ahead of its softmax: lane (d, hi)
  // takes keys kb*32 + 16j + 4hi + {0..3, 8..11}, positions 8hi..8hi+7 of the
  // 16-key group in V^T's permuted order.
  using VFrags = bf16x8[2 * (D / 32)];
  auto load_v = [&](const lds_u16* Vs, int kb, VFrags& vf) {
#pragma unroll
    for (int j = 0; j < 2; ++j)
#pragma unroll
      for (int db = 0; db < D / 32; ++db)
        vf[j * (D / 32) + db] = tile_row8<BN>(Vs, 32 * db + l32, 4 * kb + 2 * j + hi);
  };
  auto pv = [&](const VFrags& vf, const f32x16& p) {
#pragma unroll
    for (int j = 0; j < 2; ++j) {
      bf16x8 pb;
#pragma unroll
      for (int e = 0; e < 8; ++e) pb[e] = static_cast<__bf16>(p[8 * j + e]);
#pragma unroll
      for (int db = 0; db < D / 32; ++db) oacc[db] = mfma32(vf[j * (D / 32) + db], pb, oacc[db]);
    }
  };

  if (kt_begin < kt_end) stage_tile(kt_begin, kt_begin & 1);
  wait_vmem();
  __syncthreads();

  for (int kt = kt_begin; kt < kt_end; ++kt) {
    if (kt + 1 < kt_end) stage_tile(kt + 1, (kt + 1) & 1);  // lands while this tile computes
    const lds_u16* Ks = smem + (kt & 1) * C::STAGE;
    const lds_u16* Vs = Ks + C::TILE;
    const int64_t key0 = int64_t(kt) * BN;
    if (INSTR && b == 0 && hg == 0 && tid == 0) {
      const int64_t last_k = a.kv_start + min(key0 + BN, a.len_kv) - 1;
      const bool straddle = a.causal && (last_k > a.q_start + q_lo ||
                                         a.q_start + q_hi - 1 - (a.kv_start + key0) >= a.win);
      a.visits[int64_t(qt) * a.n_ktiles + kt] = straddle ? 2 : 1;
    }
    // Every tile runs software-pipelined over its 32-key sub-blocks.  A tile
    // that every row of this wave sees whole (always, in a fully visible
    // pair) is mask-free; in any other tile each sub-block's hidden scores
    // become -inf, so exp2 of them is exactly 0 (c > 0) and a sub-block no
    // row sees adds nothing.  Tiles no row of the wave sees are skipped.
    bool run = wave_active, whole = FULL;
    if constexpr (!FULL) {
      whole = key0 + BN <= a.len_kv &&
              (!a.causal || a.kv_start + key0 + BN - 1 <= a.q_start + w_lo) &&
              a.q_start + (w_hi - 1) - (a.kv_start + key0) < a.win;
      // some key of the tile inside some row's window and causal limit
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
      f32x16 s_cur = qk(Ks, 0);
#pragma unroll  // unrolled: s_cur / s_nxt rename instead of being copied
      for (int kb = 0; kb < C::NSB - 1; ++kb) {
        f32x16 s_nxt = qk(Ks, kb + 1);  // independent of the softmax below
        VFrags vf;
        load_v(Vs, kb, vf);
        mask(s_cur, kb);
        softmax(s_cur);
        pv(vf, s_cur);
        s_cur = s_nxt;
      }
      VFrags vf;
      load_v(Vs, C::NSB - 1, vf);
      mask(s_cur, C::NSB - 1);
      softmax(s_cur);
      pv(vf, s_cur);
    }
    wait_vmem();  // the next tile's segments this wave staged have landed
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

// Waves / heads per workgroup for a head grouping.
struct FwdPlan {
  int nw, hpw;
};

#ifndef DFA_FWD_WIDE_GQA
#define DFA_FWD_WIDE_GQA 1  // 8 heads of one group per workgroup when the group allows
#endif

FwdPlan plan_for(int group) {
  if (DFA_FWD_WIDE_GQA && group % 8 == 0) return {8, 8};
  if (group % 4 == 0) return {8, 4};
  if (group % 2 == 0) return {8, 2};
  return {8, 1};
}

#ifndef DFA_FWD_BN
#define DFA_FWD_BN 128
#endif
constexpr int kBN = DFA_FWD_BN;

template <int D, int NW, int HPW>
dfa_status launch_cfg(const dfa_attn_desc& d, FwdArgs a, bool instr, hipStream_t s) {
  using C = FwdCfg<D, NW, HPW, kBN>;
  a.n_qtiles = int(cdiv(d.len_q, C::BM));
  a.n_ktiles = int(cdiv(d.len_kv, kBN));
  a.n_hgroups = d.heads_q / HPW;
  dim3 grid(unsigned(a.n_qtiles) * unsigned(a.n_hgroups), unsigned(d.batch));
  auto go = [&](auto kern) {
    const dfa_status st = allow_lds(kern, C::LDS_BYTES, "fwd_bf16_kernel");
    if (st != DFA_OK) return st;
    hipLaunchKernelGGL(kern, grid, dim3(C::NT), C::LDS_BYTES, s, a);
    return check_launch("fwd_bf16_kernel");
  };
  if (pair_is_full(d, kBN))
    return instr ? go(fwd_bf16_kernel<D, NW, HPW, kBN, true, true>)
                 : go(fwd_bf16_kernel<D, NW, HPW, kBN, false, true>);
  return instr ? go(fwd_bf16_kernel<D, NW, HPW, kBN, true, false>)
               : go(fwd_bf16_kernel<D, NW, HPW, kBN, false, false>);
}

template <int D>
dfa_status launch_d(const dfa_attn_desc& d, const FwdArgs& a, bool instr, hipStream_t s) {
  const FwdPlan p = plan_for(a.group);
  if (p.hpw == 8) return launch_cfg<D, 8, 8>(d, a, instr, s);
  if (p.hpw == 4) return launch_cfg<D, 8, 4>(d, a, instr, s);
  if (p.hpw == 2) return launch_cfg<D, 8, 2>(d, a, instr, s);
  return launch_cfg<D, 8, 1>(d, a, instr, s);
}

}  // namespace

dfa_status launch_fwd_f32(const dfa_attn_desc& d, const void* q, const void* k, const void* v,
                          float* o, float* lse, hipStream_t s);

// The transposed V: [B][Hkv][d][keys rounded up to a whole key tile] bf16.
int64_t fwd_workspace_bytes(const dfa_attn_desc& d) {
  if (d.dtype != DFA_BF16 || d.batch == 0 || d.len_q == 0 || d.len_kv == 0) return 0;
  return int64_t(d.batch) * d.heads_kv * d.head_dim * (cdiv(d.len_kv, kBN) * kBN) * 2;
}

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
  // c > 0 keeps exp2(fma(-inf, c, -m)) == 0 for hidden scores; a zero scale
  // runs as the smallest normal one, whose scores (|s| * 1.2e-38) still give
  // every visible key the weight exp2(0) = 1 in fp32.
  a.c = std::max(d.scale * kLog2e, FLT_MIN);
  a.win = d.window > 0 ? d.window : kNoWindow;
  a.rows_up = rows_heaviest_first(d);
  // V^T into the caller's workspace (stream-ordered before the forward kernel;
  // its size was checked against fwd_workspace_bytes before this call)
  a.vt_ld = cdiv(d.len_kv, kBN) * kBN;
  if (uint64_t(a.vt_ld) * 2 * uint64_t(d.head_dim) >= (uint64_t(1) << 32))
    return fail(DFA_ERR_UNSUPPORTED, "dfa_attn_fwd_partial: len_kv too large for 32-bit V^T offsets");
  if (a.vt_ld > 0) {
    uint16_t* vt = static_cast<uint16_t*>(d.workspace);
    const dfa_status st = launch_kv_transpose(static_cast<const uint16_t*>(v), vt, d.batch,
                                              d.len_kv, d.heads_kv, d.head_dim, a.vt_ld, s);
    if (st != DFA_OK) return st;
    a.vt = vt;
  }
  if (d.head_dim == 128) return launch_d<128>(d, a, visits != nullptr, s);
  return launch_d<64>(d, a, visits != nullptr, s);
}

}  // namespace dfa
