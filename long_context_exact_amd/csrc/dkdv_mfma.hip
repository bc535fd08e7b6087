// dK / dV of one chunk pair on gfx950 bf16 MFMA (the key-outer half of the
// backward; see bwd_mfma.hip for the pair of kernels and their contract).
#include <algorithm>
#include <cfloat>
#include <climits>

#include "bwd_common.hpp"

namespace dfa {
namespace {

// ---------------------------------------------------------------- dK, dV
// Each wave keeps its 32 keys' K rows in VGPRs (the B operand of S for the
// whole run); the workgroup's V rows stay in LDS, Q and dO come in
// double-buffered 32-row stages, and wave 0 stages each step's row
// statistics (-log2 e * LSE and delta) into the same stage, so no wave
// holds them in registers between steps.
template <int D, int NW>
struct DkvCfg {
  static constexpr int NT = NW * 64;
  static constexpr int BK = 32 * NW;            // keys per workgroup
  static constexpr int BQ = 32;                 // query rows per step
  static constexpr int KV_TILE = BK * D;        // elements of the K (or V) tile
  static constexpr int KV_SEGS = KV_TILE / 512; // 1 KiB segments
  static constexpr int Q_TILE = BQ * D;         // elements of one Q (or dO) tile
  static constexpr int Q_SEGS = Q_TILE / 512;
  static constexpr int STATS = 2 * BQ;           // -log2 LSE and delta of a step's rows (floats)
  static constexpr int STAGE = 2 * Q_TILE + 2 * STATS;  // Q + dO + row statistics (16-bit units)
  static constexpr int LDS_BYTES = (KV_TILE + 2 * STAGE) * 2;
  // Paired row bands (see the kernel): two tiles' Q, dO and statistics per stage.
  static constexpr int LDS_BYTES_PAIR = (KV_TILE + 4 * STAGE) * 2;
  static constexpr int NPAIR = BK / BQ + 1;  // steps per head of a paired launch
  static_assert(KV_SEGS % NW == 0, "key tile segments must divide over the waves");
  static_assert((2 * Q_SEGS) % NW == 0, "Q and dO segments divide over the waves");
  static_assert(LDS_BYTES <= 160 * 1024 && LDS_BYTES_PAIR <= 160 * 1024, "fits gfx950 LDS");
};

// FULL: every row the launch runs sees every key of the block (no mask code).
// TM: tile-major step order (see tile_of below), for pairs without a window
// and, with ROT, for the mask-free band of a windowed diagonal pair.
// PAIR: the two masked row bands of a windowed diagonal pair in one launch.
// Of a key block's own row tiles (0 .. BK/BQ - 1 from its first row, where
// the causal edge crosses it) wave w sees only tiles t >= w, and of the
// tiles at the window's edge (a.pair_wt + t) only t <= w.  Step p of a head
// stages own tile p - 1 and edge tile p together, and each wave takes the
// one of the two it sees (own if p - 1 >= w, else edge): BK/BQ + 1 steps per
// head in which every wave works, against 2 * BK/BQ steps run as two bands
// in which half the waves idle on average.
template <int D, int NW, bool FULL, bool TM, bool PAIR = false, bool ROT = false>
__global__ __launch_bounds__(NW * 64) __attribute__((amdgpu_waves_per_eu(DFA_BWD_OCC, DFA_BWD_OCC)))
void dkdv_bf16_kernel(BwdArgs a) {
  using C = DkvCfg<D, NW>;
  static_assert(!PAIR || (!FULL && !TM), "paired bands run the masked, head-major kernel");
  static_assert(!ROT || TM, "the rotated order is a tile-major order");
  extern __shared__ __align__(16) uint16_t smem_generic[];
  lds_u16* smem = lds_base(smem_generic);
  lds_u16* Vs = smem;

  const int tid = threadIdx.x;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);  // wave-uniform (scalar)
  const int lane = tid & 63;
  const int l32 = lane & 31, hi = lane >> 5;
  const int half16 = (lane >> 4) & 1;
  // Workgroups in dispatch order (x, then z over the row slices) enumerate
  // (key block, row slice, key-value head) with heads fastest: workgroup i
  // runs on XCD i mod 8, so with 8 key-value heads each XCD serves one head's
  // K, V and rows.  The slices of a key block run side by side, and the key
  // blocks go first to last, or last to first when the later keys see more
  // rows (keys_down), so that the longest workgroups start first.
  const int wg = int(blockIdx.z * gridDim.x + blockIdx.x);
  const int g = wg % a.hkv;
  const int slice = wg / a.hkv % a.rsplit;
  const int rank = wg / (a.hkv * a.rsplit);
  const int kt = a.keys_down ? int(gridDim.x) / a.hkv - 1 - rank : rank;
  const int64_t b = blockIdx.y;
  const int64_t k_lo = int64_t(kt) * C::BK;
  const int64_t wk_lo = k_lo + wave * 32;
  const int64_t wk_hi = min(wk_lo + 32, a.len_kv);
  const bool wave_active = wk_lo < a.len_kv;
  const int64_t key = wk_lo + l32;

  const int64_t q_rs = int64_t(a.hq) * D;
  const int64_t kv_rs = int64_t(a.hkv) * D;

  // This workgroup's steps: its key block's query-row steps, or with a row
  // split the slice-th slice of them (uniform over the workgroup).
  const DkvSpan sp = dkdv_span(a, k_lo, C::BK, C::BQ);
  const int qt0 = sp.qt0, nq = sp.nq;
  const int n_steps = PAIR ? (sp.steps > 0 ? C::NPAIR * a.group : 0) : sp.steps;
  const int per = int(cdiv(n_steps, a.rsplit));
  const int it0 = slice * per;
  const int it1 = min(n_steps, it0 + per);
  if (it0 >= it1) return;  // the reduction skips slices without steps
  // Step it covers query tile tile_of(it) of head head_of(it).  Without a
  // window every key block's rows end at the chunk's end: tiles run from the
  // last one down with the group's heads innermost, so the workgroups running
  // side by side read the same Q / dO tile at the same time (until each
  // reaches its own first row) and share it in L2 (a diagonal pair's HBM
  // reads drop several-fold).  With a window the row ranges slide with the
  // key block, by BK/BQ tiles from one block to the next; in the mask-free
  // band every block's range is equally long, and ROT runs it tile-major in
  // rotated order, tile t at tile step t (mod nq), so that the blocks running
  // side by side again reach each tile they share at the same step.  The
  // masked windowed launches run heads outermost, tiles ascending, which keeps
  // neighbouring blocks a few steps apart in the same head's rows.
  // A step's position is it = major * M + minor: tile step and head (TM),
  // head and tile (head-major), head and paired step (PAIR).  It is divided
  // out once and then advanced step by step (scalar adds, no division).
  const int rot = ROT ? (nq - qt0 % nq) % nq : 0;  // qt0 + rot = 0 (mod nq)
  const int M = TM ? a.group : (PAIR ? C::NPAIR : nq);
  struct Pos {
    int major, minor;
  };
  auto advance = [&](Pos p) { return p.minor + 1 == M ? Pos{p.major + 1, 0} : Pos{p.major, p.minor + 1}; };
  auto tile_of = [&](Pos p) {
    if constexpr (ROT) {
      const int t = p.major + rot;
      return qt0 + (t >= nq ? t - nq : t);
    }
    return TM ? qt0 + nq - 1 - p.major : qt0 + p.minor;
  };
  auto head_of = [&](Pos p) { return g * a.group + (TM ? p.minor : p.major); };
  // PAIR: the own and the edge tile of a step (tile indices from the chunk's
  // first row) and whether each holds rows of this key block's span.
  auto pair_tiles = [&](Pos p, int& own_t, int& edge_t, bool& own_ok, bool& edge_ok) {
    const int pp = p.minor;
    own_t = qt0 + pp - 1;
    edge_t = qt0 + a.pair_wt + pp;
    own_ok = pp >= 1 && pp - 1 < nq;
    edge_ok = pp <= C::NPAIR - 2 && a.pair_wt + pp < nq;
  };

  // K of this lane's key as the B operand of S (elements d = 16*st + 8*hi
  // + e), in VGPRs for the whole loop; V rows of the workgroup in LDS.
  bf16x8 kf[D / 16];
  {
    const uint16_t* kp = a.k + (b * a.len_kv + key) * kv_rs + int64_t(g) * D;
#pragma unroll
    for (int st = 0; st < D / 16; ++st)
      kf[st] = key < a.len_kv ? ld_bf16x8(kp + 16 * st + 8 * hi) : bf16x8{};
    const uint16_t* vb = a.v + b * a.len_kv * kv_rs + int64_t(g) * D;
    // rows past the chunk re-read its last key (masked)
    const int last_row = int(min<int64_t>(a.len_kv - 1 - k_lo, C::BK - 1));
#pragma unroll
    for (int i = 0; i < C::KV_SEGS / NW; ++i) {
      const int seg = wave * (C::KV_SEGS / NW) + i;
      tile_dma_rows<D>(Vs, seg, lane, vb + k_lo * kv_rs, uint32_t(kv_rs * 2), last_row);
    }
  }

  f32x16 dk_acc[D / 32], dv_acc[D / 32];
#pragma unroll
  for (int db = 0; db < D / 32; ++db) {
    dk_acc[db] = f32x16{};
    dv_acc[db] = f32x16{};
  }

  auto stage_ptr = [&](int stage) {
    return smem + C::KV_TILE + stage * (PAIR ? 2 * C::STAGE : C::STAGE);
  };
  auto stage_q_pair = [&](Pos ps, int stage) {
    const int h = head_of(ps);
    int own_t, edge_t;
    bool own_ok, edge_ok;
    pair_tiles(ps, own_t, edge_t, own_ok, edge_ok);
    const uint16_t* qb = a.q + b * a.len_q * q_rs + int64_t(h) * D;
    const uint16_t* db_ = a.d_o + b * a.len_q * q_rs + int64_t(h) * D;
    int ln = lane;
    asm volatile("" : "+v"(ln));
    // 4 * Q_SEGS segments (own Q, own dO, edge Q, edge dO) spread over the
    // waves; a tile without rows of the span is not staged (no wave reads it)
#pragma unroll
    for (int i = 0; i < 4 * C::Q_SEGS / NW; ++i) {
      const int seg = wave + i * NW;
      const int half = seg / (2 * C::Q_SEGS);
      const int s2 = seg - half * 2 * C::Q_SEGS;
      if (!(half == 0 ? own_ok : edge_ok)) continue;
      const int64_t i0 = int64_t(half == 0 ? own_t : edge_t) * C::BQ;
      const int last_row = int(min<int64_t>(a.len_q - 1 - i0, C::BQ - 1));
      lds_u16* Qs = stage_ptr(stage) + half * C::STAGE;
      if (s2 < C::Q_SEGS)
        tile_dma_rows<D>(Qs, s2, ln, qb + i0 * q_rs, uint32_t(q_rs * 2), last_row);
      else
        tile_dma_rows<D>(Qs + C::Q_TILE, s2 - C::Q_SEGS, ln, db_ + i0 * q_rs, uint32_t(q_rs * 2),
                         last_row);
    }
  };
  auto stage_q = [&](Pos ps, int stage) {
    if constexpr (PAIR) {
      stage_q_pair(ps, stage);
      return;
    }
    const int h = head_of(ps);
    const int64_t i0 = int64_t(tile_of(ps)) * C::BQ;
    const uint16_t* qb = a.q + b * a.len_q * q_rs + int64_t(h) * D;
    const uint16_t* db_ = a.d_o + b * a.len_q * q_rs + int64_t(h) * D;
    lds_u16* Qs = stage_ptr(stage);
    lds_u16* dOs = Qs + C::Q_TILE;
    // rows past the chunk re-read its last row (their P is 0)
    const int last_row = FULL ? C::BQ - 1 : int(min<int64_t>(a.len_q - 1 - i0, C::BQ - 1));
    // The lane's staging offsets are recomputed every step (a few VALU ops)
    // rather than hoisted out of the loop, where they would hold registers.
    int ln = lane;
    asm volatile("" : "+v"(ln));
    // 2 * Q_SEGS segments (Q then dO) spread over the waves
    if constexpr (C::Q_SEGS == NW) {  // segment `wave` of each, without a branch on it
      tile_dma_rows<D>(Qs, wave, ln, qb + i0 * q_rs, uint32_t(q_rs * 2), last_row);
      tile_dma_rows<D>(dOs, wave, ln, db_ + i0 * q_rs, uint32_t(q_rs * 2), last_row);
      return;
    }
#pragma unroll
    for (int i = 0; i < 2 * C::Q_SEGS / NW; ++i) {
      const int seg = wave + i * NW;
      if (seg < C::Q_SEGS)
        tile_dma_rows<D>(Qs, seg, ln, qb + i0 * q_rs, uint32_t(q_rs * 2), last_row);
      else
        tile_dma_rows<D>(dOs, seg - C::Q_SEGS, ln, db_ + i0 * q_rs, uint32_t(q_rs * 2), last_row);
    }
  };

  // Row statistics of a step, staged by wave 0 into the step's LDS stage:
  // lane r < 32 holds -log2(e) * LSE of row r (-inf for rows without keys or
  // past the chunk, so that P = exp2(fma(s, c, nl)) = 0), lane 32 + r holds
  // delta of row r.  Every wave then reads its lanes' rows from LDS.  The
  // loads are issued with the next stage and consumed only after the wait
  // that ends the step: consuming them at once would hold wave 0, and with
  // it the step's barrier, behind that stage's transfer.
  static_assert(C::BQ <= 64, "one lane per row of a step");
  float raw_l = 0.f, raw_d = 0.f;
  bool raw_ok = false;
  auto load_stats = [&](Pos ps) {
    const int h = head_of(ps);
    if constexpr (PAIR) {  // lanes 0..31: the own tile's rows, 32..63: the edge tile's
      int own_t, edge_t;
      bool own_ok, edge_ok;
      pair_tiles(ps, own_t, edge_t, own_ok, edge_ok);
      const bool edge = lane >= C::BQ;
      const int64_t row = int64_t(edge ? edge_t : own_t) * C::BQ + (lane & (C::BQ - 1));
      raw_ok = (edge ? edge_ok : own_ok) && row >= 0 && row < a.len_q;
      const int64_t li = (b * a.hq + h) * a.len_q + min<int64_t>(max<int64_t>(row, 0), a.len_q - 1);
      raw_l = a.lse[li];
      raw_d = a.delta[li];
      return;
    }
    const int64_t row = int64_t(tile_of(ps)) * C::BQ + lane;
    raw_ok = lane < C::BQ && (FULL || row < a.len_q);
    const int64_t li = (b * a.hq + h) * a.len_q + min<int64_t>(row, a.len_q - 1);
    raw_l = a.lse[li];
    raw_d = a.delta[li];
  };
  auto store_stats = [&](int stage) {
    const float x = raw_ok ? raw_l : -INFINITY;
    // every row of a fully visible pair sees keys, so its LSE is finite
    const float nl = (FULL || x > -INFINITY) ? -x * kLog2e : -INFINITY;
    const float dl = raw_ok ? raw_d : 0.f;
    if constexpr (PAIR) {
      static_assert(2 * C::BQ == 64, "one lane per row of the two tiles");
      lds_f32* st = reinterpret_cast<lds_f32*>(stage_ptr(stage) + (lane >= C::BQ ? C::STAGE : 0) +
                                               2 * C::Q_TILE);
      st[lane & (C::BQ - 1)] = nl;
      st[C::BQ + (lane & (C::BQ - 1))] = dl;
      return;
    }
    lds_f32* st = reinterpret_cast<lds_f32*>(stage_ptr(stage) + 2 * C::Q_TILE);
    if (lane < C::BQ) {
      st[lane] = nl;
      st[C::BQ + lane] = dl;
    }
  };

  Pos cur{it0 / M, it0 % M};
  stage_q(cur, 0);
  if (wave == 0) load_stats(cur);
  wait_vmem();
  if (wave == 0) store_stats(0);
  __syncthreads();

#pragma unroll 1
  for (int it = it0; it < it1; ++it) {
    const int stage = (it - it0) & 1;
    const Pos nxt = advance(cur);
    if (it + 1 < it1) {  // lands while this step computes
      stage_q(nxt, stage ^ 1);
      if (wave == 0) load_stats(nxt);
    }
    const lds_u16* Qs = stage_ptr(stage);
    int64_t r0;  // first row of this step's tile (for this wave)
    bool any = wave_active;
    if constexpr (PAIR) {
      int own_t, edge_t;
      bool own_ok, edge_ok;
      pair_tiles(cur, own_t, edge_t, own_ok, edge_ok);
      const bool own = cur.minor - 1 >= wave;  // this wave's keys are seen by the own tile
      if (!own) Qs += C::STAGE;
      r0 = int64_t(own ? own_t : edge_t) * C::BQ;
      if (!(own ? own_ok : edge_ok)) any = false;
    } else {
      r0 = int64_t(tile_of(cur)) * C::BQ;
    }
    const lds_u16* dOs = Qs + C::Q_TILE;
    const lds_f32* stats = reinterpret_cast<const lds_f32*>(Qs + 2 * C::Q_TILE);
    if constexpr (!FULL) {
      if (any && a.causal) any = a.q_start + min<int64_t>(r0 + C::BQ, a.len_q) - 1 >= a.kv_start + wk_lo;
      if (any) any = a.q_start + r0 - (a.kv_start + wk_hi - 1) < a.win;
    }
    if (any) {
      // S first, then dP: the exponentials below can run while dP's
      // instructions are still in the matrix pipe.
      f32x16 s = f32x16{}, dp = f32x16{};
#pragma unroll
      for (int st = 0; st < D / 16; ++st)
        s = mfma32(tile_row8<D>(Qs, l32, 2 * st + hi), kf[st], s);
#pragma unroll
      for (int st = 0; st < D / 16; ++st)
        dp = mfma32(tile_row8<D>(dOs, l32, 2 * st + hi), tile_row8<D>(Vs, wave * 32 + l32, 2 * st + hi), dp);
      if constexpr (D == 128) {
        // Schedule of the 16 products above: each operand's LDS read is
        // issued three products ahead of the product that takes it (left to
        // itself, at this register budget, the scheduler issues each read
        // just before its product, and the product then waits out the LDS
        // latency).  Groups in order: 3 Q reads; S0..S4 each followed by
        // the next Q read; S5..S7 each followed by one dO and one V read;
        // dP0..dP4 likewise; dP5..dP7.
        __builtin_amdgcn_sched_group_barrier(0x100, 3, 0);  // 0x100: LDS reads
#pragma unroll
        for (int k = 0; k < 5; ++k) {
          __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);  // 0x008: MFMA
          __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);
        }
#pragma unroll
        for (int k = 0; k < 8; ++k) {
          __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
          __builtin_amdgcn_sched_group_barrier(0x100, 2, 0);
        }
        __builtin_amdgcn_sched_group_barrier(0x008, 3, 0);
      }
      bool need_mask = false;
      if constexpr (!FULL)
        need_mask = (a.causal && a.q_start + r0 < a.kv_start + wk_hi - 1) ||
                    (r0 + C::BQ > a.len_q) || (wk_lo + 32 > a.len_kv) ||
                    a.q_start + r0 + C::BQ - 1 - (a.kv_start + wk_lo) >= a.win;
      if (need_mask) {  // hidden scores -> -inf, so P = exp2(-inf) = 0 (c > 0)
        // wave-uniform bounds for the wave's first key, then this lane's key
        // offset l32: row ri of the step sees the key iff rmin <= ri <= rmax
        const int rmin0 = a.causal ? clamp_off(a.kv_start + wk_lo - a.q_start - r0) : -(1 << 30);
        const int rmax0 = clamp_off(a.kv_start + wk_lo + a.win - 1 - a.q_start - r0);
        const int rmin = rmin0 + l32;
        const int rmax = min(clamp_off(a.len_q - 1 - r0), rmax0 + l32);
        const bool key_ok = l32 < clamp_off(a.len_kv - wk_lo);
#pragma unroll
        for (int r = 0; r < 16; ++r) {
          const int ri = 8 * (r >> 2) + 4 * hi + (r & 3);
          if (!key_ok || ri < rmin || ri > rmax) s[r] = -INFINITY;
        }
      }
      // P, then dV^T += dO^T P; dS is formed while those instructions run.
      // This lane's rows are 8 * (r / 4) + 4 * hi + r % 4.
#pragma unroll
      for (int r4 = 0; r4 < 4; ++r4) {
        const f32x4 nl = *reinterpret_cast<const DFA_LDS f32x4*>(stats + 8 * r4 + 4 * hi);
#pragma unroll
        for (int e = 0; e < 4; ++e) s[4 * r4 + e] = exp2_fast(fmaf(s[4 * r4 + e], a.c, nl[e]));
      }
#pragma unroll
      for (int j = 0; j < 2; ++j) {
        bf16x8 pb;
#pragma unroll
        for (int e = 0; e < 8; ++e) pb[e] = static_cast<__bf16>(s[8 * j + e]);
        const int t0 = 16 * j + 4 * hi;
#pragma unroll
        for (int db = 0; db < D / 32; ++db) {
          const int c0 = 32 * db + 16 * half16;
          const bf16x8 ta = cat4(tile_tr4<D>(dOs, t0, c0, lane), tile_tr4<D>(dOs, t0 + 8, c0, lane));
          dv_acc[db] = mfma32(ta, pb, dv_acc[db]);
        }
      }
#pragma unroll
      for (int r4 = 0; r4 < 4; ++r4) {
        const f32x4 dl = *reinterpret_cast<const DFA_LDS f32x4*>(stats + C::BQ + 8 * r4 + 4 * hi);
#pragma unroll
        for (int e = 0; e < 4; ++e) dp[4 * r4 + e] = s[4 * r4 + e] * (dp[4 * r4 + e] - dl[e]);
      }
#pragma unroll
      for (int j = 0; j < 2; ++j) {
        bf16x8 sb;
#pragma unroll
        for (int e = 0; e < 8; ++e) sb[e] = static_cast<__bf16>(dp[8 * j + e]);
        const int t0 = 16 * j + 4 * hi;
#pragma unroll
        for (int db = 0; db < D / 32; ++db) {
          const int c0 = 32 * db + 16 * half16;
          const bf16x8 ua = cat4(tile_tr4<D>(Qs, t0, c0, lane), tile_tr4<D>(Qs, t0 + 8, c0, lane));
          dk_acc[db] = mfma32(ua, sb, dk_acc[db]);
        }
      }
    }
    // The next stage this wave staged (and, for wave 0, the next step's row
    // statistics) must land before the barrier.
    if (it + 1 < it1) {
      wait_vmem();
      if (wave == 0) store_stats(stage ^ 1);
    }
    __syncthreads();
    cur = nxt;
  }

  if (!wave_active || key >= a.len_kv) return;
  if (a.rsplit > 1) {  // store this slice's partial for the reduction
    const int64_t n = int64_t(a.rsplit) * gridDim.y * a.len_kv * kv_rs;
    float* wk = a.ws + ((int64_t(slice) * gridDim.y + b) * a.len_kv + key) * kv_rs +
                int64_t(g) * D;
    float* wv = wk + n;
#pragma unroll
    for (int db = 0; db < D / 32; ++db)
#pragma unroll
      for (int r4 = 0; r4 < 4; ++r4) {
        const int d = 32 * db + 8 * r4 + 4 * hi;
        f32x4 xk, xv;
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          xk[e] = a.scale * dk_acc[db][4 * r4 + e];
          xv[e] = dv_acc[db][4 * r4 + e];
        }
        *reinterpret_cast<f32x4*>(wk + d) = xk;
        *reinterpret_cast<f32x4*>(wv + d) = xv;
      }
    return;
  }
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

// dk, dv += the row-split slices' partials, summed in slice order (so the
// result does not depend on which slice finished first).  One thread per 4
// consecutive elements of [B][len_kv][Hkv][d]; slices a key block did not
// run (fewer steps than slices) are skipped exactly as the kernel skipped them.
template <int BK, int BQ>
__global__ __launch_bounds__(256) void dkdv_split_reduce_kernel(BwdArgs a, int64_t n4, int32_t row4) {
  const int64_t i = int64_t(blockIdx.x) * 256 + threadIdx.x;
  if (i >= n4) return;
  const int64_t key = (i / row4) % a.len_kv;
  const DkvSpan sp = dkdv_span(a, (key / BK) * BK, BK, BQ);
  if (sp.steps == 0) return;
  const int per = int(cdiv(sp.steps, a.rsplit));
  const int used = int(cdiv(sp.steps, per));
  const f32x4* wk = reinterpret_cast<const f32x4*>(a.ws);
  const f32x4* wv = wk + int64_t(a.rsplit) * n4;
  f32x4 sk = wk[i], sv = wv[i];
  for (int z = 1; z < used; ++z) {
    sk += wk[int64_t(z) * n4 + i];
    sv += wv[int64_t(z) * n4 + i];
  }
  f32x4* dk = reinterpret_cast<f32x4*>(a.dk);
  f32x4* dv = reinterpret_cast<f32x4*>(a.dv);
  dk[i] += sk;
  dv[i] += sv;
}

constexpr int kDkvNW = 8;
constexpr int kMaxSplit = 64;                                // slices per key block
constexpr int kMinSplitSteps = 32;                           // steps per slice, at least
constexpr int64_t kMaxSplitBytes = int64_t(4) << 30;         // workspace cap
// The split plan is sized for the MI355X's 256 compute units rather than
// queried from the device, so that it (and the workspace it needs) is a pure
// function of the descriptor, known on the host before any HIP call.
constexpr int64_t kSplitCUs = 256;

// Slices per key block of the row split (1: no split).  Split when the
// longest key block's steps exceed twice an even share of all steps over the
// compute units (few key blocks with many rows: a short key range such as
// global tokens, or the blocks a window band reaches).
template <int D>
int dkdv_row_split(const dfa_attn_desc& d) {
  using C = DkvCfg<D, kDkvNW>;
  const BwdArgs a = bwd_args_of(d);
  const int64_t nkb = cdiv(d.len_kv, C::BK);
  int64_t total = 0, longest = 0;
  for (int64_t kb = 0; kb < nkb; ++kb) {
    const int st = dkdv_span(a, kb * C::BK, C::BK, C::BQ).steps;
    total += st;
    longest = std::max<int64_t>(longest, st);
  }
  total *= int64_t(d.heads_kv) * d.batch;
  const int64_t share = std::max<int64_t>(1, cdiv(total, kSplitCUs));
  int64_t split = longest > 2 * share ? cdiv(longest, share) : 1;
  split = std::min<int64_t>({split, kMaxSplit, std::max<int64_t>(1, longest / kMinSplitSteps)});
  split = std::min<int64_t>(split, kMaxSplitBytes / dkdv_split_bytes_per_slice(d));
  return int(std::max<int64_t>(split, 1));
}

template <int D>
dfa_status rsplit_reduce(const dfa_attn_desc& d, const BwdArgs& a, hipStream_t s, dfa_status st);

// How the dK/dV kernel runs a descriptor: its row split, and whether (and
// where) it runs as row bands.  A diagonal pair (query and key chunk the
// same tokens) of whole key blocks runs as row bands, each a launch over
// every key block: the block's own BK/BQ row tiles (where the causal edge
// crosses it) in the masked kernel, the rows from there to W rows past its
// first key (every one of which sees all its keys) in the mask-free kernel,
// and, with a window shorter than the chunk, the rows from W on (where the
// window edge crosses it) in the masked kernel too, paired with the own
// rows in one launch (see the kernel's PAIR mode).  The masked kernel's mask
// branch splits every step's code, so it is kept to the steps that need it;
// the bands add into dk, dv one after the other, so the result stays
// deterministic.
struct DkvPlan {
  int rsplit;    // row slices per key block (1: none)
  bool banded;
  bool paired;   // the own and the window-edge rows in one paired launch
  int own, wt;   // band limits in row tiles: [0, own) masked, [own, wt) mask-free, [wt, ..) masked
  int launches;  // dK/dV kernel launches (the split reduction not counted)
};

template <int D>
DkvPlan dkdv_plan(const dfa_attn_desc& d) {
  using C = DkvCfg<D, kDkvNW>;
  DkvPlan p{dkdv_row_split<D>(d), false, false, 0, INT32_MAX, 1};
  if (pair_is_full(d, C::BK) && d.len_q % C::BQ == 0) return p;
  p.banded = p.rsplit == 1 && d.causal && d.q_start == d.kv_start && d.len_q == d.len_kv &&
             d.len_kv % C::BK == 0 &&
             (d.window <= 0 || (d.window % C::BQ == 0 && d.window >= 2 * C::BK));
  if (!p.banded) return p;
  p.own = C::BK / C::BQ;
  p.wt = d.window > 0 ? int(std::min<int64_t>(d.window / C::BQ, INT32_MAX)) : INT32_MAX;
  p.paired = d.window > 0 && d.window < d.len_q;
  p.launches = 2;
  return p;
}

template <int D>
dfa_status launch_dkdv(const dfa_attn_desc& d, BwdArgs a, hipStream_t s) {
  using C = DkvCfg<D, kDkvNW>;
  const int64_t nkb = cdiv(d.len_kv, C::BK);
  const DkvPlan p = dkdv_plan<D>(d);
  // Row split into the caller's workspace (sized by bwd_workspace_bytes and
  // checked before this call).
  a.rsplit = p.rsplit;
  a.ws = a.rsplit > 1 ? static_cast<float*>(d.workspace) : nullptr;
  a.keys_down = dkdv_keys_down(d);
  dim3 grid(unsigned(nkb) * unsigned(d.heads_kv), unsigned(d.batch), unsigned(a.rsplit));
  auto go = [&](auto kern, const BwdArgs& args, int lds_bytes = C::LDS_BYTES) {
    const dfa_status st = allow_lds(kern, lds_bytes, "dkdv_bf16_kernel");
    if (st != DFA_OK) return st;
    hipLaunchKernelGGL(kern, grid, dim3(C::NT), lds_bytes, s, args);
    return check_launch("dkdv_bf16_kernel");
  };
  // a fully visible pair's key blocks all run the same rows: tile-major order
  if (pair_is_full(d, C::BK) && d.len_q % C::BQ == 0)
    return rsplit_reduce<D>(d, a, s, go(dkdv_bf16_kernel<D, kDkvNW, true, true>, a));
  const bool tm = d.window <= 0;
  if (p.banded) {
    BwdArgs band = a;
    dfa_status st;
    if (p.paired) {  // own rows and window-edge rows, paired (whole span, masked)
      band.pair_wt = p.wt;
      st = go(dkdv_bf16_kernel<D, kDkvNW, false, false, true>, band, C::LDS_BYTES_PAIR);
      band.pair_wt = 0;
    } else {
      band.band_lo = 0;
      band.band_hi = p.own;
      st = tm ? go(dkdv_bf16_kernel<D, kDkvNW, false, true>, band)
              : go(dkdv_bf16_kernel<D, kDkvNW, false, false>, band);
    }
    if (st != DFA_OK) return st;
    band.band_lo = p.own;
    band.band_hi = p.wt;
    return tm ? go(dkdv_bf16_kernel<D, kDkvNW, true, true>, band)
              : go(dkdv_bf16_kernel<D, kDkvNW, true, true, false, true>, band);
  }
  return rsplit_reduce<D>(d, a, s,
                          tm ? go(dkdv_bf16_kernel<D, kDkvNW, false, true>, a)
                             : go(dkdv_bf16_kernel<D, kDkvNW, false, false>, a));
}

// After a launch that split rows (a.rsplit > 1), the fixed-order reduction of
// its slices into dk, dv.
template <int D>
dfa_status rsplit_reduce(const dfa_attn_desc& d, const BwdArgs& a, hipStream_t s, dfa_status st) {
  using C = DkvCfg<D, kDkvNW>;
  if (st != DFA_OK || a.rsplit == 1) return st;
  const int64_t n4 = int64_t(d.batch) * d.len_kv * d.heads_kv * D / 4;
  hipLaunchKernelGGL((dkdv_split_reduce_kernel<C::BK, C::BQ>), dim3(unsigned(cdiv(n4, 256))),
                     dim3(256), 0, s, a, n4, int32_t(d.heads_kv * D / 4));
  return check_launch("dkdv_split_reduce_kernel");
}

}  // namespace

dfa_status launch_dkdv_bf16(const dfa_attn_desc& d, const BwdArgs& a, hipStream_t s) {
  if (d.head_dim == 128) return launch_dkdv<128>(d, a, s);
  return launch_dkdv<64>(d, a, s);
}

bool dkdv_keys_down(const dfa_attn_desc& d) {
  using C = DkvCfg<128, kDkvNW>;
  static_assert(C::BK == DkvCfg<64, kDkvNW>::BK && C::BQ == DkvCfg<64, kDkvNW>::BQ,
                "key blocks and row steps do not depend on head_dim");
  if (d.batch == 0 || d.len_q == 0 || d.len_kv == 0) return false;
  const BwdArgs a = bwd_args_of(d);
  const int64_t nkb = cdiv(d.len_kv, C::BK);
  return dkdv_span(a, (nkb - 1) * C::BK, C::BK, C::BQ).steps > dkdv_span(a, 0, C::BK, C::BQ).steps;
}

int dkdv_launches(const dfa_attn_desc& d) {
  if (d.batch == 0 || d.len_q == 0 || d.len_kv == 0) return 0;
  if (d.dtype != DFA_BF16) return 1;
  return d.head_dim == 128 ? dkdv_plan<128>(d).launches : dkdv_plan<64>(d).launches;
}

int64_t dkdv_split_bytes_per_slice(const dfa_attn_desc& d) {
  return int64_t(2) * d.batch * d.len_kv * d.heads_kv * d.head_dim * int64_t(sizeof(float));
}

int64_t dkdv_workspace_bytes(const dfa_attn_desc& d) {
  if (d.batch == 0 || d.len_q == 0 || d.len_kv == 0) return 0;
  const int split = d.head_dim == 128 ? dkdv_row_split<128>(d) : dkdv_row_split<64>(d);
  return split > 1 ? split * dkdv_split_bytes_per_slice(d) : 0;
}

}  // namespace dfa
