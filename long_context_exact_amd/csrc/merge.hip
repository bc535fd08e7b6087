// HBM-bound helpers of the hot path: the LSE merge of partial states, the
// backward preprocess delta = rowsum(dO * O), and the empty-pair fill.
//
// LSE merge ([DistFlashAttn §3.2, Fig. 3]: the owner rescales and sums the
// per-pair outputs its helpers send back, each with its log-sum-exp):
//   M = max_r LSE_r, LSE = M + ln sum_r exp(LSE_r - M),
//   O = sum_r exp(LSE_r - LSE) O_r          (ascending r, fp32).
// One thread owns 4 consecutive head_dim elements of one (row, head); the
// n partial pointers travel in the kernel arguments.
#include <algorithm>
#include <type_traits>

#include "kernels.hpp"

namespace dfa {
namespace {

constexpr int kMaxParts = 64;

struct MergeArgs {
  const float* o[kMaxParts];
  const float* lse[kMaxParts];
  void* o_out;
  float* lse_out;
  int64_t rows;      // batch * len_q * heads (row-head pairs)
  int64_t len_q;
  int32_t heads, n, d4;  // d4 = head_dim / 4
};

template <bool BF16_OUT>
__global__ __launch_bounds__(256) void merge_kernel(MergeArgs a) {
  const int64_t t = int64_t(blockIdx.x) * 256 + threadIdx.x;
  const int64_t rh = t / a.d4;  // (b, i, h) row-head index, h fastest
  const int c4 = int(t % a.d4);
  if (rh >= a.rows) return;
  const int h = int(rh % a.heads);
  const int64_t bi = rh / a.heads;  // b * len_q + i
  const int64_t b = bi / a.len_q, i = bi % a.len_q;
  const int64_t lidx = (b * a.heads + h) * a.len_q + i;

  float mx = -INFINITY;
  for (int r = 0; r < a.n; ++r) mx = fmaxf(mx, a.lse[r][lidx]);
  f32x4 acc = {0.f, 0.f, 0.f, 0.f};
  float out_lse = -INFINITY;
  if (mx > -INFINITY) {
    float tot = 0.f;
    for (int r = 0; r < a.n; ++r) tot += expf(a.lse[r][lidx] - mx);
    out_lse = mx + logf(tot);
    // Eight partials' loads in flight before the first is used (one at a
    // time leaves HBM half idle); the sum keeps its ascending order.
    constexpr int U = 8;
    int r = 0;
    for (; r + U <= a.n; r += U) {
      f32x4 x[U];
#pragma unroll
      for (int u = 0; u < U; ++u) x[u] = reinterpret_cast<const f32x4*>(a.o[r + u] + rh * 4 * a.d4)[c4];
#pragma unroll
      for (int u = 0; u < U; ++u) acc += expf(a.lse[r + u][lidx] - out_lse) * x[u];
    }
    for (; r < a.n; ++r) {
      const float w = expf(a.lse[r][lidx] - out_lse);
      const f32x4 x = reinterpret_cast<const f32x4*>(a.o[r] + rh * 4 * a.d4)[c4];
      acc += w * x;
    }
  }
  if (BF16_OUT) {
    uint16_t* out = static_cast<uint16_t*>(a.o_out) + rh * 4 * a.d4 + 4 * c4;
    const uint32_t lo = uint32_t(f32_to_bf16_rne(acc[0])) | (uint32_t(f32_to_bf16_rne(acc[1])) << 16);
    const uint32_t hi = uint32_t(f32_to_bf16_rne(acc[2])) | (uint32_t(f32_to_bf16_rne(acc[3])) << 16);
    *reinterpret_cast<uint2*>(out) = make_uint2(lo, hi);
  } else {
    reinterpret_cast<f32x4*>(static_cast<float*>(a.o_out) + rh * 4 * a.d4)[c4] = acc;
  }
  // All threads of one row-head sit in one wave (head_dim / 4 <= 32 divides
  // 64), so every read of LSE_r above precedes this write in the wave's
  // program order: lse_out may alias lse_parts[0].
  if (c4 == 0) a.lse_out[lidx] = out_lse;
}

// delta[b, h, i] = sum_d dO[b, i, h, d] * O[b, i, h, d]; 8 elements per
// lane, head_dim / 8 lanes per row (a power of two <= 16).  fp32 inputs (the
// exact path) sum in fp64, bf16 inputs in fp32.
template <typename T, int D>
__global__ __launch_bounds__(256) void delta_kernel(const T* o, const T* d_o, float* delta,
                                                    int64_t rows, int64_t len_q, int32_t heads) {
  using Acc = std::conditional_t<sizeof(T) == 2, float, double>;
  constexpr int LPR = D / 8;
  const int64_t t = int64_t(blockIdx.x) * 256 + threadIdx.x;
  const int64_t rh = t / LPR;
  const int c = int(t % LPR);
  Acc s = 0;
  if (rh < rows) {
    const T* po = o + rh * D + 8 * c;
    const T* pd = d_o + rh * D + 8 * c;
#pragma unroll
    for (int e = 0; e < 8; ++e) {
      Acc x, y;
      if constexpr (sizeof(T) == 2) {
        x = bf16_to_f32(po[e]);
        y = bf16_to_f32(pd[e]);
      } else {
        x = po[e];
        y = pd[e];
      }
      s += x * y;
    }
  }
#pragma unroll
  for (int off = LPR / 2; off > 0; off >>= 1) s += __shfl_xor(s, off);
  if (rh < rows && c == 0) {
    const int h = int(rh % heads);
    const int64_t bi = rh / heads;
    delta[((bi / len_q) * heads + h) * len_q + bi % len_q] = float(s);
  }
}

__global__ __launch_bounds__(256) void fill_kernel(float* o, int64_t n_o, float* lse,
                                                   int64_t n_lse) {
  const int64_t stride = int64_t(gridDim.x) * 256;
  for (int64_t i = int64_t(blockIdx.x) * 256 + threadIdx.x; i < n_o; i += stride) o[i] = 0.f;
  for (int64_t i = int64_t(blockIdx.x) * 256 + threadIdx.x; i < n_lse; i += stride)
    lse[i] = -INFINITY;
}

}  // namespace

dfa_status launch_merge(int32_t n, const float* const* o_parts, const float* const* lse_parts,
                        int32_t batch, int32_t heads, int64_t len_q, int32_t head_dim,
                        int32_t out_dtype, void* o_out, float* lse_out, hipStream_t s) {
  MergeArgs a{};
  for (int r = 0; r < n; ++r) {
    a.o[r] = o_parts[r];
    a.lse[r] = lse_parts[r];
  }
  a.o_out = o_out;
  a.lse_out = lse_out;
  a.rows = int64_t(batch) * len_q * heads;
  a.len_q = len_q;
  a.heads = heads;
  a.n = n;
  a.d4 = head_dim / 4;
  const int64_t threads = a.rows * a.d4;
  if (threads == 0) return DFA_OK;
  const dim3 grid(unsigned(cdiv(threads, 256)));
  if (out_dtype == DFA_BF16)
    hipLaunchKernelGGL(merge_kernel<true>, grid, dim3(256), 0, s, a);
  else
    hipLaunchKernelGGL(merge_kernel<false>, grid, dim3(256), 0, s, a);
  return check_launch("merge_kernel");
}

dfa_status launch_delta(const dfa_attn_desc& d, const void* o, const void* d_o, float* delta,
                        hipStream_t s) {
  const int64_t rows = int64_t(d.batch) * d.len_q * d.heads_q;
  if (rows == 0) return DFA_OK;
  const dim3 grid(unsigned(cdiv(rows * (d.head_dim / 8), 256)));
  if (d.dtype == DFA_BF16) {
    auto po = static_cast<const uint16_t*>(o);
    auto pd = static_cast<const uint16_t*>(d_o);
    if (d.head_dim == 128)
      hipLaunchKernelGGL((delta_kernel<uint16_t, 128>), grid, dim3(256), 0, s, po, pd, delta,
                         rows, d.len_q, d.heads_q);
    else
      hipLaunchKernelGGL((delta_kernel<uint16_t, 64>), grid, dim3(256), 0, s, po, pd, delta,
                         rows, d.len_q, d.heads_q);
  } else {
    auto po = static_cast<const float*>(o);
    auto pd = static_cast<const float*>(d_o);
    if (d.head_dim == 128)
      hipLaunchKernelGGL((delta_kernel<float, 128>), grid, dim3(256), 0, s, po, pd, delta, rows,
                         d.len_q, d.heads_q);
    else
      hipLaunchKernelGGL((delta_kernel<float, 64>), grid, dim3(256), 0, s, po, pd, delta, rows,
                         d.len_q, d.heads_q);
  }
  return check_launch("delta_kernel");
}

dfa_status launch_fill_empty(int64_t n_o, float* o, int64_t n_lse, float* lse, hipStream_t s) {
  if (n_o == 0 && n_lse == 0) return DFA_OK;
  const int64_t blocks = std::min<int64_t>(4096, cdiv(std::max(n_o, n_lse), 256));
  hipLaunchKernelGGL(fill_kernel, dim3(unsigned(blocks)), dim3(256), 0, s, o, n_o, lse, n_lse);
  return check_launch("fill_kernel");
}

}  // namespace dfa
