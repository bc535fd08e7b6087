// Exact fp32 forward and backward of one chunk pair (fp32 inputs).
//
// These kernels carry the fp32 workloads, whose tolerance (1e-5 absolute
// against float64) rules out bf16 MFMA.  One wave owns one query row (or
// one key row in the dK/dV kernel); lanes split head_dim, dot products are
// wave reductions.  Inputs and outputs are fp32, but scores, exponentials
// and every sum are carried in fp64: a gradient summed over a head group
// and a few hundred rows in fp32 drifts past 1e-5 once it reaches ~10, while
// in fp64 only the final rounding to fp32 remains.  Same semantics as the
// MFMA path: causal prefix only, partial O plus natural-log LSE, backward
// from the saved O and LSE.
#include "kernels.hpp"

namespace dfa {
namespace {

__device__ __forceinline__ double wave_sum(double x) {
#pragma unroll
  for (int off = 32; off > 0; off >>= 1) x += __shfl_xor(x, off);
  return x;
}

struct F32Args {
  const float* q;
  const float* k;
  const float* v;
  const float* o;
  const float* d_o;
  const float* lse;
  const float* delta;
  float* out_o;
  float* out_lse;
  float* dq;
  float* dk;
  float* dv;
  int64_t len_q, len_kv, q_start, kv_start;
  int32_t hq, hkv, group, causal;
  float scale;
  int64_t win;  // sliding window in tokens; a huge value when there is none
};

// Lanes hold head_dim elements lane and lane + 64 (when D == 128).
template <int D>
struct Row {
  float x[D / 64];
  __device__ void load(const float* p, int lane) {
#pragma unroll
    for (int i = 0; i < D / 64; ++i) x[i] = p[lane + 64 * i];
  }
  __device__ double dot(const Row& o) const {
    double s = 0.0;
#pragma unroll
    for (int i = 0; i < D / 64; ++i) s += double(x[i]) * double(o.x[i]);
    return wave_sum(s);
  }
};

// Keys [first_key, visible_keys) of the chunk are visible to local query
// row `row`: the causal prefix, cut below by the sliding window.
__device__ __forceinline__ int64_t visible_keys(const F32Args& a, int64_t row) {
  if (!a.causal) return a.len_kv;
  const int64_t lim = a.q_start + row - a.kv_start + 1;
  return lim < 0 ? 0 : min(lim, a.len_kv);
}
__device__ __forceinline__ int64_t first_key(const F32Args& a, int64_t row) {
  return max<int64_t>(0, a.q_start + row - a.win + 1 - a.kv_start);
}

template <int D>
__global__ __launch_bounds__(256) void fwd_f32_kernel(F32Args a) {
  const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
  const int64_t row = int64_t(blockIdx.x) * 4 + wave;
  const int h = blockIdx.y;
  const int64_t b = blockIdx.z;
  if (row >= a.len_q) return;
  const int g = h / a.group;
  const int64_t q_rs = int64_t(a.hq) * D, kv_rs = int64_t(a.hkv) * D;
  Row<D> q;
  q.load(a.q + (b * a.len_q + row) * q_rs + int64_t(h) * D, lane);
  const float* kb = a.k + b * a.len_kv * kv_rs + int64_t(g) * D;
  const float* vb = a.v + b * a.len_kv * kv_rs + int64_t(g) * D;
  double m = -INFINITY, l = 0.0, acc[D / 64] = {};
  const int64_t nk = visible_keys(a, row);
  for (int64_t j = first_key(a, row); j < nk; ++j) {
    Row<D> k, v;
    k.load(kb + j * kv_rs, lane);
    v.load(vb + j * kv_rs, lane);
    const double s = double(a.scale) * q.dot(k);
    const double m_new = fmax(m, s);
    const double alpha = exp(m - m_new);  // m = -inf on the first key -> 0
    const double p = exp(s - m_new);
    l = l * alpha + p;
#pragma unroll
    for (int i = 0; i < D / 64; ++i) acc[i] = acc[i] * alpha + p * double(v.x[i]);
    m = m_new;
  }
  float* orow = a.out_o + (b * a.len_q + row) * q_rs + int64_t(h) * D;
#pragma unroll
  for (int i = 0; i < D / 64; ++i) orow[lane + 64 * i] = l > 0.0 ? float(acc[i] / l) : 0.f;
  if (lane == 0)
    a.out_lse[(b * a.hq + h) * a.len_q + row] = l > 0.0 ? float(m + log(l)) : -INFINITY;
}

// dQ of one query row: sum over visible keys of dS_ij K_j.
template <int D>
__global__ __launch_bounds__(256) void dq_f32_kernel(F32Args a) {
  const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
  const int64_t row = int64_t(blockIdx.x) * 4 + wave;
  const int h = blockIdx.y;
  const int64_t b = blockIdx.z;
  if (row >= a.len_q) return;
  const float lse = a.lse[(b * a.hq + h) * a.len_q + row];
  if (!(lse > -INFINITY)) return;  // the row saw no key: no gradient
  const float dl = a.delta[(b * a.hq + h) * a.len_q + row];
  const int g = h / a.group;
  const int64_t q_rs = int64_t(a.hq) * D, kv_rs = int64_t(a.hkv) * D;
  Row<D> q, dO;
  q.load(a.q + (b * a.len_q + row) * q_rs + int64_t(h) * D, lane);
  dO.load(a.d_o + (b * a.len_q + row) * q_rs + int64_t(h) * D, lane);
  const float* kb = a.k + b * a.len_kv * kv_rs + int64_t(g) * D;
  const float* vb = a.v + b * a.len_kv * kv_rs + int64_t(g) * D;
  double acc[D / 64] = {};
  const int64_t nk = visible_keys(a, row);
  for (int64_t j = first_key(a, row); j < nk; ++j) {
    Row<D> k, v;
    k.load(kb + j * kv_rs, lane);
    v.load(vb + j * kv_rs, lane);
    const double p = exp(double(a.scale) * q.dot(k) - double(lse));
    const double ds = p * (dO.dot(v) - double(dl));
#pragma unroll
    for (int i = 0; i < D / 64; ++i) acc[i] += ds * double(k.x[i]);
  }
  float* out = a.dq + (b * a.len_q + row) * q_rs + int64_t(h) * D;
#pragma unroll
  for (int i = 0; i < D / 64; ++i) out[lane + 64 * i] += float(double(a.scale) * acc[i]);
}

// dK, dV of one key row of one key/value head: sum over the heads of its
// group and over the query rows that see it.
template <int D>
__global__ __launch_bounds__(256) void dkdv_f32_kernel(F32Args a) {
  const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
  const int64_t j = int64_t(blockIdx.x) * 4 + wave;
  const int g = blockIdx.y;
  const int64_t b = blockIdx.z;
  if (j >= a.len_kv) return;
  const int64_t q_rs = int64_t(a.hq) * D, kv_rs = int64_t(a.hkv) * D;
  Row<D> k, v;
  k.load(a.k + (b * a.len_kv + j) * kv_rs + int64_t(g) * D, lane);
  v.load(a.v + (b * a.len_kv + j) * kv_rs + int64_t(g) * D, lane);
  int64_t i0 = 0;  // first query row that sees key j
  if (a.causal) i0 = max<int64_t>(0, a.kv_start + j - a.q_start);
  // rows past the last one whose window reaches key j
  const int64_t i1 = min<int64_t>(a.len_q, a.kv_start + j + a.win - a.q_start);
  double dk[D / 64] = {}, dv[D / 64] = {};
  for (int hh = 0; hh < a.group; ++hh) {
    const int h = g * a.group + hh;
    for (int64_t i = i0; i < i1; ++i) {
      const float lse = a.lse[(b * a.hq + h) * a.len_q + i];
      if (!(lse > -INFINITY)) continue;
      Row<D> q, dO;
      q.load(a.q + (b * a.len_q + i) * q_rs + int64_t(h) * D, lane);
      dO.load(a.d_o + (b * a.len_q + i) * q_rs + int64_t(h) * D, lane);
      const double p = exp(double(a.scale) * q.dot(k) - double(lse));
      const double ds = p * (dO.dot(v) - double(a.delta[(b * a.hq + h) * a.len_q + i]));
#pragma unroll
      for (int t = 0; t < D / 64; ++t) {
        dv[t] += p * double(dO.x[t]);
        dk[t] += ds * double(q.x[t]);
      }
    }
  }
  float* ok = a.dk + (b * a.len_kv + j) * kv_rs + int64_t(g) * D;
  float* ov = a.dv + (b * a.len_kv + j) * kv_rs + int64_t(g) * D;
#pragma unroll
  for (int t = 0; t < D / 64; ++t) {
    ok[lane + 64 * t] += float(double(a.scale) * dk[t]);
    ov[lane + 64 * t] += float(dv[t]);
  }
}

F32Args make_args(const dfa_attn_desc& d) {
  F32Args a{};
  a.len_q = d.len_q;
  a.len_kv = d.len_kv;
  a.q_start = d.q_start;
  a.kv_start = d.kv_start;
  a.hq = d.heads_q;
  a.hkv = d.heads_kv;
  a.group = d.heads_q / d.heads_kv;
  a.causal = d.causal;
  a.win = d.window > 0 ? d.window : kNoWindow;
  a.scale = d.scale;
  return a;
}

}  // namespace

dfa_status launch_fwd_f32(const dfa_attn_desc& d, const void* q, const void* k, const void* v,
                          float* o, float* lse, hipStream_t s) {
  F32Args a = make_args(d);
  a.q = static_cast<const float*>(q);
  a.k = static_cast<const float*>(k);
  a.v = static_cast<const float*>(v);
  a.out_o = o;
  a.out_lse = lse;
  dim3 grid(unsigned(cdiv(d.len_q, 4)), unsigned(d.heads_q), unsigned(d.batch));
  if (d.head_dim == 128)
    hipLaunchKernelGGL(fwd_f32_kernel<128>, grid, dim3(256), 0, s, a);
  else
    hipLaunchKernelGGL(fwd_f32_kernel<64>, grid, dim3(256), 0, s, a);
  return check_launch("fwd_f32_kernel");
}

dfa_status launch_bwd_f32(const dfa_attn_desc& d, const void* q, const void* k, const void* v,
                          const float* lse, const void* d_o, const float* delta, float* dq,
                          float* dk, float* dv, hipStream_t s, int parts) {
  F32Args a = make_args(d);
  a.q = static_cast<const float*>(q);
  a.k = static_cast<const float*>(k);
  a.v = static_cast<const float*>(v);
  a.d_o = static_cast<const float*>(d_o);
  a.lse = lse;
  a.delta = delta;
  a.dq = dq;
  a.dk = dk;
  a.dv = dv;
  dim3 gq(unsigned(cdiv(d.len_q, 4)), unsigned(d.heads_q), unsigned(d.batch));
  dim3 gk(unsigned(cdiv(d.len_kv, 4)), unsigned(d.heads_kv), unsigned(d.batch));
  if (d.head_dim == 128) {
    if (parts & 2) hipLaunchKernelGGL(dq_f32_kernel<128>, gq, dim3(256), 0, s, a);
    if (parts & 1) hipLaunchKernelGGL(dkdv_f32_kernel<128>, gk, dim3(256), 0, s, a);
  } else {
    if (parts & 2) hipLaunchKernelGGL(dq_f32_kernel<64>, gq, dim3(256), 0, s, a);
    if (parts & 1) hipLaunchKernelGGL(dkdv_f32_kernel<64>, gk, dim3(256), 0, s, a);
  }
  return check_launch("dq_f32_kernel / dkdv_f32_kernel");
}

}  // namespace dfa
