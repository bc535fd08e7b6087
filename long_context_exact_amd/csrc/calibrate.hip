// Matrix-core calibration (test support, not on the hot path): a loop of
// v_mfma_f32_32x32x16_bf16 with operands in registers, no memory traffic, so
// that timing it for several seconds gives the dense bf16 rate this board
// sustains under its power and current limits -- the practical ceiling the
// attention kernels are compared with, beside the published peak.
#include "kernels.hpp"

#pragma clang diagnostic ignored "-Winline-asm"

namespace dfa {
namespace {

// Every wave runs four independent accumulation chains.  With random_ops the
// operands are eight pseudo-random bf16 pairs per lane (xorshift bits, like
// real data), a different pair for every product, so the datapath inputs keep
// switching; otherwise one constant pair (the least switching).
// Two waves per SIMD, like the attention kernels.
// With kAgprAcc the accumulators are pinned to the accumulation registers
// (AGPRs) through the instruction's register constraints.
template <bool kAgprAcc>
__global__ __launch_bounds__(256) __attribute__((amdgpu_waves_per_eu(2, 2)))
void mfma_loop_kernel(float* sink, int32_t iters, int32_t random_ops) {
  const int t = threadIdx.x;
  bf16x8 a[8], b[8];
  uint32_t h = 2654435761u * (blockIdx.x * 256u + t + 1u);
  for (int j = 0; j < 8; ++j)
    for (int e = 0; e < 8; ++e) {
      if (random_ops) {
        h ^= h << 13; h ^= h >> 17; h ^= h << 5;
        a[j][e] = static_cast<__bf16>(float(int(h & 0xffffu)) / 32768.0f - 1.0f);
        h ^= h << 13; h ^= h >> 17; h ^= h << 5;
        b[j][e] = static_cast<__bf16>(float(int(h & 0xffffu)) / 32768.0f - 1.0f);
      } else {
        a[j][e] = static_cast<__bf16>(0.001f * float(t + e));
        b[j][e] = static_cast<__bf16>(0.002f * float(e));
      }
    }
  f32x16 acc[4];
  for (int c = 0; c < 4; ++c) acc[c] = f32x16{};
  if constexpr (kAgprAcc) {
    for (int i = 0; i < iters; i += 2) {
#pragma unroll
      for (int c = 0; c < 4; ++c)
        asm volatile("v_mfma_f32_32x32x16_bf16 %0, %1, %2, %0" : "+a"(acc[c]) : "v"(a[c]), "v"(b[c]));
#pragma unroll
      for (int c = 0; c < 4; ++c)
        asm volatile("v_mfma_f32_32x32x16_bf16 %0, %1, %2, %0"
                     : "+a"(acc[c]) : "v"(a[c + 4]), "v"(b[c + 4]));
    }
  } else {
    for (int i = 0; i < iters; i += 2) {
#pragma unroll
      for (int c = 0; c < 4; ++c) acc[c] = mfma32(a[c], b[c], acc[c]);
#pragma unroll
      for (int c = 0; c < 4; ++c) acc[c] = mfma32(a[c + 4], b[c + 4], acc[c]);
    }
  }
  float s = 0.f;
  for (int c = 0; c < 4; ++c) s += acc[c][0] + acc[c][15];
  if (s == 12345.0f) sink[blockIdx.x * 256 + t] = s;  // keeps the products; practically never stores
}

}  // namespace

dfa_status launch_mfma_loop(int32_t workgroups, int32_t iters, int32_t mode, float* sink,
                            hipStream_t s) {
  if (mode & 2)
    hipLaunchKernelGGL(mfma_loop_kernel<true>, dim3(unsigned(workgroups)), dim3(256), 0, s, sink,
                       iters, mode & 1);
  else
    hipLaunchKernelGGL(mfma_loop_kernel<false>, dim3(unsigned(workgroups)), dim3(256), 0, s, sink,
                       iters, mode & 1);
  return check_launch("mfma_loop_kernel");
}

}  // namespace dfa
