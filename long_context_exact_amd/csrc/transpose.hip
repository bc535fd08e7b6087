// Transposed key/value copies for the products that contract over keys.
#include "kernels.hpp"

namespace dfa {
namespace {

// X [B][len][H][D] -> X^T [B][H][D][ld] (X = K or V): per 64 keys, staged
// through LDS; within every 16-key group the key with index bits (b3 b2 b1
// b0) is stored at position (b2 b3 b1 b0), the order in which a 32x32
// accumulator hands its key axis over as the B operand of the next product
// (P^T in the forward's P V); keys past len are 0.
template <int D>
__global__ __launch_bounds__(256) void kv_transpose_kernel(const uint16_t* v, uint16_t* vt,
                                                           int64_t len, int32_t heads, int64_t ld) {
  constexpr int CPR = D / 8;  // 16-byte chunks per key row
  __shared__ __align__(16) uint16_t tile[64][D + 8];
  const int64_t k0 = int64_t(blockIdx.x) * 64;
  const int64_t bg = blockIdx.y;  // b * heads + g
  const int64_t b = bg / heads;
  const int g = int(bg % heads);
  const int t = threadIdx.x;
  for (int c = t; c < 64 * CPR; c += 256) {
    const int r = c / CPR, ch = c % CPR;
    const int64_t key = k0 + r;
    uint4 val = make_uint4(0u, 0u, 0u, 0u);
    if (key < len) val = *reinterpret_cast<const uint4*>(v + ((b * len + key) * heads + g) * D + ch * 8);
    *reinterpret_cast<uint4*>(&tile[r][ch * 8]) = val;
  }
  __syncthreads();
  for (int c = t; c < D * 8; c += 256) {
    const int dd = c / 8, p8 = c % 8;  // 8 positions 8*p8 .. 8*p8+7 of row dd
    typedef unsigned short u16x8 __attribute__((ext_vector_type(8)));
    u16x8 out;
#pragma unroll
    for (int e = 0; e < 8; ++e) {
      const int pos = p8 * 8 + e;
      const int w = pos & 15;
      out[e] = tile[(pos & ~15) | (w & 3) | ((w & 4) << 1) | ((w & 8) >> 1)][dd];
    }
    *reinterpret_cast<u16x8*>(vt + (bg * D + dd) * ld + k0 + p8 * 8) = out;
  }
}

}  // namespace

dfa_status launch_kv_transpose(const uint16_t* x, uint16_t* xt, int32_t batch, int64_t len,
                               int32_t heads, int32_t head_dim, int64_t ld, hipStream_t s) {
  if (ld % 64 != 0 || ld < len) return fail(DFA_ERR_INVALID, "launch_kv_transpose: bad ld");
  if (ld == 0) return DFA_OK;
  const dim3 grid(unsigned(ld / 64), unsigned(batch) * unsigned(heads));
  if (head_dim == 128)
    hipLaunchKernelGGL(kv_transpose_kernel<128>, grid, dim3(256), 0, s, x, xt, len, heads, ld);
  else
    hipLaunchKernelGGL(kv_transpose_kernel<64>, grid, dim3(256), 0, s, x, xt, len, heads, ld);
  return check_launch("kv_transpose_kernel");
}

}  // namespace dfa
