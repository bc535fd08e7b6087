// Internal helpers shared by the gfx950 kernels of libdfa: vector types,
// the bf16 MFMA wrapper, bf16 conversion and cross-lane helpers.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include <cmath>
#include <string>

#include "dfa.h"
#include "errors.hpp"

namespace dfa {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x4 __attribute__((ext_vector_type(4)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef float f32x4 __attribute__((ext_vector_type(4)));

constexpr float kLog2e = 1.4426950408889634f;
constexpr float kLn2 = 0.6931471805599453f;

// 32x32x16 bf16 matrix FMA, fp32 accumulate (one wave).  Operand layout, with
// l the lane (0..63) and e the vector element (0..7):
//   A[i][k]: i = l % 32, k = 8 * (l / 32) + e
//   B[k][j]: j = l % 32, k = 8 * (l / 32) + e
//   C[i][j] element r (0..15): j = l % 32, i = 8 * (r / 4) + 4 * (l / 32) + r % 4
__device__ __forceinline__ f32x16 mfma32(bf16x8 a, bf16x8 b, f32x16 c) {
  return __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, c, 0, 0, 0);
}

// 16x16x32 bf16 matrix FMA, fp32 accumulate (one wave):
//   A[i][k]: i = l % 16, k = 8 * (l / 16) + e
//   B[k][j]: j = l % 16, k = 8 * (l / 16) + e
//   C[i][j] element r (0..3): j = l % 16, i = 4 * (l / 16) + r
__device__ __forceinline__ f32x4 mfma16(bf16x8 a, bf16x8 b, f32x4 c) {
  return __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, c, 0, 0, 0);
}

__device__ __forceinline__ float exp2_fast(float x) { return __builtin_amdgcn_exp2f(x); }

// Value of `x` held by lane (l ^ 32) of the wave.
__device__ __forceinline__ float xor32(float x) { return __shfl_xor(x, 32); }
// max(x, x of lane l ^ 32) in one v_permlane32_swap (no LDS round trip).
__device__ __forceinline__ float max_xor32(float x) {
  const unsigned u = __builtin_bit_cast(unsigned, x);
  const auto r = __builtin_amdgcn_permlane32_swap(u, u, false, false);
  return fmaxf(__builtin_bit_cast(float, unsigned(r[0])), __builtin_bit_cast(float, unsigned(r[1])));
}

__device__ __forceinline__ bf16x8 ld_bf16x8(const uint16_t* p) {
  return __builtin_bit_cast(bf16x8, *reinterpret_cast<const uint4*>(p));
}

__device__ __forceinline__ uint4 ld_u4(const uint16_t* p) {
  return *reinterpret_cast<const uint4*>(p);
}

__device__ __forceinline__ bf16x8 cat4(bf16x4 a, bf16x4 b) {
  return bf16x8{a[0], a[1], a[2], a[3], b[0], b[1], b[2], b[3]};
}

// ---- row-major bf16 tiles in LDS ------------------------------------------
// A tile holds rows of D bf16 (no padding).  gfx950's LDS serves 256 bytes
// (64 four-byte banks) per cycle; a ds_read_b128 takes four cycles, each
// serving the 16 lanes that agree in lane bit 5 and in the parity of lane
// bits 2..4 (measured with the bank-conflict counter).  The 16-byte chunks
// are XOR-swizzled per row such that each of these touches 16 distinct
// 16-byte slots of a 256-byte bank line:
//  * a 16-byte fragment read of one chunk where lane l reads row l % 32
//    (each cycle then holds 16 rows that differ mod 16),
//  * a 32x32-operand transpose read: 4 consecutive rows x 4 adjacent chunks,
//  * a 16x16-operand transpose read: 8 consecutive rows x 2 adjacent chunks,
//  * a 16-byte store of 16 consecutive chunks (one row, or two of D = 64).
// Chunk c of row r sits at c ^ g(r) with
//   D = 128: g = 4 * (r % 4) + 2 * ((r / 4) % 2) + (r / 8) % 2,
//   D = 64:  g = 4 * ((r / 2) % 2) + 2 * ((r / 4) % 2) + (r / 8) % 2.
template <int D>
__device__ __forceinline__ int swz(int row, int chunk) {
  static_assert(D == 64 || D == 128, "tile rows of 64 or 128 elements");
  const int lo = (((row >> 2) & 1) << 1) | ((row >> 3) & 1);
  const int g = D == 128 ? (((row & 3) << 2) | lo) : ((((row >> 1) & 1) << 2) | lo);
  return row * D + ((chunk ^ g) << 3);
}

// LDS pointers carry the LDS address space, so tile addressing stays 32-bit.
#define DFA_LDS __attribute__((address_space(3)))
typedef DFA_LDS uint16_t lds_u16;
typedef DFA_LDS float lds_f32;
typedef short i16x4 __attribute__((ext_vector_type(4)));

__device__ __forceinline__ lds_u16* lds_base(uint16_t* generic_smem) {
  return (lds_u16*)(generic_smem);
}

// 8 consecutive elements (one chunk) of one row.
typedef unsigned u32x4 __attribute__((ext_vector_type(4)));

template <int D>
__device__ __forceinline__ bf16x8 tile_row8(const lds_u16* t, int row, int chunk) {
  return __builtin_bit_cast(bf16x8, *(const DFA_LDS u32x4*)(t + swz<D>(row, chunk)));
}

template <int D>
__device__ __forceinline__ void tile_store16(lds_u16* t, int row, int chunk, uint4 v) {
  *(DFA_LDS u32x4*)(t + swz<D>(row, chunk)) = u32x4{v.x, v.y, v.z, v.w};
}

// Transpose read (ds_read_b64_tr_b16).  Within each group of 16 lanes, lane j
// fetches 4 elements at (row0 + j/4, col0 + 4*(j%4)); the hardware returns to
// lane i the elements (row0 + e, col0 + i), e = 0..3.  So each lane receives
// 4 consecutive rows of its own column: an MFMA operand whose contraction
// index runs along the tile's rows.  row0 % 4 == 0, col0 % 16 == 0.
template <int D>
__device__ __forceinline__ bf16x4 tile_tr4(const lds_u16* t, int row0, int col0, int lane) {
  const int j = lane & 15;
  const int row = row0 + (j >> 2);
  const int col = col0 + 4 * (j & 3);
  const lds_u16* p = t + swz<D>(row, col >> 3) + (col & 4);
  const i16x4 r = __builtin_amdgcn_ds_read_tr16_b64_v4i16((DFA_LDS i16x4*)(p));
  return __builtin_bit_cast(bf16x4, r);
}

// Direct global -> LDS transfer of 16 bytes per lane (global_load_lds_dwordx4):
// lane i writes the 16 bytes at LDS byte address M0 + 16 * i.  Issued from
// inline assembly on purpose: when the compiler sees these transfers it makes
// every later LDS read it cannot prove disjoint from them (the transposed
// reads) wait for all of them, which stalls each tile loop on the prefetch of
// its next tile.  Callers instead order the transfers themselves with
// wait_vmem() and a barrier before the staged tile is read.  M0 is set
// inside each statement (1 wait state before the transfer reads it); no other
// code in these kernels uses M0.
#pragma clang diagnostic push
#pragma clang diagnostic ignored "-Winline-asm"
__device__ __forceinline__ void lds_dma16(const void* base, uint32_t off, const void DFA_LDS* dst_wave) {
  const uint32_t m0 = __builtin_amdgcn_readfirstlane(
      static_cast<uint32_t>(reinterpret_cast<uintptr_t>(dst_wave)));
  asm volatile("s_mov_b32 m0, %0\n\ts_nop 0\n\tglobal_load_lds_dwordx4 %1, %2"
               :: "s"(m0), "v"(off), "s"(base) : "memory", "m0");
}
#pragma clang diagnostic pop

// Staging of segment `seg` (1 KiB) of a swizzled tile: row r of the tile is
// read from tile_base + r * row_bytes (tile_base wave-uniform, so each lane
// adds only a 32-bit offset), and rows past `last_row` re-read row last_row
// (ragged ends; those rows are masked by the caller).  To land chunk c of row
// r at its swizzled slot, the lane whose slot is (r, p) loads the global
// chunk c = p ^ g(r).
template <int D>
__device__ __forceinline__ void tile_dma_rows(lds_u16* tile, int seg, int lane, const uint16_t* tile_base,
                                              uint32_t row_bytes, int last_row) {
  constexpr int ROWS_PER_SEG = 512 / D;  // 1 KiB / (2 bytes * D)
  constexpr int CHUNKS = D / 8;
  const int row = seg * ROWS_PER_SEG + lane / CHUNKS;
  // logical chunk whose swizzled slot is lane % CHUNKS (g is an involution partner)
  const int logical = (swz<D>(row, lane % CHUNKS) - row * D) >> 3;
  const uint32_t off = uint32_t(min(row, last_row)) * row_bytes + uint32_t(logical) * 16u;
  lds_dma16(tile_base, off, tile + seg * 512);
}

// Wait for this wave's outstanding global loads (including LDS-direct ones).
__device__ __forceinline__ void wait_vmem() { __builtin_amdgcn_s_waitcnt(0x0F70); }

// Round-to-nearest-even fp32 -> bf16 of 8 consecutive accumulator elements.
__device__ __forceinline__ bf16x8 pack8(const float* p) {
  bf16x8 r;
#pragma unroll
  for (int e = 0; e < 8; ++e) r[e] = static_cast<__bf16>(p[e]);
  return r;
}

__device__ __forceinline__ float bf16_to_f32(uint16_t u) {
  return __uint_as_float(static_cast<uint32_t>(u) << 16);
}

__device__ __forceinline__ uint16_t f32_to_bf16_rne(float f) {
  return __builtin_bit_cast(uint16_t, static_cast<__bf16>(f));
}

// Maps a pending HIP launch error to DFA_ERR_HIP (with the HIP message).
dfa_status check_launch(const char* what);

__host__ __device__ inline int64_t cdiv(int64_t a, int64_t b) { return (a + b - 1) / b; }

// A 64-bit offset clamped into [-2^30, 2^30]: mask bounds compared against
// in-tile offsets (< 2^8) keep their meaning and become 32-bit compares.
__device__ __forceinline__ int clamp_off(int64_t x) {
  return static_cast<int>(max<int64_t>(-(int64_t(1) << 30), min<int64_t>(x, int64_t(1) << 30)));
}

}  // namespace dfa
