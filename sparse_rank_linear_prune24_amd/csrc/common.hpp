// Internal helpers shared by the gfx950 kernels of libsplr (not part of the public ABI).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace splr {

typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x16_t __attribute__((ext_vector_type(16)));
typedef float f32x4_t __attribute__((ext_vector_type(4)));
typedef float f32x2_t __attribute__((ext_vector_type(2)));
typedef uint32_t u32x4_t __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2_t __attribute__((ext_vector_type(2)));
typedef uint16_t u16x4_t __attribute__((ext_vector_type(4)));

constexpr int kWave = 64;

__device__ __forceinline__ bf16x8_t as_bf16x8(u32x4_t v) { return __builtin_bit_cast(bf16x8_t, v); }

__device__ __forceinline__ bf16x16_t cat16(bf16x8_t lo, bf16x8_t hi) {
  return __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7, 8, 9, 10, 11, 12, 13, 14, 15);
}

__device__ __forceinline__ float bf16_bits_to_float(uint32_t b) { return __uint_as_float(b << 16); }

// float -> bfloat16 bits, round to nearest even (NaN stays a quiet NaN). Branch-free: both results
// are formed and one is selected.
__device__ __forceinline__ uint32_t float_to_bf16_bits(float f) {
  const uint32_t u = __float_as_uint(f);
  const uint32_t rounded = (u + 0x7FFFu + ((u >> 16) & 1u)) >> 16;
  const uint32_t quiet_nan = (u >> 16) | 0x40u;
  return (u & 0x7FFFFFFFu) > 0x7F800000u ? quiet_nan : rounded;
}

// Split eight float32 values into bfloat16 high parts and bfloat16 corrections:
// x ~= hi + lo with |x - hi - lo| <= 2^-18 |x| (about 16 significant bits).
__device__ __forceinline__ void split_hi_lo(const float (&x)[8], bf16x8_t& hi, bf16x8_t& lo) {
  u32x4_t h, l;
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    uint32_t h0 = float_to_bf16_bits(x[2 * i]), h1 = float_to_bf16_bits(x[2 * i + 1]);
    uint32_t l0 = float_to_bf16_bits(x[2 * i] - bf16_bits_to_float(h0));
    uint32_t l1 = float_to_bf16_bits(x[2 * i + 1] - bf16_bits_to_float(h1));
    h[i] = h0 | (h1 << 16);
    l[i] = l0 | (l1 << 16);
  }
  hi = as_bf16x8(h);
  lo = as_bf16x8(l);
}

__device__ __forceinline__ f32x4_t mfma16x16x32(bf16x8_t a, bf16x8_t b, f32x4_t c) {
  return __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, c, 0, 0, 0);
}

// Structured-sparse MFMA, 16x16 output, 64 dense K. A: 8 kept bf16 per lane (4 groups of the
// lane's 16-column K slice), B: 16 bf16 per lane, idx: the lane's 4 group nibbles in bits [15:0].
__device__ __forceinline__ f32x4_t smfmac16x16x64(bf16x8_t a, bf16x16_t b, f32x4_t c, int idx) {
  return __builtin_amdgcn_smfmac_f32_16x16x64_bf16(a, b, c, idx, 0, 0);
}
// The same with the index taken from bits [31:16] of `idx` when ABID is 1 (bits [15:0] when 0): a
// 32-bit metadata word holds the indices of two tile columns.
template <int ABID>
__device__ __forceinline__ f32x4_t smfmac16x16x64_half(bf16x8_t a, bf16x16_t b, f32x4_t c, uint32_t idx) {
  return __builtin_amdgcn_smfmac_f32_16x16x64_bf16(a, b, c, (int)idx, 0, ABID);
}

// Keep positions of four keys (2:4 projection): i outranks j <=> k_i > k_j, or k_i == k_j and i < j. An
// entry is kept iff it outranks at least two of the other three (ranks of four entries in a
// strict order are 3, 2, 1, 0). Returns the nibble (a | b << 2) and the kept bit patterns.
template <typename Key>
__device__ __forceinline__ uint32_t top2_of_4(Key k0, Key k1, Key k2, Key k3, uint32_t e0, uint32_t e1, uint32_t e2,
                                              uint32_t e3, uint32_t& va, uint32_t& vb) {
  int w0, w1, w2, w3;
  if constexpr (sizeof(Key) == 8) {
    // 64-bit keys: one compare per pair (k_j > k_i is 1 - (k_i >= k_j) for totally ordered keys)
    const int c01 = k0 >= k1, c02 = k0 >= k2, c03 = k0 >= k3, c12 = k1 >= k2, c13 = k1 >= k3, c23 = k2 >= k3;
    w0 = c01 + c02 + c03;
    w1 = 1 - c01 + c12 + c13;
    w2 = 2 - c02 - c12 + c23;
    w3 = 3 - c03 - c13 - c23;
  } else {
    // 32-bit keys: both compares of a pair are cheap, and this form measured slightly faster
    w0 = (k0 >= k1) + (k0 >= k2) + (k0 >= k3);
    w1 = (k1 > k0) + (k1 >= k2) + (k1 >= k3);
    w2 = (k2 > k0) + (k2 > k1) + (k2 >= k3);
    w3 = (k3 > k0) + (k3 > k1) + (k3 > k2);
  }
  const bool keep0 = w0 >= 2, keep1 = w1 >= 2, keep2 = w2 >= 2, keep3 = w3 >= 2;
  const int a = keep0 ? 0 : (keep1 ? 1 : 2);
  const int b = keep3 ? 3 : (keep2 ? 2 : 1);
  va = keep0 ? e0 : (keep1 ? e1 : e2);
  vb = keep3 ? e3 : (keep2 ? e2 : e1);
  return (uint32_t)(a | (b << 2));
}

__host__ __device__ constexpr inline int64_t ceil_div(int64_t a, int64_t b) { return (a + b - 1) / b; }

// Packed metadata: blocks of 8 tile columns of one tile row (TKB = ceil(TK / 8) per tile row),
// 1 KiB each; slot L (the lane of the MFMA operand: row L % 16, groups 4 (L / 16) .. +3 of a tile)
// owns 16 bytes, one 16-bit unit per tile column, the unit of tile column tk at 2 (tk % 8). Group
// gi of the tile sits at bits 4 (gi % 4) of its unit.
__host__ __device__ constexpr inline int meta_blocks(int TK) { return (TK + 7) / 8; }
__device__ __forceinline__ uint32_t meta_unit(const uint32_t* __restrict__ meta, int TKB, int64_t tr, int tk, int L) {
  return ((const uint16_t*)meta)[(((size_t)tr * TKB + tk / 8) * 64 + L) * 8 + tk % 8];
}

}  // namespace splr
