// 2:4 projection + pack on gfx950.
//
// Hard thresholding per group of four (HASSLE-free page, §4.1.1; the 2:4 constraint as in the
// 3BASiL article, "A three-block ADMM replaces alternating minimization"): keep the two entries of
// largest magnitude as bit copies, ties to the lower column.
//
// The work is pure HBM streaming: each lane owns one 16-byte chunk of R per step (two bf16 groups
// or one fp32 group), ranks the four entries of a group with integer compares of the sign-cleared
// bit patterns (six compares, no floating point, so the result is bit-exact and independent of
// denormal modes), writes its kept pair as one 8-byte store, and the lanes of a quad (bf16) or an
// octet (fp32) merge their nibbles into one metadata word with cross-lane shuffles. Loads of a wave
// cover 1 KiB of contiguous R, value stores 512 contiguous bytes.
#include "common.hpp"
#include "kernels.hpp"

namespace splr {
namespace {

constexpr int kPackThreads = 256;
constexpr int kPackIter = 4;  // chunks per lane, loaded before any is processed

// Rank four magnitude keys; returns the keep mask bits for positions a < b via (a, b).
__device__ __forceinline__ void top2_of_4(uint32_t k0, uint32_t k1, uint32_t k2, uint32_t k3, int& a,
                                          int& b, bool& keep0, bool& keep1, bool& keep2, bool& keep3) {
  // i outranks j  <=>  k_i > k_j, or k_i == k_j and i < j.  An entry is kept iff it outranks at
  // least two of the other three (the ranks of four distinct-by-order entries are 3, 2, 1, 0).
  const int w0 = (k0 >= k1) + (k0 >= k2) + (k0 >= k3);
  const int w1 = (k1 > k0) + (k1 >= k2) + (k1 >= k3);
  const int w2 = (k2 > k0) + (k2 > k1) + (k2 >= k3);
  const int w3 = (k3 > k0) + (k3 > k1) + (k3 > k2);
  keep0 = w0 >= 2;
  keep1 = w1 >= 2;
  keep2 = w2 >= 2;
  keep3 = w3 >= 2;
  a = keep0 ? 0 : (keep1 ? 1 : 2);
  b = keep3 ? 3 : (keep2 ? 2 : 1);
}

// One bf16 group held in two dwords (e0 | e1 << 16, e2 | e3 << 16) -> packed kept pair, nibble.
__device__ __forceinline__ uint32_t select_bf16_group(uint32_t lo, uint32_t hi, uint32_t& nibble) {
  const uint32_t e0 = lo & 0xFFFFu, e1 = lo >> 16, e2 = hi & 0xFFFFu, e3 = hi >> 16;
  int a, b;
  bool k0, k1, k2, k3;
  top2_of_4(e0 & 0x7FFFu, e1 & 0x7FFFu, e2 & 0x7FFFu, e3 & 0x7FFFu, a, b, k0, k1, k2, k3);
  const uint32_t va = k0 ? e0 : (k1 ? e1 : e2);
  const uint32_t vb = k3 ? e3 : (k2 ? e2 : e1);
  nibble = (uint32_t)(a | (b << 2));
  return va | (vb << 16);
}

__global__ __launch_bounds__(kPackThreads) void prune24_pack_bf16_kernel(const u32x4_t* __restrict__ R,
                                                                        u32x2_t* __restrict__ values,
                                                                        uint32_t* __restrict__ meta,
                                                                        int64_t n_chunks) {
  const int64_t base = (int64_t)blockIdx.x * (kPackThreads * kPackIter) + threadIdx.x;
  u32x4_t x[kPackIter];
#pragma unroll
  for (int it = 0; it < kPackIter; ++it) {
    const int64_t c = base + (int64_t)it * kPackThreads;
    x[it] = c < n_chunks ? __builtin_nontemporal_load(R + c) : u32x4_t{0, 0, 0, 0};
  }
#pragma unroll
  for (int it = 0; it < kPackIter; ++it) {
    const int64_t c = base + (int64_t)it * kPackThreads;
    uint32_t n0, n1;
    const uint32_t v0 = select_bf16_group(x[it][0], x[it][1], n0);
    const uint32_t v1 = select_bf16_group(x[it][2], x[it][3], n1);
    // chunk c holds groups 2c, 2c+1 -> byte (c % 4) of metadata word c / 4
    uint32_t w = n0 | (n1 << 4);
    w |= (uint32_t)__shfl_down((int)w, 1) << 8;
    w |= (uint32_t)__shfl_down((int)w, 2) << 16;
    if (c < n_chunks) {
      values[c] = u32x2_t{v0, v1};
      if ((threadIdx.x & 3) == 0) meta[c >> 2] = w;
    }
  }
}

__global__ __launch_bounds__(kPackThreads) void prune24_pack_f32_kernel(const u32x4_t* __restrict__ R,
                                                                       u32x2_t* __restrict__ values,
                                                                       uint32_t* __restrict__ meta,
                                                                       int64_t n_chunks) {
  const int64_t base = (int64_t)blockIdx.x * (kPackThreads * kPackIter) + threadIdx.x;
  u32x4_t x[kPackIter];
#pragma unroll
  for (int it = 0; it < kPackIter; ++it) {
    const int64_t c = base + (int64_t)it * kPackThreads;
    x[it] = c < n_chunks ? __builtin_nontemporal_load(R + c) : u32x4_t{0, 0, 0, 0};
  }
#pragma unroll
  for (int it = 0; it < kPackIter; ++it) {
    const int64_t c = base + (int64_t)it * kPackThreads;
    const uint32_t e0 = x[it][0], e1 = x[it][1], e2 = x[it][2], e3 = x[it][3];
    int a, b;
    bool k0, k1, k2, k3;
    top2_of_4(e0 & 0x7FFFFFFFu, e1 & 0x7FFFFFFFu, e2 & 0x7FFFFFFFu, e3 & 0x7FFFFFFFu, a, b, k0, k1, k2, k3);
    const uint32_t va = k0 ? e0 : (k1 ? e1 : e2);
    const uint32_t vb = k3 ? e3 : (k2 ? e2 : e1);
    // chunk c is group c -> nibble (c % 8) of metadata word c / 8
    uint32_t w = (uint32_t)(a | (b << 2));
    w |= (uint32_t)__shfl_down((int)w, 1) << 4;
    w |= (uint32_t)__shfl_down((int)w, 2) << 8;
    w |= (uint32_t)__shfl_down((int)w, 4) << 16;
    if (c < n_chunks) {
      values[c] = u32x2_t{va, vb};
      if ((threadIdx.x & 7) == 0) meta[c >> 3] = w;
    }
  }
}

}  // namespace

hipError_t launch_prune24_pack(const void* R, int64_t n_out, int64_t n_in, bool bf16, void* values,
                               uint32_t* meta, hipStream_t stream) {
  // 16-byte chunks: bf16 -> 8 entries (2 groups), fp32 -> 4 entries (1 group)
  const int64_t n_chunks = n_out * n_in / (bf16 ? 8 : 4);
  const int64_t blocks = ceil_div(n_chunks, (int64_t)kPackThreads * kPackIter);
  if (bf16)
    prune24_pack_bf16_kernel<<<dim3((unsigned)blocks), dim3(kPackThreads), 0, stream>>>(
        (const u32x4_t*)R, (u32x2_t*)values, meta, n_chunks);
  else
    prune24_pack_f32_kernel<<<dim3((unsigned)blocks), dim3(kPackThreads), 0, stream>>>(
        (const u32x4_t*)R, (u32x2_t*)values, meta, n_chunks);
  return hipGetLastError();
}

}  // namespace splr
