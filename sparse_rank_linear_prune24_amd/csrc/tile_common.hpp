// Device helpers shared by the layer-product kernels (prefill in linear_bf16.hip, decode in
// decode.hip): the LDS barrier that keeps register prefetches in flight, compile-time loops, the
// T pair builder of the rank-r term, the rank-r MFMA block and the Y store.
#pragma once

#include <type_traits>
#include <utility>

#include "common.hpp"

namespace splr {
namespace {

// LDS row pitch of staged X in 16-byte units (128 bytes + 32 pad). With this pitch the B-fragment
// reads (16 rows x one 16-byte chunk per quarter wave) run at the full ds_read_b128 rate on gfx950;
// a 16-byte pad leaves them 2-way bank conflicted.
constexpr int kXPitchU4 = 10;
// ranks (in blocks of 64) whose T pair the decode kernel builds before its K loop; larger r builds
// it block by block after the loop
constexpr int kPreRankBlocks = 1;


// LDS writes of this wave complete, then workgroup barrier. One asm statement with a memory
// clobber: the compiler moves no LDS access across it, and (unlike __syncthreads(), whose fence
// drains every outstanding global load) it leaves the register prefetches in flight.
// The builtin wait after it is free at run time; it tells the compiler's wait-count tracking that no
// LDS access is outstanding, so it adds no conservative waits after the barrier.
__device__ __forceinline__ void lds_barrier() {
  asm volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory");
  __builtin_amdgcn_s_waitcnt(0xc07f);  // lgkmcnt(0); vmcnt and expcnt at their maximum (no wait)
}


// f(std::integral_constant<int, 0>{}) ... f(std::integral_constant<int, N-1>{}), in order
template <typename F, int... I>
__device__ __forceinline__ void static_for_impl(F&& f, std::integer_sequence<int, I...>) {
  (f(std::integral_constant<int, I>{}), ...);
}
template <int N, typename F>
__device__ __forceinline__ void static_for(F&& f) {
  static_for_impl(f, std::make_integer_sequence<int, N>{});
}

// ----------------------------------------------------------------------------------- epilogue

// Builds T rows m0 .. m0+ROWS-1, ranks j0 .. j0+63, as the bfloat16 pair (hi = RNE(T), lo =
// RNE(T - hi)) in two LDS planes with the X row pitch (bytes 16c .. 16c+15 of a row hold ranks
// j0 + 8c .. +7). T is the sum of `slices` float32 partials [slices][M][r], added in slice order.
// All NT threads take part; thread t handles 4 consecutive ranks of a row per item, so one wave
// load covers 4 rows x 256 contiguous bytes. Ranks >= r give zeros; rows past M repeat row M-1
// (never stored). issue() starts the loads of a round of slices, finish() adds them (and any
// further rounds) and writes the LDS planes, so the first round can overlap other work.
template <int ROWS, int NT, int G = 0>
struct TPairBuilder {
  static constexpr int kQuads = ROWS * 16;  // 4 ranks each
  static constexpr int kIters = (kQuads + NT - 1) / NT;
  // slices per round: G, else as many as keep <= 16 loads in flight per thread
  static constexpr int kGroup = G > 0 ? G : (kIters >= 8 ? 1 : 16 / kIters);
  const float* src[kIters];
  bool ok[kIters];
  f32x4_t sum[kIters];
  f32x4_t v[kIters][kGroup];
  size_t stride;
  int slices, tid;

  __device__ __forceinline__ void init(const float* __restrict__ Tpart, int n_slices, int M, int r, int m0, int j0,
                                       int t) {
    stride = (size_t)M * r;
    slices = n_slices;
    tid = t;
#pragma unroll
    for (int it = 0; it < kIters; ++it) {
      const int q = tid + it * NT;
      const int row = q >> 4, j = j0 + 4 * (q & 15);
      ok[it] = q < kQuads && j < r;
      src[it] = Tpart + (size_t)min(m0 + row, M - 1) * r + (ok[it] ? j : 0);
      sum[it] = f32x4_t{0, 0, 0, 0};
    }
  }
  // loads are unconditional (clamped, valid addresses) and masked when added: no lane branches
  __device__ __forceinline__ void issue(int z0) {
#pragma unroll
    for (int it = 0; it < kIters; ++it)
#pragma unroll
      for (int u = 0; u < kGroup; ++u)
        v[it][u] = *(const f32x4_t*)(src[it] + (size_t)(z0 + u < slices ? z0 + u : 0) * stride);
  }
  __device__ __forceinline__ void accumulate(int z0) {
#pragma unroll
    for (int it = 0; it < kIters; ++it)
#pragma unroll
      for (int u = 0; u < kGroup; ++u) sum[it] += (ok[it] && z0 + u < slices) ? v[it][u] : f32x4_t{0, 0, 0, 0};
  }
  __device__ __forceinline__ void finish(u32x4_t* hi, u32x4_t* lo) {
    accumulate(0);
    for (int z0 = kGroup; z0 < slices; z0 += kGroup) {
      issue(z0);
      // every load of the round is issued before the first use (under register pressure the
      // scheduler would otherwise pair each load with its use and serialise the latencies)
      __builtin_amdgcn_sched_barrier(0);
      accumulate(z0);
    }
#pragma unroll
    for (int it = 0; it < kIters; ++it) {
      const int q = tid + it * NT;
      if (q >= kQuads) continue;
      uint32_t h[4], l[4];
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        h[e] = float_to_bf16_bits(sum[it][e]);
        l[e] = float_to_bf16_bits(sum[it][e] - bf16_bits_to_float(h[e]));
      }
      const int o = (q >> 4) * 2 * kXPitchU4 + (q & 15);  // in 8-byte units
      ((u32x2_t*)hi)[o] = u32x2_t{h[0] | (h[1] << 16), h[2] | (h[3] << 16)};
      ((u32x2_t*)lo)[o] = u32x2_t{l[0] | (l[1] << 16), l[2] | (l[3] << 16)};
    }
  }
};

template <int ROWS, int NT>
__device__ __forceinline__ void build_t_pair(const float* __restrict__ Tpart, int slices, int M, int r, int m0,
                                             int j0, u32x4_t* hi, u32x4_t* lo, int tid) {
  TPairBuilder<ROWS, NT> tb;
  tb.init(Tpart, slices, M, r, m0, j0, tid);
  tb.issue(0);
  __builtin_amdgcn_sched_barrier(0);
  tb.finish(hi, lo);
}

// acc[i][j] (rows n = nrow0 + 16 i + ..., tokens = LDS rows 16 j + ...) += U[n][j0 .. j0+63] .
// T[token][j0 .. j0+63], with T as the LDS pair built by build_t_pair. Dense U is the sum of two 2:4
// operands with fixed patterns (ranks 0,1 and 2,3 of each group of four), and T = hi + lo, so each
// fragment takes four structured-sparse MFMAs.
// U comes from global memory (rows past n_out and ranks >= r read as zero).
template <int NI, int NJ>
__device__ __forceinline__ void lowrank_block(f32x4_t (&acc)[NI][NJ], const uint16_t* __restrict__ U,
                                              const u32x4_t* hi, const u32x4_t* lo, int n_out, int r, int j0,
                                              int nrow0, int lane) {
  const int sub = lane & 15, quad = lane >> 4;
  const u32x4_t zero = {0, 0, 0, 0};
  // A operand: U[n][j0 + 16q .. +15] split into the (0,1) and (2,3) positions of each group
  const int ju = j0 + 16 * quad;
  u32x4_t ud[NI][2];
#pragma unroll
  for (int i = 0; i < NI; ++i) {
    const int n = nrow0 + 16 * i + sub;
    const bool ok = n < n_out && ju < r;
    const uint16_t* p = U + (size_t)(ok ? n : 0) * r + (ok ? ju : 0);
    ud[i][0] = ok ? *(const u32x4_t*)p : zero;
    ud[i][1] = ok ? *(const u32x4_t*)(p + 8) : zero;
  }
  // B operand: T[token][j0 + 8q .. +7] and T[token][j0 + 32 + 8q .. +7]
  bf16x16_t th[NJ], tl[NJ];
#pragma unroll
  for (int j = 0; j < NJ; ++j) {
    const int row = (16 * j + sub) * kXPitchU4;
    th[j] = cat16(as_bf16x8(hi[row + quad]), as_bf16x8(hi[row + 4 + quad]));
    tl[j] = cat16(as_bf16x8(lo[row + quad]), as_bf16x8(lo[row + 4 + quad]));
  }
#pragma unroll
  for (int i = 0; i < NI; ++i) {
    const bf16x8_t u01 = as_bf16x8(u32x4_t{ud[i][0][0], ud[i][0][2], ud[i][1][0], ud[i][1][2]});
    const bf16x8_t u23 = as_bf16x8(u32x4_t{ud[i][0][1], ud[i][0][3], ud[i][1][1], ud[i][1][3]});
#pragma unroll
    for (int j = 0; j < NJ; ++j) {
      acc[i][j] = smfmac16x16x64(u01, th[j], acc[i][j], 0x4444);
      acc[i][j] = smfmac16x16x64(u23, th[j], acc[i][j], 0xEEEE);
      acc[i][j] = smfmac16x16x64(u01, tl[j], acc[i][j], 0x4444);
      acc[i][j] = smfmac16x16x64(u23, tl[j], acc[i][j], 0xEEEE);
    }
  }
}

// Store acc[i][j] (rows n = nrow0 + 16 i + 4*(lane/16) + 0..3, token m = mrow0 + 16 j + lane%16), as
// float32, or (y_bf16) rounded to bfloat16 (to nearest even); NT: non-temporal vector stores.
template <int NI, int NJ, bool NT = false>
__device__ __forceinline__ void store_tile(const f32x4_t (&acc)[NI][NJ], void* __restrict__ Yv, int y_bf16, int M,
                                           int n_out, int nrow0, int mrow0, int lane) {
  const bool vec_ok = (n_out & 3) == 0;
  if (y_bf16) {
#pragma unroll
    for (int j = 0; j < NJ; ++j) {
      const int m = mrow0 + 16 * j + (lane & 15);
      if (m >= M) continue;
      uint16_t* yrow = (uint16_t*)Yv + (size_t)m * n_out;
#pragma unroll
      for (int i = 0; i < NI; ++i) {
        const int n = nrow0 + 16 * i + 4 * (lane >> 4);
        uint32_t h[4];
#pragma unroll
        for (int e = 0; e < 4; ++e) h[e] = float_to_bf16_bits(acc[i][j][e]);
        if (vec_ok && n + 3 < n_out) {
          const u32x2_t w = u32x2_t{h[0] | (h[1] << 16), h[2] | (h[3] << 16)};
          if constexpr (NT) __builtin_nontemporal_store(w, (u32x2_t*)(yrow + n));
          else *(u32x2_t*)(yrow + n) = w;
        } else {
#pragma unroll
          for (int e = 0; e < 4; ++e)
            if (n + e < n_out) yrow[n + e] = (uint16_t)h[e];
        }
      }
    }
    return;
  }
  float* __restrict__ Y = (float*)Yv;
#pragma unroll
  for (int j = 0; j < NJ; ++j) {
    const int m = mrow0 + 16 * j + (lane & 15);
    if (m >= M) continue;
    float* yrow = Y + (size_t)m * n_out;
#pragma unroll
    for (int i = 0; i < NI; ++i) {
      const int n = nrow0 + 16 * i + 4 * (lane >> 4);
      if (vec_ok && n + 3 < n_out) {
        if constexpr (NT) __builtin_nontemporal_store(acc[i][j], (f32x4_t*)(yrow + n));
        else *(f32x4_t*)(yrow + n) = acc[i][j];
      } else {
#pragma unroll
        for (int s = 0; s < 4; ++s)
          if (n + s < n_out) yrow[n + s] = acc[i][j][s];
      }
    }
  }
}

// Y bytes above which the prefill kernels store Y non-temporally (whole token rows through LDS)
constexpr double kNonTemporalYBytes = 96.0 * (1 << 20);

}  // namespace
}  // namespace splr
