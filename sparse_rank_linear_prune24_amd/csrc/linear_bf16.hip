// Y = X S^T + (X V^T) U^T for bfloat16 operands, float32 accumulation and output (LoSparse page,
// §3.2: the sparse product and the low-rank product are evaluated side by side and summed).
//
// The sparse product runs on gfx950's structured-sparse MFMA, v_smfmac_f32_16x16x64_bf16, as
// Y^T tiles = S_tile * X_tile^T: S is the sparse A operand, X^T the dense B operand. Lane layouts:
//   A (S):  lane l -> row l%16, dense columns 16*(l/16) .. +15 (kept values 8*(l/16) .. +7), index
//           operand = the 4 nibbles of those groups in bits [15:0]
//   B (X):  lane l -> token l%16, columns 8*(l/16)+0..7 and 32+8*(l/16)+0..7
//   D:      lane l -> rows (n) 4*(l/16)+0..3, token l%16
// The packed layout stores each 16-row x 64-column tile in exactly this A order, so a wave reads
// its S fragment as 1 KiB of contiguous memory and its metadata as 128 contiguous bytes. X is
// row-major: it is loaded with row-contiguous (coalesced) 16-byte loads and staged in LDS with a
// padded 160-byte row pitch, from which the B fragments are read without bank conflicts.
//
// The rank-r term is folded into the same accumulators with the same instruction (before the main
// loop when r <= 64, so that it overlaps the loop's first loads; block by block after it otherwise):
// dense U is the sum of two 2:4 matrices with fixed patterns (positions 0,1 and 2,3 of every group
// of four ranks), so acc += U_tile T_tile^T is two structured-sparse MFMAs per 64 ranks with
// constant index operands. T (float32) enters as a bfloat16 high part plus a bfloat16 correction.
// Y is stored once.
//
// Kernels:
//   prefill -- workgroup tile 16*NI*4 rows x 16*NJ tokens, 4 waves, each owning 16*NI rows and all
//              tokens, so every S fragment is used by one wave and goes global -> registers; X is
//              shared through a two-slot LDS ring; P K steps of loads in flight; one barrier per
//              K step; workgroups remapped so the tiles that one XCD (own L2) runs share X and S.
//   decode  -- few tokens: HBM-bound on S. A workgroup owns 16 rows; its 4 waves take interleaved
//              64-column K steps, stream S straight into registers and X through a private LDS
//              slot each, and combine their partial accumulators through LDS in a fixed order.
#include <type_traits>
#include <utility>

#include "common.hpp"
#include "kernels.hpp"

namespace splr {
namespace {

// LDS row pitch of staged X in 16-byte units (128 bytes + 32 pad). With this pitch the B-fragment
// reads (16 rows x one 16-byte chunk per quarter wave) run at the full ds_read_b128 rate on gfx950;
// a 16-byte pad leaves them 2-way bank conflicted.
constexpr int kXPitchU4 = 10;
// ranks (in blocks of 64) whose T pair the stage-2 kernels build before their main loop; larger r
// builds it block by block after the loop
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

constexpr int gcd_int(int a, int b) { return b == 0 ? a : gcd_int(b, a % b); }

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

// Stages U rows n0 .. n0+ROWS-1, ranks j0 .. j0+63 in LDS (X row pitch, bytes 16c .. 16c+15 of a row
// = ranks j0 + 8c .. +7) with row-contiguous loads (8 rows x 128 bytes per wave load); rows past
// n_out and ranks >= r are zero. issue() / finish() as for the T pair.
template <int ROWS, int NT>
struct UStager {
  static constexpr int kChunks = ROWS * 8;
  static constexpr int kIters = (kChunks + NT - 1) / NT;
  u32x4_t v[kIters];
  bool ok[kIters];
  int tid;
  __device__ __forceinline__ void issue(const uint16_t* __restrict__ U, int n_out, int r, int n0, int j0, int t) {
    tid = t;
#pragma unroll
    for (int it = 0; it < kIters; ++it) {
      const int c = tid + it * NT;
      const int row = c >> 3, j = j0 + 8 * (c & 7);
      ok[it] = c < kChunks && n0 + row < n_out && j < r;
      v[it] = *(const u32x4_t*)(U + (size_t)min(n0 + row, n_out - 1) * r + (j < r ? j : 0));
    }
  }
  __device__ __forceinline__ void finish(u32x4_t* dst) {
#pragma unroll
    for (int it = 0; it < kIters; ++it) {
      const int c = tid + it * NT;
      if (c < kChunks) dst[(c >> 3) * kXPitchU4 + (c & 7)] = ok[it] ? v[it] : u32x4_t{0, 0, 0, 0};
    }
  }
};

// acc[i][j] (rows n = nrow0 + 16 i + ..., tokens = LDS rows 16 j + ...) += U[n][j0 .. j0+63] .
// T[token][j0 .. j0+63], with T as the LDS pair built by build_t_pair. Dense U is the sum of two 2:4
// operands with fixed patterns (ranks 0,1 and 2,3 of each group of four), and T = hi + lo, so each
// fragment takes four structured-sparse MFMAs.
// U comes from `ulds` when given (rows of the block staged by UStager, this wave's first row at
// `urow0`), else from global memory.
template <int NI, int NJ>
__device__ __forceinline__ void lowrank_block(f32x4_t (&acc)[NI][NJ], const uint16_t* __restrict__ U,
                                              const u32x4_t* hi, const u32x4_t* lo, int n_out, int r, int j0,
                                              int nrow0, int lane, const u32x4_t* ulds = nullptr, int urow0 = 0) {
  const int sub = lane & 15, quad = lane >> 4;
  const u32x4_t zero = {0, 0, 0, 0};
  // A operand: U[n][j0 + 16q .. +15] split into the (0,1) and (2,3) positions of each group
  const int ju = j0 + 16 * quad;
  u32x4_t ud[NI][2];
#pragma unroll
  for (int i = 0; i < NI; ++i) {
    if (ulds) {
      const int row = (urow0 + 16 * i + sub) * kXPitchU4 + 2 * quad;
      ud[i][0] = ulds[row];
      ud[i][1] = ulds[row + 1];
    } else {
      const int n = nrow0 + 16 * i + sub;
      const bool ok = n < n_out && ju < r;
      const uint16_t* p = U + (size_t)(ok ? n : 0) * r + (ok ? ju : 0);
      ud[i][0] = ok ? *(const u32x4_t*)p : zero;
      ud[i][1] = ok ? *(const u32x4_t*)(p + 8) : zero;
    }
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

// Store acc[i][j] like store_tile, but through a per-wave LDS buffer `buf` (64 tokens x 64 rows of
// float32, row pitch kYPitch floats) so that the global stores are row-contiguous: the wave writes
// its accumulators for 64 tokens into the buffer (16-byte writes, a 16-lane phase on distinct
// banks), reads them back as 256-byte segments of token rows and stores four token rows per
// instruction, which runs faster than storing the fragment order (16 token rows x 64 bytes per
// instruction). All addressing is derived here from the lane and the tile origin.
constexpr int kYPitch = 68;
constexpr int kRowsEpilogueMaxTiles = 256;  // one workgroup per CU of MI355X
constexpr double kNonTemporalYBytes = 192.0 * (1 << 20);
template <int NI, int NJ>
__device__ __forceinline__ void store_tile_rows(const f32x4_t (&acc)[NI][NJ], float* buf, void* __restrict__ Yv,
                                                int y_bf16, int M, int n_out, int nrow0, int mrow0) {
  static_assert(NI == 4 && NJ % 4 == 0, "a wave owns 64 rows; tokens go through the buffer 64 at a time");
  const int lane = threadIdx.x & 63;
  const int wr = (lane & 15) * kYPitch + 4 * (lane >> 4);   // write: token lane%16, rows 4*(lane/16)
  const int rd = (lane >> 4) * kYPitch + 4 * (lane & 15);   // read: token lane/16, rows 4*(lane%16)
  const int n = nrow0 + 4 * (lane & 15);
  const bool vec_ok = (n_out & 3) == 0 && n + 3 < n_out;
#pragma unroll
  for (int h = 0; h < NJ / 4; ++h) {
#pragma unroll
    for (int jj = 0; jj < 4; ++jj)
#pragma unroll
      for (int i = 0; i < NI; ++i) *(f32x4_t*)(buf + wr + 16 * jj * kYPitch + 16 * i) = acc[i][4 * h + jj];
#pragma unroll
    for (int t = 0; t < 16; ++t) {
      const f32x4_t v = *(const f32x4_t*)(buf + rd + 4 * t * kYPitch);
      const int m = mrow0 + 64 * h + 4 * t + (lane >> 4);
      if (m >= M) continue;
      if (y_bf16) {
        uint16_t* yrow = (uint16_t*)Yv + (size_t)m * n_out;
        uint32_t hb[4];
#pragma unroll
        for (int e = 0; e < 4; ++e) hb[e] = float_to_bf16_bits(v[e]);
        if (vec_ok) {
          *(u32x2_t*)(yrow + n) = u32x2_t{hb[0] | (hb[1] << 16), hb[2] | (hb[3] << 16)};
        } else {
#pragma unroll
          for (int e = 0; e < 4; ++e)
            if (n + e < n_out) yrow[n + e] = (uint16_t)hb[e];
        }
      } else {
        float* yrow = (float*)Yv + (size_t)m * n_out;
        if (vec_ok) {
          *(f32x4_t*)(yrow + n) = v;
        } else {
#pragma unroll
          for (int e = 0; e < 4; ++e)
            if (n + e < n_out) yrow[n + e] = v[e];
        }
      }
    }
  }
}

// ----------------------------------------------------------------------------------- prefill

// EPI: how Y is stored -- kEpiDirect (fragment order), kEpiRows (row-contiguous through LDS),
// kEpiDirectNT (fragment order, non-temporal)
constexpr int kEpiDirect = 0, kEpiRows = 1, kEpiDirectNT = 2;
template <int NI, int NJ, int P, int PX, int EPI>
__global__ __launch_bounds__(256) void linear_prefill_kernel(
    const uint16_t* __restrict__ X, const u32x4_t* __restrict__ values, const uint32_t* __restrict__ meta,
    const uint16_t* __restrict__ U, const float* __restrict__ Tpart, int slices, void* __restrict__ Y, int y_bf16,
    int M, int K, int n_out, int r, int tiles_n, int tiles_m, int tiles_per_xcd, int group_m) {
  constexpr int WAVES = 4;
  constexpr int BN = 16 * NI * WAVES;
  constexpr int BM = 16 * NJ;
  constexpr int kXLoads = BM / (8 * WAVES);  // X load instructions per wave per step (8 tokens each)
  static_assert(BM % (8 * WAVES) == 0, "X stage must split evenly over the waves");
  static_assert(P >= 2 && PX >= 2 && P % 2 == 0 && PX % 2 == 0, "prefetch distances must be even");
  constexpr int kUnroll = P * PX / gcd_int(P, PX);  // unroll factor: every register slot index is a constant
  // the two LDS slots are separate objects, so the compiler may move reads of one past writes of
  // the other
  __shared__ u32x4_t xs0[BM * kXPitchU4];
  __shared__ u32x4_t xs1[BM * kXPitchU4];
  // T's bfloat16 pair for this tile's tokens (hi, lo planes per 64 ranks), built before the main
  // loop when r <= 64 * kPreRankBlocks (registers are free then and the loads overlap the start),
  // and this tile's U rows when r <= 64
  __shared__ u32x4_t tpair[2 * kPreRankBlocks][BM * kXPitchU4];
  __shared__ u32x4_t ulds[BN * kXPitchU4];

  // XCD-aware tile order: workgroup b runs on XCD b % 8; each XCD gets a contiguous range of
  // logical tiles, walked in groups of `group_m` token tiles, so its tiles share X and S rows.
  const int b = blockIdx.x;
  const int logical = (b & 7) * tiles_per_xcd + (b >> 3);
  if (logical >= tiles_n * tiles_m) return;
  const int per_group = group_m * tiles_n;
  const int g = logical / per_group;
  const int first_m = g * group_m;
  const int gsize = min(group_m, tiles_m - first_m);
  const int in_group = logical - g * per_group;
  const int m0 = (first_m + in_group % gsize) * BM;
  const int n0 = (in_group / gsize) * BN;

  // the wave index is uniform across the wave; readfirstlane lets the compiler see that (scalar
  // loop control instead of exec-mask loops)
  const int lane = threadIdx.x & 63, wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int sub = lane & 15, quad = lane >> 4;
  const int TK = (K + 63) / 64, TR = (n_out + 15) / 16;
  const int nk_pad = (TK + kUnroll - 1) / kUnroll * kUnroll;

  // S fragments of this wave: tile rows (clamped; rows past n_out are zero padding or unused)
  const u32x4_t* vsrc[NI];
  const uint16_t* msrc[NI];  // this lane's 16 index bits: half (quad & 1) of its metadata word
#pragma unroll
  for (int i = 0; i < NI; ++i) {
    const int tr = min(n0 / 16 + wave * NI + i, TR - 1);
    vsrc[i] = values + (size_t)tr * TK * 64 + lane;
    msrc[i] = (const uint16_t*)(meta + (size_t)tr * TK * 32 + sub + 16 * (quad >> 1)) + (quad & 1);
  }
  // X rows this lane loads: token m0 + wave*BM/4 + 8 t + lane/8, 16-byte chunk lane%8 of a step
  const int xchunk = lane & 7;
  const uint16_t* xsrc[kXLoads];
  int xdst[kXLoads];
#pragma unroll
  for (int t = 0; t < kXLoads; ++t) {
    const int tloc = wave * (BM / WAVES) + 8 * t + (lane >> 3);
    xsrc[t] = X + (size_t)min(m0 + tloc, M - 1) * K + 8 * xchunk;
    xdst[t] = tloc * kXPitchU4 + xchunk;
  }

  u32x4_t xr[PX][kXLoads];  // X register ring: X of step kc is loaded PX steps before it goes to LDS
  u32x4_t sa[P][NI];
  uint32_t sw[P][NI];  // index operands, zero-extended 16-bit loads
  bf16x16_t bx[2][NJ];
  auto load_x = [&](int kc, u32x4_t (&v)[kXLoads]) {
    int col = min(kc, TK - 1) * 64;
    if (col + 8 * xchunk >= K) col -= 32;  // half tail step: re-read valid columns (S is zero there)
#pragma unroll
    for (int t = 0; t < kXLoads; ++t) v[t] = *(const u32x4_t*)(xsrc[t] + col);
  };
  auto load_s = [&](int kc, u32x4_t (&va)[NI], uint32_t (&wa)[NI]) {
    const int kk = min(kc, TK - 1);
#pragma unroll
    for (int i = 0; i < NI; ++i) {
      va[i] = vsrc[i][(size_t)kk * 64];
      wa[i] = msrc[i][(size_t)kk * 64];
    }
  };
  auto store_x = [&](u32x4_t* slot, const u32x4_t (&v)[kXLoads]) {
#pragma unroll
    for (int t = 0; t < kXLoads; ++t) slot[xdst[t]] = v[t];
  };
  auto read_b = [&](const u32x4_t* slot, bf16x16_t (&b)[NJ]) {
#pragma unroll
    for (int j = 0; j < NJ; ++j) {
      const int row = (16 * j + sub) * kXPitchU4;
      b[j] = cat16(as_bf16x8(slot[row + quad]), as_bf16x8(slot[row + 4 + quad]));
    }
  };
  f32x4_t acc[NI][NJ];
#pragma unroll
  for (int i = 0; i < NI; ++i)
#pragma unroll
    for (int j = 0; j < NJ; ++j) acc[i][j] = f32x4_t{0, 0, 0, 0};

  // Software pipeline, one barrier per K step. At step kc (S register slot kc % P, X register slot
  // (kc+2) % PX, LDS slot and B register parity b = kc % 2): the B fragments of step kc are already
  // in registers bx[b], X of step kc+1 is in LDS slot b^1, X of step kc+2 is in registers. The step
  // writes X of step kc+2 into LDS slot b (whose reads, of step kc, completed before the previous
  // barrier), reads the B fragments of step kc+1 into bx[b^1] while its MFMAs run, refills the S
  // slot of step kc-1 with step kc+P-1 and the X register slot with step kc+2+PX, and ends with the
  // barrier. The instruction order inside a step is pinned (LDS writes, then LDS reads and global
  // loads each paired with an MFMA), and no instruction crosses a step boundary. Padding steps
  // (kc >= TK) zero the S operand.
  auto step = [&](int kc, auto uu, auto masked) {
    constexpr int u = decltype(uu)::value;
    constexpr int d = u % P, b = u & 1, dprev = (u + P - 1) % P, xq = (u + 2) % PX;
    store_x(b ? xs1 : xs0, xr[xq]);
    read_b(b ? xs0 : xs1, bx[b ^ 1]);
    const uint32_t keep = (!decltype(masked)::value || kc < TK) ? ~0u : 0u;
    bf16x8_t a[NI];
    int idx[NI];
#pragma unroll
    for (int i = 0; i < NI; ++i) {
      a[i] = decltype(masked)::value ? as_bf16x8(sa[d][i] & keep) : as_bf16x8(sa[d][i]);
      idx[i] = (int)(sw[d][i] & keep);
    }
#pragma unroll
    for (int j = 0; j < NJ; ++j)
#pragma unroll
      for (int i = 0; i < NI; ++i) acc[i][j] = smfmac16x16x64(a[i], bx[b][j], acc[i][j], idx[i]);
    load_s(kc + P - 1, sa[dprev], sw[dprev]);
    load_x(kc + 2 + PX, xr[xq]);
    // pinned order: the LDS writes, LDS reads and global loads are spread evenly over the MFMAs,
    // one after each MFMA, in kXLoads rounds of (1 LDS write, 2*NJ/kXLoads LDS reads, the loads'
    // share), so that no queue fills and blocks the in-order issue of the MFMAs
    constexpr int kReads = 2 * NJ, kLoads = 2 * NI + kXLoads, kMfma = NI * NJ, kRounds = kXLoads;
    static_assert(kReads % kRounds == 0 && kLoads % kRounds == 0, "even spread");
    static_assert(kRounds * (1 + kReads / kRounds + kLoads / kRounds) <= kMfma, "one MFMA per memory op");
#pragma unroll
    for (int q = 0; q < kRounds; ++q) {
      __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
      __builtin_amdgcn_sched_group_barrier(0x200, 1, 0);
#pragma unroll
      for (int t = 0; t < kReads / kRounds; ++t) {
        __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
        __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);
      }
#pragma unroll
      for (int t = 0; t < kLoads / kRounds; ++t) {
        __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
        __builtin_amdgcn_sched_group_barrier(0x020, 1, 0);
      }
    }
    __builtin_amdgcn_sched_group_barrier(0x008, kMfma - kRounds * (1 + (kReads + kLoads) / kRounds), 0);
    lds_barrier();
    __builtin_amdgcn_sched_barrier(0);
  };

  // rank-r operands staged before the main loop: loads issued here, finished after the loop's
  // prologue has issued its own loads (published by the prologue's barriers)
  const bool t_pre = r <= 64 * kPreRankBlocks, u_pre = r <= 64;
  TPairBuilder<BM, 64 * WAVES, 2> tb[kPreRankBlocks];
  UStager<BN, 64 * WAVES> us;
  if (t_pre) {
#pragma unroll
    for (int b = 0; b < kPreRankBlocks; ++b)
      if (64 * b < r) {
        tb[b].init(Tpart, slices, M, r, m0, 64 * b, threadIdx.x);
        tb[b].issue(0);
      }
  }
  if (u_pre && r > 0) us.issue(U, n_out, r, n0, 0, threadIdx.x);

  // Prologue: virtual steps v = -VS .. -1 issue exactly what a step would (X of step v+2 into LDS,
  // S of step v+P-1, X of step v+2+PX), so the loop is entered with the loads in flight in the same
  // order as in the steady state and the wait counts the compiler derives need no extra waits.
  constexpr int VS = (P - 1 > PX + 2) ? P - 1 : PX + 2;
  static_for<VS>([&](auto ii) {
    constexpr int v = decltype(ii)::value - VS;
    if constexpr (v >= -2) store_x(((v + 2) & 1) ? xs1 : xs0, xr[(v + 2 + PX) % PX]);
    if constexpr (v + P - 1 >= 0) load_s(v + P - 1, sa[(v + P - 1) % P], sw[(v + P - 1) % P]);
    if constexpr (v + 2 + PX >= 0) load_x(v + 2 + PX, xr[(v + 2 + PX) % PX]);
  });
  if (t_pre) {
#pragma unroll
    for (int b = 0; b < kPreRankBlocks; ++b)
      if (64 * b < r) tb[b].finish(tpair[2 * b], tpair[2 * b + 1]);
  }
  if (u_pre && r > 0) us.finish(ulds);
  lds_barrier();
  const int nrow0 = n0 + wave * 16 * NI;
  // rank-r term first when T's pair is already in LDS: its MFMAs run while the main loop's first
  // loads are in flight (the accumulators start from U T^T instead of zero)
  if (t_pre) {
#pragma unroll
    for (int b = 0; b < kPreRankBlocks; ++b)
      if (64 * b < r)
        lowrank_block<NI, NJ>(acc, U, tpair[2 * b], tpair[2 * b + 1], n_out, r, 64 * b, nrow0, lane,
                              u_pre ? ulds : nullptr, wave * 16 * NI);
  }
  __builtin_amdgcn_sched_barrier(0);
  read_b(xs0, bx[0]);
  lds_barrier();  // every wave's reads of slot 0 are done before step 0 overwrites it
  __builtin_amdgcn_sched_barrier(0);
  const int nk_full = TK / kUnroll * kUnroll;  // steps that need no masking
  for (int kc0 = 0; kc0 < nk_full; kc0 += kUnroll)
    static_for<kUnroll>([&](auto u) { step(kc0 + decltype(u)::value, u, std::false_type{}); });
  for (int kc0 = nk_full; kc0 < nk_pad; kc0 += kUnroll)
    static_for<kUnroll>([&](auto u) { step(kc0 + decltype(u)::value, u, std::true_type{}); });

  // larger r: the rank-r term, 64 ranks at a time, after the loop; the workgroup builds T's pair
  // block by block in the now free X slots (the last step's barrier has retired every read of them)
  // and stages the block's U rows in the U slot (unused before the loop when r > 64), the loads of
  // both in flight together
  if (!t_pre) {
    for (int j0 = 0; j0 < r; j0 += 64) {
      TPairBuilder<BM, 64 * WAVES, 2> tbp;
      UStager<BN, 64 * WAVES> usp;
      tbp.init(Tpart, slices, M, r, m0, j0, threadIdx.x);
      tbp.issue(0);
      usp.issue(U, n_out, r, n0, j0, threadIdx.x);
      __builtin_amdgcn_sched_barrier(0);
      tbp.finish(xs0, xs1);
      usp.finish(ulds);
      lds_barrier();
      lowrank_block<NI, NJ>(acc, U, xs0, xs1, n_out, r, j0, nrow0, lane, ulds, wave * 16 * NI);
      lds_barrier();
    }
  }
  if constexpr (EPI == kEpiRows) {
    // Y leaves through LDS (every slot is free now: the last barrier above retired all reads of
    // them); waves 0, 1 use the T pair slot, waves 2, 3 the U slot
    static_assert(2 * 64 * kYPitch * 4 <= (int)sizeof(tpair) && 2 * 64 * kYPitch * 4 <= (int)sizeof(ulds),
                  "epilogue buffers fit");
    float* ybuf = (wave < 2 ? (float*)&tpair[0][0] : (float*)&ulds[0]) + (wave & 1) * 64 * kYPitch;
    store_tile_rows<NI, NJ>(acc, ybuf, Y, y_bf16, M, n_out, nrow0, m0);
  } else {
    store_tile<NI, NJ, EPI == kEpiDirectNT>(acc, Y, y_bf16, M, n_out, nrow0, m0, lane);
  }
}

// ----------------------------------------------------------------------------------- decode

template <int MB, int P, int WAVES>
__global__ __launch_bounds__(64 * WAVES) void linear_decode_kernel(
    const uint16_t* __restrict__ X, const u32x4_t* __restrict__ values, const uint32_t* __restrict__ meta,
    const uint16_t* __restrict__ U, const float* __restrict__ Tpart, int slices, void* __restrict__ Y, int y_bf16, int M, int K,
    int n_out, int r) {
  constexpr int kXLoads = 2 * MB;  // 8 tokens x 128 bytes per load instruction, 16*MB tokens
  __shared__ u32x4_t xs[WAVES][16 * MB * kXPitchU4];
  __shared__ f32x4_t red[(WAVES - 1) * MB * 64];
  __shared__ u32x4_t tpair[2 * kPreRankBlocks][16 * MB * kXPitchU4];  // as in the prefill kernel
  // the wave index is uniform across the wave; readfirstlane lets the compiler see that (scalar
  // loop control instead of exec-mask loops)
  const int lane = threadIdx.x & 63, wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int sub = lane & 15, quad = lane >> 4;
  const int tr = blockIdx.x, m0 = blockIdx.y * 16 * MB;
  const int TK = (K + 63) / 64;

  const u32x4_t* vsrc = values + (size_t)tr * TK * 64 + lane;
  const uint16_t* msrc = (const uint16_t*)(meta + (size_t)tr * TK * 32 + sub + 16 * (quad >> 1)) + (quad & 1);
  const int xchunk = lane & 7;
  const uint16_t* xsrc[kXLoads];
  int xdst[kXLoads];
#pragma unroll
  for (int t = 0; t < kXLoads; ++t) {
    const int tloc = 8 * t + (lane >> 3);
    xsrc[t] = X + (size_t)min(m0 + tloc, M - 1) * K + 8 * xchunk;
    xdst[t] = tloc * kXPitchU4 + xchunk;
  }
  u32x4_t* st = xs[wave];

  f32x4_t acc[1][MB];
#pragma unroll
  for (int j = 0; j < MB; ++j) acc[0][j] = f32x4_t{0, 0, 0, 0};

  // This wave's steps are kc = wave, wave + 4, ...; a ring of P steps of loads stays in flight:
  // slot u holds step s0 + u and is refilled with step s0 + u + P as soon as it has been consumed.
  // Branch-free: steps past the wave's last one load a clamped step and contribute through a
  // zeroed S operand.
  const int my_steps = (TK - wave + WAVES - 1) / WAVES;
  const int n_pad = max(1, (my_steps + P - 1) / P) * P;  // at least the final round (a wave may have no steps)
  u32x4_t sa[P], xr[P][kXLoads];
  uint32_t sw[P];
  auto load = [&](int s, u32x4_t& va, uint32_t& wa, u32x4_t (&xv)[kXLoads]) {
    const int kc = min(wave + s * WAVES, TK - 1);
    va = vsrc[(size_t)kc * 64];
    wa = msrc[(size_t)kc * 64];
    int col = kc * 64;
    if (col + 8 * xchunk >= K) col -= 32;  // half tail step: re-read valid columns (S is zero there)
#pragma unroll
    for (int t = 0; t < kXLoads; ++t) xv[t] = *(const u32x4_t*)(xsrc[t] + col);
  };

  // T's pair: its loads go out first, the ring's next, and the pair is written to LDS while the
  // ring's loads are in flight (published by the barrier after the loop)
  const bool t_pre = r <= 64 * kPreRankBlocks;
  TPairBuilder<16 * MB, 64 * WAVES> tb;
  if (t_pre && r > 0) {
    tb.init(Tpart, slices, M, r, m0, 0, threadIdx.x);
    tb.issue(0);
  }
  static_for<P>([&](auto uu) {  // issued in slot order (fenced), as the loop refills them
    constexpr int u = decltype(uu)::value;
    load(u, sa[u], sw[u], xr[u]);
    asm volatile("" ::: "memory");
  });
  if (t_pre && r > 0) tb.finish(tpair[0], tpair[1]);

  auto step = [&](int s, auto uu, auto refill) {
    constexpr int u = decltype(uu)::value;
#pragma unroll
    for (int t = 0; t < kXLoads; ++t) st[xdst[t]] = xr[u][t];
    const uint32_t keep = s < my_steps ? ~0u : 0u;  // wave-uniform
    const bf16x8_t a = as_bf16x8(sa[u] & keep);
    const int idx = (int)(sw[u] & keep);
    if constexpr (decltype(refill)::value) load(s + P, sa[u], sw[u], xr[u]);
    // compiler-only fence: the refill stays in this step (not rotated into the next iteration,
    // which would shorten the prefetch distance of this slot)
    asm volatile("" ::: "memory");
#pragma unroll
    for (int j = 0; j < MB; ++j) {
      const int row = (16 * j + sub) * kXPitchU4;
      const bf16x16_t bx = cat16(as_bf16x8(st[row + quad]), as_bf16x8(st[row + 4 + quad]));
      acc[0][j] = smfmac16x16x64(a, bx, acc[0][j], idx);
    }
  };
  // every round but the last refills its slots; the last round loads nothing past the end
  for (int s0 = 0; s0 + P < n_pad; s0 += P)
    static_for<P>([&](auto uu) { step(s0 + decltype(uu)::value, uu, std::true_type{}); });
  static_for<P>([&](auto uu) { step(n_pad - P + decltype(uu)::value, uu, std::false_type{}); });

  // fixed-order combination of the waves' partial sums (into wave 0)
  if (wave > 0) {
#pragma unroll
    for (int j = 0; j < MB; ++j) red[((wave - 1) * MB + j) * 64 + lane] = acc[0][j];
  }
  __syncthreads();
  if (wave == 0) {
#pragma unroll
    for (int w = 1; w < WAVES; ++w)
#pragma unroll
      for (int j = 0; j < MB; ++j) acc[0][j] += red[((w - 1) * MB + j) * 64 + lane];
  }
  // rank-r term, 64 ranks at a time: wave 0 adds U T^T, with T's pair from before the loop or, for
  // larger r, built block by block by all waves
  if (t_pre) {
    if (wave == 0) {
#pragma unroll
      for (int b = 0; b < kPreRankBlocks; ++b)
        if (64 * b < r) lowrank_block<1, MB>(acc, U, tpair[2 * b], tpair[2 * b + 1], n_out, r, 64 * b, tr * 16, lane);
    }
  } else {
    for (int j0 = 0; j0 < r; j0 += 64) {
      build_t_pair<16 * MB, 64 * WAVES>(Tpart, slices, M, r, m0, j0, xs[0], xs[1], threadIdx.x);
      lds_barrier();
      if (wave == 0) lowrank_block<1, MB>(acc, U, xs[0], xs[1], n_out, r, j0, tr * 16, lane);
      lds_barrier();
    }
  }
  if (wave == 0) store_tile<1, MB>(acc, Y, y_bf16, M, n_out, tr * 16, m0, lane);
}

template <int MB>
hipError_t launch_decode(const void* X, int64_t M, int64_t n_in, const void* values, const uint32_t* meta,
                         int64_t n_out, const void* U, int64_t r, const float* Tpart, int slices, void* Y,
                         int y_bf16, hipStream_t stream) {
  constexpr int P = MB == 1 ? 8 : 4, W = 4;
  dim3 grid((unsigned)ceil_div(n_out, 16), (unsigned)ceil_div(M, 16 * MB));
  linear_decode_kernel<MB, P, W><<<grid, dim3(64 * W), 0, stream>>>(
      (const uint16_t*)X, (const u32x4_t*)values, meta, (const uint16_t*)U, Tpart, slices, Y, y_bf16, (int)M,
      (int)n_in, (int)n_out, (int)r);
  return hipGetLastError();
}

}  // namespace

hipError_t launch_linear_bf16(const void* X, int64_t M, int64_t n_in, const void* values, const uint32_t* meta,
                              int64_t n_out, const void* U, int64_t r, const float* Tpart, int slices, void* Y,
                              bool y_bf16, hipStream_t stream) {
  const int yb = y_bf16 ? 1 : 0;
  if (M <= 16) return launch_decode<1>(X, M, n_in, values, meta, n_out, U, r, Tpart, slices, Y, yb, stream);
  if (M <= 32) return launch_decode<2>(X, M, n_in, values, meta, n_out, U, r, Tpart, slices, Y, yb, stream);
  if (M <= kDecodeMaxTokens)
    return launch_decode<4>(X, M, n_in, values, meta, n_out, U, r, Tpart, slices, Y, yb, stream);

  constexpr int NI = 4, NJ = 8, P = 4, PX = 2;
  constexpr int BN = 16 * NI * 4, BM = 16 * NJ;
  const int tiles_n = (int)ceil_div(n_out, BN), tiles_m = (int)ceil_div(M, BM);
  const int n_tiles = tiles_n * tiles_m;
  const int per_xcd = (int)ceil_div(n_tiles, 8);
  const int group_m = 4;
  // When every tile runs at once (one workgroup per CU), the Y stores of all tiles come at the end
  // together and are exposed: the row-contiguous epilogue stores them faster. With several tiles per
  // CU the stores overlap the next tile's loop, and with r > 64 the extra registers of that
  // epilogue cost spills in the rank-r blocks after the loop: there the direct epilogue is faster.
  // A Y larger than three quarters of the 256 MB Infinity Cache is stored non-temporally: kept in the
  // cache it evicts the S and X rows that later tile groups re-read (measured: -6 to -11 % on
  // 4096/8192 tokens x 14336 outputs; +5 % slower on 8192 x 4096, 134 MB, so the threshold sits
  // between).
  const bool y_nt = (double)M * n_out * (y_bf16 ? 2 : 4) > kNonTemporalYBytes;
  const dim3 grid((unsigned)(8 * per_xcd)), block(256);
  if (n_tiles <= kRowsEpilogueMaxTiles && r <= 64)
    linear_prefill_kernel<NI, NJ, P, PX, kEpiRows><<<grid, block, 0, stream>>>(
        (const uint16_t*)X, (const u32x4_t*)values, meta, (const uint16_t*)U, Tpart, slices, Y, yb, (int)M,
        (int)n_in, (int)n_out, (int)r, tiles_n, tiles_m, per_xcd, group_m);
  else if (y_nt)
    linear_prefill_kernel<NI, NJ, P, PX, kEpiDirectNT><<<grid, block, 0, stream>>>(
        (const uint16_t*)X, (const u32x4_t*)values, meta, (const uint16_t*)U, Tpart, slices, Y, yb, (int)M,
        (int)n_in, (int)n_out, (int)r, tiles_n, tiles_m, per_xcd, group_m);
  else
    linear_prefill_kernel<NI, NJ, P, PX, kEpiDirect><<<grid, block, 0, stream>>>(
        (const uint16_t*)X, (const u32x4_t*)values, meta, (const uint16_t*)U, Tpart, slices, Y, yb, (int)M,
        (int)n_in, (int)n_out, (int)r, tiles_n, tiles_m, per_xcd, group_m);
  return hipGetLastError();
}

}  // namespace splr
