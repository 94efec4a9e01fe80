// First stage of the low-rank product, T = X V^T (LoSparse page, §3.2: the input is multiplied by
// the thin factors; in the orientation used here X [M x n_in] times V^T [n_in x r]).
//
// bf16: a workgroup owns 16*TF tokens x 16*RF ranks over one slice of K; its waves take interleaved
// 64-column K steps of the slice, each wave staging its own X and V rows in a private LDS region
// (row-contiguous loads, padded pitch) with several steps of loads in flight, and feed gfx950's
// structured-sparse MFMA: X is the dense B operand; V is the A operand, dense V being the sum of two
// 2:4 matrices with fixed patterns (positions 0,1 and 2,3 of every group of four columns). The
// waves' partial sums are combined through LDS in wave order and each slice writes its float32
// partial sum of T; the second stage adds the slices in slice order (deterministic, no atomics).
// fp32: one wave per output, lanes stride over K, fixed-order butterfly reduction.
#include <algorithm>
#include <type_traits>
#include <utility>

#include "common.hpp"
#include "kernels.hpp"

namespace splr {
namespace {

constexpr int kPitchU4 = 10;  // LDS row pitch in 16-byte units (128 bytes + 32 pad): conflict-free b128 reads

int cdiv(int64_t a, int64_t b) { return (int)((a + b - 1) / b); }

// f(std::integral_constant<int, 0>{}) ... f(std::integral_constant<int, N-1>{}), in order
template <typename F, int... I>
__device__ __forceinline__ void static_for_impl(F&& f, std::integer_sequence<int, I...>) {
  (f(std::integral_constant<int, I>{}), ...);
}
template <int N, typename F>
__device__ __forceinline__ void static_for(F&& f) {
  static_for_impl(f, std::make_integer_sequence<int, N>{});
}

// Grid (token blocks, rank blocks, K slices); slice z covers K steps [z*steps_per_slice, ...) and
// writes the float32 partial sum part[z][m][j].
template <int TF, int RF, int WAVES, int D>
__global__ __launch_bounds__(64 * WAVES) void lowrank_bf16_kernel(const uint16_t* __restrict__ X,
                                                                 const uint16_t* __restrict__ V, int M, int K,
                                                                 int r, int steps_per_slice,
                                                                 float* __restrict__ part) {
  constexpr int kRows = 16 * (TF + RF);  // staged rows per wave: X tokens, then V ranks
  constexpr int kLoads = kRows / 8;      // 8 rows x 128 bytes per load instruction
  __shared__ u32x4_t stage[WAVES][kRows * kPitchU4];
  __shared__ f32x4_t red[(WAVES - 1) * RF * TF * 64];
  // the wave index is uniform across the wave; readfirstlane lets the compiler see that (scalar
  // loop control instead of exec-mask loops)
  const int lane = threadIdx.x & 63, wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int sub = lane & 15, quad = lane >> 4;
  const int m0 = blockIdx.x * 16 * TF, j0 = blockIdx.y * 16 * RF;
  const int TK = (K + 63) / 64;
  const int kb = blockIdx.z * steps_per_slice, ke = min(TK, kb + steps_per_slice);
  const bool half_tail = (K & 63) != 0;  // the last step holds 32 valid columns
  u32x4_t* st = stage[wave];

  // this lane's rows: instruction t covers staged rows 8t .. 8t+7, 16-byte chunk lane % 8 of a step
  // (rank rows are always valid: 16*RF divides r)
  const int ch = lane & 7;
  const uint16_t* src[kLoads];
  int dst[kLoads];
#pragma unroll
  for (int t = 0; t < kLoads; ++t) {
    const int row = 8 * t + (lane >> 3);
    dst[t] = row * kPitchU4 + ch;
    src[t] = row < 16 * TF ? X + (size_t)min(m0 + row, M - 1) * K + 8 * ch
                           : V + (size_t)(j0 + row - 16 * TF) * K + 8 * ch;
  }
  auto load = [&](int kc, u32x4_t (&v)[kLoads]) {
    int col = min(kc, TK - 1) * 64;
    if (col + 8 * ch >= K) col -= 32;  // 32-column tail step: re-read valid columns (masked below)
#pragma unroll
    for (int t = 0; t < kLoads; ++t) v[t] = *(const u32x4_t*)(src[t] + col);
  };

  f32x4_t acc[RF][TF];
#pragma unroll
  for (int a = 0; a < RF; ++a)
#pragma unroll
    for (int f = 0; f < TF; ++f) acc[a][f] = f32x4_t{0, 0, 0, 0};

  // This wave's steps are kc = kb + wave, kb + wave + WAVES, ... < ke; a ring of D steps of loads
  // stays in flight: slot u holds step s0 + u and is refilled with step s0 + u + D right after it is
  // written to LDS; the final round refills nothing. The loop is branch-free: steps past the wave's
  // last one (and the duplicated half of a 32-column tail step) contribute through a zeroed A
  // operand, never through masked loads.
  const int my_steps = max(0, (ke - kb - wave + WAVES - 1) / WAVES);
  const int n_pad = max(1, (my_steps + D - 1) / D) * D;  // at least the final round (a wave may have no steps)
  u32x4_t ring[D][kLoads];
  static_for<D>([&](auto uu) {  // issued in slot order (fenced), as the loop refills them
    load(kb + wave + decltype(uu)::value * WAVES, ring[decltype(uu)::value]);
    asm volatile("" ::: "memory");
  });
  auto step = [&](int s, auto uu, auto refill) {
    constexpr int u = decltype(uu)::value;
    const int kc = kb + wave + s * WAVES;
#pragma unroll
    for (int t = 0; t < kLoads; ++t) st[dst[t]] = ring[u][t];
    if constexpr (decltype(refill)::value) load(kc + D * WAVES, ring[u]);
    // compiler-only fence: the refill stays in this step (not rotated into the next iteration,
    // which would shorten the prefetch distance of this slot)
    asm volatile("" ::: "memory");
    // A operand (V rows j0 + 16 a + sub, dense columns 16 q .. 16 q + 15) as two fixed-pattern
    // 2:4 halves; zero when the step is past this wave's last, or when it is the tail step and
    // these columns are the re-read ones (q >= 2)
    const bool live = s < my_steps && !(half_tail && kc == TK - 1 && quad >= 2);
    const uint32_t keep = live ? ~0u : 0u;
    bf16x16_t bx[TF];
#pragma unroll
    for (int f = 0; f < TF; ++f) {
      const int xrow = (16 * f + sub) * kPitchU4;
      bx[f] = cat16(as_bf16x8(st[xrow + quad]), as_bf16x8(st[xrow + 4 + quad]));
    }
#pragma unroll
    for (int a = 0; a < RF; ++a) {
      const int vrow = (16 * TF + 16 * a + sub) * kPitchU4;
      const u32x4_t d0 = st[vrow + 2 * quad] & keep, d1 = st[vrow + 2 * quad + 1] & keep;
      const bf16x8_t a01 = as_bf16x8(u32x4_t{d0[0], d0[2], d1[0], d1[2]});
      const bf16x8_t a23 = as_bf16x8(u32x4_t{d0[1], d0[3], d1[1], d1[3]});
#pragma unroll
      for (int f = 0; f < TF; ++f) {
        acc[a][f] = smfmac16x16x64(a01, bx[f], acc[a][f], 0x4444);
        acc[a][f] = smfmac16x16x64(a23, bx[f], acc[a][f], 0xEEEE);
      }
    }
  };
  // every round but the last refills its slots; the last round loads nothing past the end
  for (int s0 = 0; s0 + D < n_pad; s0 += D)
    static_for<D>([&](auto uu) { step(s0 + decltype(uu)::value, uu, std::true_type{}); });
  static_for<D>([&](auto uu) { step(n_pad - D + decltype(uu)::value, uu, std::false_type{}); });

  // combine the waves in order; D rows = ranks j0 + 16 a + 4*(lane/16) + 0..3, column = token
  // m0 + 16 f + lane%16
  if (wave > 0) {
#pragma unroll
    for (int a = 0; a < RF; ++a)
#pragma unroll
      for (int f = 0; f < TF; ++f) red[(((wave - 1) * RF + a) * TF + f) * 64 + lane] = acc[a][f];
  }
  __syncthreads();
  if (wave != 0) return;
#pragma unroll
  for (int w = 1; w < WAVES; ++w)
#pragma unroll
    for (int a = 0; a < RF; ++a)
#pragma unroll
      for (int f = 0; f < TF; ++f) acc[a][f] += red[(((w - 1) * RF + a) * TF + f) * 64 + lane];
  float* pz = part + (size_t)blockIdx.z * M * r;
#pragma unroll
  for (int a = 0; a < RF; ++a) {
    const int j = j0 + 16 * a + 4 * quad;
#pragma unroll
    for (int f = 0; f < TF; ++f) {
      const int m = m0 + 16 * f + sub;
      if (m < M) *(f32x4_t*)(pz + (size_t)m * r + j) = acc[a][f];
    }
  }
}

// LDS writes of this wave complete, then workgroup barrier (one asm statement with a memory
// clobber, so that register prefetches stay in flight across it; the builtin wait after it tells
// the compiler's wait-count tracking that no LDS access is outstanding).
__device__ __forceinline__ void lds_barrier() {
  asm volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory");
  __builtin_amdgcn_s_waitcnt(0xc07f);
}

// Tile kernel for many tokens: a workgroup owns BM = 16*TMW*WM tokens x BR = 16*TRW*WR ranks over
// one K slice (grid: x = token block * rank_blocks + rank block, z = K slice), so that X is read
// from memory once when
// BR covers r. Per 64-column K step the four waves stage the step's X rows into one slot of a
// two-slot LDS ring (row-contiguous 16-byte loads, one barrier per step) and wave w computes its
// 16*TMW tokens x 16*TRW ranks: X fragments come from the slot, V fragments (small, L2-resident)
// straight from global memory into registers. Loads of both run P steps ahead in registers. V is
// the A operand (two fixed 2:4 halves, as above), X the B operand. Rows past M and ranks past r
// repeat the last valid row and are never stored.
template <int TMW, int TRW, int WM, int WR, int P>
__global__ __launch_bounds__(256) void lowrank_tile_kernel(const uint16_t* __restrict__ X,
                                                          const uint16_t* __restrict__ V, int M, int K, int r,
                                                          int rank_blocks, int steps_per_slice,
                                                          float* __restrict__ part) {
  static_assert(WM * WR == 4, "four waves");
  constexpr int BM = 16 * TMW * WM, BR = 16 * TRW * WR;
  constexpr int kChunks = BM * 8;                  // 16-byte chunks of X per step
  constexpr int kLoads = (kChunks + 255) / 256;    // per thread per step
  __shared__ u32x4_t slot[2][BM * kPitchU4];
  const int lane = threadIdx.x & 63, wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int sub = lane & 15, quad = lane >> 4;
  const int wm = wave % WM, wr = wave / WM;
  const int mb = blockIdx.x / rank_blocks;
  const int j0 = (blockIdx.x - mb * rank_blocks) * BR, m0 = mb * BM;
  const int TK = (K + 63) / 64;
  const int kb = blockIdx.z * steps_per_slice;
  const int n_steps = min(TK, kb + steps_per_slice) - kb;  // >= 1 by the choice of slices
  const bool half_tail = (K & 63) != 0;                      // the last step holds 32 valid columns

  // X: thread chunk c -> token row c / 8, 16-byte chunk c % 8 of the step
  const uint16_t* xsrc[kLoads];
  int xdst[kLoads], xch[kLoads];
#pragma unroll
  for (int t = 0; t < kLoads; ++t) {
    const int c = min((int)threadIdx.x + 256 * t, kChunks - 1);
    xch[t] = c & 7;
    xdst[t] = threadIdx.x + 256 * t < kChunks ? (c >> 3) * kPitchU4 + xch[t] : -1;
    xsrc[t] = X + (size_t)min(m0 + (c >> 3), M - 1) * K + 8 * xch[t];
  }
  // V: A fragment of rank block a -> row j0 + 16 (wr TRW + a) + lane%16, dense columns 16 q .. 16 q + 15
  const uint16_t* vsrc[TRW];
#pragma unroll
  for (int a = 0; a < TRW; ++a) vsrc[a] = V + (size_t)min(j0 + 16 * (wr * TRW + a) + sub, r - 1) * K + 16 * quad;

  auto loadx = [&](int kc, u32x4_t (&v)[kLoads]) {
#pragma unroll
    for (int t = 0; t < kLoads; ++t) {
      int col = kc * 64;
      if (col + 8 * xch[t] >= K) col -= 32;  // 32-column tail step: re-read valid columns (zeroed below)
      v[t] = *(const u32x4_t*)(xsrc[t] + col);
    }
  };
  auto loadv = [&](int kc, u32x4_t (&v)[TRW][2]) {
    int col = kc * 64;
    if (col + 16 * quad >= K) col -= 32;  // as above
#pragma unroll
    for (int a = 0; a < TRW; ++a) {
      v[a][0] = *(const u32x4_t*)(vsrc[a] + col);
      v[a][1] = *(const u32x4_t*)(vsrc[a] + col + 8);
    }
  };

  f32x4_t acc[TRW][TMW];
#pragma unroll
  for (int a = 0; a < TRW; ++a)
#pragma unroll
    for (int i = 0; i < TMW; ++i) acc[a][i] = f32x4_t{0, 0, 0, 0};

  // A ring of P steps of loads stays in flight: register slot u holds step s0 + u and is refilled
  // with step s0 + u + P as soon as it has been consumed. Branch-free (conditional loads would make
  // the compiler wait for every outstanding load): steps are padded to a multiple of P, loads past
  // the slice's last step re-read that step, and padded steps contribute through a zeroed A operand.
  const int n_pad = (n_steps + P - 1) / P * P;
  u32x4_t xring[P][kLoads], vring[P][TRW][2];
  static_for<P>([&](auto uu) {  // issued in slot order (fenced), as the loop refills them
    constexpr int u = decltype(uu)::value;
    loadx(kb + min(u, n_steps - 1), xring[u]);
    loadv(kb + min(u, n_steps - 1), vring[u]);
    asm volatile("" ::: "memory");
  });
  auto step = [&](int s, auto uu, auto refill) {
    constexpr int u = decltype(uu)::value;
    constexpr bool kRefill = decltype(refill)::value;
    const int next = kb + min(s + P, n_steps - 1);
    u32x4_t* sl = slot[s & 1];
#pragma unroll
    for (int t = 0; t < kLoads; ++t)
      if (xdst[t] >= 0) sl[xdst[t]] = xring[u][t];
    if constexpr (kRefill) loadx(next, xring[u]);
    asm volatile("" ::: "memory");  // compiler-only fence: the refill stays in this step
    lds_barrier();
    const int kc = kb + s;
    // A operand zero past the slice's last step, and for the re-read upper half of a 32-column tail
    // step (dense columns 32..63)
    const bool live = s < n_steps && !(half_tail && kc == TK - 1 && quad >= 2);
    const uint32_t keep = live ? ~0u : 0u;
    bf16x8_t a01[TRW], a23[TRW];
#pragma unroll
    for (int a = 0; a < TRW; ++a) {
      const u32x4_t d0 = vring[u][a][0] & keep, d1 = vring[u][a][1] & keep;
      a01[a] = as_bf16x8(u32x4_t{d0[0], d0[2], d1[0], d1[2]});
      a23[a] = as_bf16x8(u32x4_t{d0[1], d0[3], d1[1], d1[3]});
    }
    if constexpr (kRefill) loadv(next, vring[u]);
    asm volatile("" ::: "memory");
    bf16x16_t bx[TMW];
#pragma unroll
    for (int i = 0; i < TMW; ++i) {
      const int xrow = (16 * (wm * TMW + i) + sub) * kPitchU4;
      bx[i] = cat16(as_bf16x8(sl[xrow + quad]), as_bf16x8(sl[xrow + 4 + quad]));
    }
#pragma unroll
    for (int a = 0; a < TRW; ++a)
#pragma unroll
      for (int i = 0; i < TMW; ++i) {
        acc[a][i] = smfmac16x16x64(a01[a], bx[i], acc[a][i], 0x4444);
        acc[a][i] = smfmac16x16x64(a23[a], bx[i], acc[a][i], 0xEEEE);
      }
  };
  // every round but the last refills its slots; the last round loads nothing more
  for (int s0 = 0; s0 + P < n_pad; s0 += P)
    static_for<P>([&](auto uu) { step(s0 + decltype(uu)::value, uu, std::true_type{}); });
  static_for<P>([&](auto uu) { step(n_pad - P + decltype(uu)::value, uu, std::false_type{}); });

  // D rows = ranks j0 + 16 (wr TRW + a) + 4*(lane/16) + 0..3, column = token m0 + 16 (wm TMW + i) + lane%16
  float* pz = part + (size_t)blockIdx.z * M * r;
#pragma unroll
  for (int a = 0; a < TRW; ++a) {
    const int j = j0 + 16 * (wr * TRW + a) + 4 * quad;
#pragma unroll
    for (int i = 0; i < TMW; ++i) {
      const int m = m0 + 16 * (wm * TMW + i) + sub;
      if (m < M && j < r) *(f32x4_t*)(pz + (size_t)m * r + j) = acc[a][i];
    }
  }
}

// One wave per output T[m][j] (outputs numbered m * r + j, 64-bit); the grid strides over them.
__global__ __launch_bounds__(256) void lowrank_f32_kernel(const float* __restrict__ X, const float* __restrict__ V,
                                                         int M, int K, int r, float* __restrict__ T) {
  const int lane = threadIdx.x & 63;
  const int64_t outputs = (int64_t)M * r;
  for (int64_t o = (int64_t)blockIdx.x * 4 + (threadIdx.x >> 6); o < outputs; o += (int64_t)gridDim.x * 4) {
    const int64_t m = o / r, j = o - m * r;
    const float* x = X + (size_t)m * K;
    const float* v = V + (size_t)j * K;
    float t = 0.0f;
    for (int k = lane; k < K; k += 64) t = fmaf(x[k], v[k], t);
#pragma unroll
    for (int off = 32; off > 0; off >>= 1) t += __shfl_xor(t, off);
    if (lane == 0) T[o] = t;
  }
}

}  // namespace

namespace {

// bf16 first-stage shape, chosen by measurement on MI355X. For r <= 64, lowrank_bf16_kernel: ~256
// small workgroups, 16 ranks each for decode-sized inputs (M <= 16) and 32 otherwise (when 32
// divides r), K split into slices only as far as needed to reach ~256 workgroups (at most
// kMaxLowrankSlices); each X row is staged at most twice, by concurrently running workgroups.
// For r > 64 the rank blocks of that kernel would stream X from memory r/32 times: the tile kernel
// takes 128 ranks per workgroup (X read once for r <= 128) and 16, 32 or 64 tokens by M.
struct LowrankShape {
  bool tile;
  int tf, rf;   // lowrank_bf16_kernel: 16*tf tokens x 16*rf ranks
  int bm;       // tile kernel: bm tokens x 128 ranks
  int slices, steps_per_slice;
};

// For decode-sized inputs (M <= 16) every workgroup of the second stage reads all K slices of T
// (float32 partials), so more slices cost more there than they save here: at most 8 (measured at
// 16 tokens x 4096 x rank 64: 2.83 + 6.44 us per call with 8, 2.91 + 6.59 with 16, 3.24 + 6.44
// with 4).
constexpr int64_t kDecodeMaxSlices = 8;

LowrankShape lowrank_shape(int64_t M, int64_t n_in, int64_t r) {
  constexpr int64_t kWant = 256;
  LowrankShape sh{};
  const int64_t TK = (n_in + 63) / 64;
  int64_t base;
  if (M <= 16 || r <= 64) {
    sh.tile = false;
    sh.tf = M <= 16 ? 1 : 2;
    sh.rf = (M > 16 && r % 32 == 0) ? 2 : 1;
    base = ceil_div(M, 16 * sh.tf) * (r / (16 * sh.rf));
  } else {
    sh.tile = true;
    sh.bm = M >= 4096 ? 64 : (M >= 1024 ? 32 : 16);
    base = ceil_div(M, sh.bm) * ceil_div(r, 128);
  }
  const int64_t slices =
      std::min<int64_t>(std::min<int64_t>(M <= 16 ? kDecodeMaxSlices : kMaxLowrankSlices, TK),
                       std::max<int64_t>(1, ceil_div(kWant, base)));
  sh.steps_per_slice = (int)ceil_div(TK, slices);
  sh.slices = (int)ceil_div(TK, sh.steps_per_slice);
  return sh;
}

dim3 part_grid(const LowrankShape& sh, int64_t M, int64_t r) {
  return dim3((unsigned)cdiv(M, 16 * sh.tf), (unsigned)(r / (16 * sh.rf)), (unsigned)sh.slices);
}
dim3 tile_grid(const LowrankShape& sh, int64_t M, int64_t r) {
  return dim3((unsigned)(ceil_div(r, 128) * ceil_div(M, sh.bm)), 1u, (unsigned)sh.slices);
}
constexpr int64_t kMaxF32Blocks = int64_t(1) << 20;
dim3 f32_grid(int64_t M, int64_t r) { return dim3((unsigned)std::min(ceil_div(M * r, 4), kMaxF32Blocks)); }

template <int TF, int RF>
void launch_part(const LowrankShape& sh, const void* X, const void* V, int64_t M, int64_t n_in, int64_t r,
                 float* part, hipStream_t stream) {
  const dim3 grid = part_grid(sh, M, r);
  if (sh.steps_per_slice >= 16)
    lowrank_bf16_kernel<TF, RF, 4, 4><<<grid, dim3(256), 0, stream>>>((const uint16_t*)X, (const uint16_t*)V, (int)M,
                                                                    (int)n_in, (int)r, sh.steps_per_slice, part);
  else
    lowrank_bf16_kernel<TF, RF, 4, 2><<<grid, dim3(256), 0, stream>>>((const uint16_t*)X, (const uint16_t*)V, (int)M,
                                                                    (int)n_in, (int)r, sh.steps_per_slice, part);
}

template <int TMW>
void launch_tile(const LowrankShape& sh, const void* X, const void* V, int64_t M, int64_t n_in, int64_t r,
                 float* part, hipStream_t stream) {
  const dim3 grid = tile_grid(sh, M, r);
  lowrank_tile_kernel<TMW, 2, 1, 4, 4><<<grid, dim3(256), 0, stream>>>(
      (const uint16_t*)X, (const uint16_t*)V, (int)M, (int)n_in, (int)r, cdiv(r, 128), sh.steps_per_slice, part);
}

}  // namespace

bool lowrank_grids_fit(int64_t M, int64_t n_in, int64_t r, bool bf16) {
  if (r == 0) return true;
  if (!bf16) return grid_fits(f32_grid(M, r), 256);
  const LowrankShape sh = lowrank_shape(M, n_in, r);
  return grid_fits(sh.tile ? tile_grid(sh, M, r) : part_grid(sh, M, r), 256);
}

int lowrank_slices(int64_t M, int64_t n_in, int64_t r, bool bf16) {
  return (r == 0 || !bf16) ? 1 : lowrank_shape(M, n_in, r).slices;
}

size_t lowrank_workspace_bytes(int64_t M, int64_t n_in, int64_t r, bool bf16) {
  if (r == 0) return 0;
  return (size_t)lowrank_slices(M, n_in, r, bf16) * M * r * sizeof(float);
}

hipError_t launch_lowrank(const void* X, const void* V, int64_t M, int64_t n_in, int64_t r, bool bf16,
                          void* workspace, hipStream_t stream) {
  if (r == 0) return hipSuccess;
  float* part = (float*)workspace;
  if (bf16) {
    const LowrankShape sh = lowrank_shape(M, n_in, r);
    if (!sh.tile) {
      if (sh.tf == 1) launch_part<1, 1>(sh, X, V, M, n_in, r, part, stream);
      else if (sh.rf == 2) launch_part<2, 2>(sh, X, V, M, n_in, r, part, stream);
      else launch_part<2, 1>(sh, X, V, M, n_in, r, part, stream);
    } else if (sh.bm == 16) {
      launch_tile<1>(sh, X, V, M, n_in, r, part, stream);
    } else if (sh.bm == 32) {
      launch_tile<2>(sh, X, V, M, n_in, r, part, stream);
    } else {
      launch_tile<4>(sh, X, V, M, n_in, r, part, stream);
    }
  } else {
    lowrank_f32_kernel<<<f32_grid(M, r), dim3(256), 0, stream>>>(
        (const float*)X, (const float*)V, (int)M, (int)n_in, (int)r, part);
  }
  return hipGetLastError();
}

}  // namespace splr
