// Y = X S^T + (X V^T) U^T for few tokens (M <= 64, bfloat16; LoSparse page, §3.2): the decode
// kernel. HBM-bound on S: a workgroup owns 16 rows; its 4 waves take interleaved 64-column K steps,
// stream S straight into registers (non-temporal loads) and X through a private LDS slot each, and
// combine their partial accumulators through LDS in a fixed order; wave 0 adds the rank-r term and
// stores Y.
#include "common.hpp"
#include "kernels.hpp"
#include "tile_common.hpp"

namespace splr {
namespace {

// ----------------------------------------------------------------------------------- decode

// U's rows tr0 + lane%16, ranks 16 (lane / 16) .. +15 of the first 64-rank block (zeros past n_out
// or r), as loaded; pair01 / pair23 give the (0,1) and (2,3) halves of every group of four ranks,
// the A operands of the two structured-sparse MFMAs that make one dense product
struct URow {
  u32x4_t d0, d1;
  __device__ __forceinline__ void load(const uint16_t* __restrict__ U, int n_out, int r, int tr0, int lane) {
    const int n = tr0 + (lane & 15), ju = 16 * (lane >> 4);
    const bool ok = n < n_out && ju < r;
    const uint16_t* p = U + (size_t)(ok ? n : 0) * r + (ok ? ju : 0);
    const u32x4_t zero = {0, 0, 0, 0};
    d0 = ok ? *(const u32x4_t*)p : zero;
    d1 = ok ? *(const u32x4_t*)(p + 8) : zero;
  }
  __device__ __forceinline__ bf16x8_t pair01() const { return as_bf16x8(u32x4_t{d0[0], d0[2], d1[0], d1[2]}); }
  __device__ __forceinline__ bf16x8_t pair23() const { return as_bf16x8(u32x4_t{d0[1], d0[3], d1[1], d1[3]}); }
};

template <int MB, int P, int WAVES>
__global__ __launch_bounds__(64 * WAVES) void linear_decode_kernel(
    const uint16_t* __restrict__ X, const u32x4_t* __restrict__ values, const uint32_t* __restrict__ meta,
    const uint16_t* __restrict__ U, const float* __restrict__ Tpart, int slices, void* __restrict__ Y, int y_bf16, int M, int K,
    int n_out, int r) {
  constexpr int kXLoads = 2 * MB;  // 8 tokens x 128 bytes per load instruction, 16*MB tokens
  __shared__ u32x4_t xs[WAVES][16 * MB * kXPitchU4];
  __shared__ f32x4_t red[(WAVES - 1) * MB * 64];
  __shared__ u32x4_t tpair[2 * kPreRankBlocks][16 * MB * kXPitchU4];  // T's bfloat16 pair (hi, lo)
  // the wave index is uniform across the wave; readfirstlane lets the compiler see that (scalar
  // loop control instead of exec-mask loops)
  const int lane = threadIdx.x & 63, wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int sub = lane & 15, quad = lane >> 4;
  const int tr = blockIdx.x, m0 = blockIdx.y * 16 * MB;
  const int TK = (K + 63) / 64;

  const u32x4_t* vsrc = values + (size_t)tr * TK * 64 + lane;
  const uint16_t* msrc = (const uint16_t*)meta + ((size_t)tr * meta_blocks(TK) * 64 + lane) * 8;
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
    // S is read once per call: non-temporal, so it does not displace X, T and U, which every
    // workgroup re-reads (8.35 -> 7.85 us per 16-token call at 4096 x 4096)
    va = __builtin_nontemporal_load(vsrc + (size_t)kc * 64);
    wa = msrc[(size_t)(kc >> 3) * 512 + (kc & 7)];
    int col = kc * 64;
    if (col + 8 * xchunk >= K) col -= 32;  // half tail step: re-read valid columns (S is zero there)
#pragma unroll
    for (int t = 0; t < kXLoads; ++t) xv[t] = *(const u32x4_t*)(xsrc[t] + col);
  };

  // T's pair: its loads go out first, the ring's next, and the pair is written to LDS while the
  // ring's loads are in flight (published by the barrier after the loop)
  const bool t_pre = r <= 64 * kPreRankBlocks;
  TPairBuilder<16 * MB, 64 * WAVES, MB == 1 ? 8 : 0> tb;  // 16 tokens: at most 8 K slices, all in one round
  if (t_pre && r > 0) {
    tb.init(Tpart, slices, M, r, m0, 0, threadIdx.x);
    tb.issue(0);
  }
  // U's fragments for wave 0's rank-r term, loaded now: after the loop their memory latency would
  // be exposed at the end of the call
  URow uf;
  if (t_pre && r > 0 && wave == 0) uf.load(U, n_out, r, tr * 16, lane);
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
    static_assert(kPreRankBlocks == 1, "one block of U fragments loaded ahead");
    if (wave == 0 && r > 0) {
      const bf16x8_t u01 = uf.pair01(), u23 = uf.pair23();
#pragma unroll
      for (int j = 0; j < MB; ++j) {
        const int row = (16 * j + sub) * kXPitchU4;
        const bf16x16_t th = cat16(as_bf16x8(tpair[0][row + quad]), as_bf16x8(tpair[0][row + 4 + quad]));
        const bf16x16_t tl = cat16(as_bf16x8(tpair[1][row + quad]), as_bf16x8(tpair[1][row + 4 + quad]));
        acc[0][j] = smfmac16x16x64(u01, th, acc[0][j], 0x4444);
        acc[0][j] = smfmac16x16x64(u23, th, acc[0][j], 0xEEEE);
        acc[0][j] = smfmac16x16x64(u01, tl, acc[0][j], 0x4444);
        acc[0][j] = smfmac16x16x64(u23, tl, acc[0][j], 0xEEEE);
      }
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

dim3 decode_grid(int64_t M, int64_t n_out, int MB) {
  return dim3((unsigned)ceil_div(n_out, 16), (unsigned)ceil_div(M, 16 * MB));
}

template <int MB>
hipError_t launch_decode(const void* X, int64_t M, int64_t n_in, const void* values, const uint32_t* meta,
                         int64_t n_out, const void* U, int64_t r, const float* Tpart, int slices, void* Y,
                         int y_bf16, hipStream_t stream) {
  constexpr int P = MB == 1 ? 8 : 4, W = 4;
  const dim3 grid = decode_grid(M, n_out, MB);
  linear_decode_kernel<MB, P, W><<<grid, dim3(64 * W), 0, stream>>>(
      (const uint16_t*)X, (const u32x4_t*)values, meta, (const uint16_t*)U, Tpart, slices, Y, y_bf16, (int)M,
      (int)n_in, (int)n_out, (int)r);
  return hipGetLastError();
}

}  // namespace

bool decode_grids_fit(int64_t M, int64_t n_out) {
  return grid_fits(decode_grid(M, n_out, M <= 16 ? 1 : (M <= 32 ? 2 : 4)), 256);
}

hipError_t launch_linear_decode(const void* X, int64_t M, int64_t n_in, const void* values, const uint32_t* meta,
                                int64_t n_out, const void* U, int64_t r, const float* Tpart, int slices, void* Y,
                                bool y_bf16, hipStream_t stream) {
  const int yb = y_bf16 ? 1 : 0;
  if (M <= 16) return launch_decode<1>(X, M, n_in, values, meta, n_out, U, r, Tpart, slices, Y, yb, stream);
  if (M <= 32) return launch_decode<2>(X, M, n_in, values, meta, n_out, U, r, Tpart, slices, Y, yb, stream);
  return launch_decode<4>(X, M, n_in, values, meta, n_out, U, r, Tpart, slices, Y, yb, stream);
}

}  // namespace splr
