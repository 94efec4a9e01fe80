// Y = X S^T + (X V^T) U^T for bfloat16 operands, float32 accumulation and output (LoSparse page,
// §3.2: the sparse product and the low-rank product are evaluated side by side and summed).
//
// The sparse product runs on gfx950's structured-sparse MFMA, v_smfmac_f32_16x16x64_bf16, as
// Y^T tiles = S_tile * X_tile^T: S is the sparse A operand (16 rows x 64 columns, stored as the 32
// kept values), X^T the dense B operand. The packed layout feeds it without conversion: a lane's
// A operand is 8 consecutive kept values of one row (16 bytes), and its index operand is the 16
// metadata bits of the same 4 groups, i.e. one half of a metadata word.
// Lane layouts (gfx950):
//   A (S):  lane l -> row l%16, dense columns 16*(l/16) .. +15  (kept values 8*(l/16) .. +7)
//   B (X):  lane l -> token l%16, columns 8*(l/16)+0..7 and 32+8*(l/16)+0..7
//   D:      lane l -> rows (n) 4*(l/16)+0..3, token l%16
// The low-rank epilogue uses dense v_mfma_f32_16x16x32_bf16, whose D layout is the same, so it
// accumulates into the same registers: acc += U_tile * T_tile^T, with T (float32) split into a
// bfloat16 high part and a bfloat16 correction. Y is stored once.
//
// Two kernels:
//   prefill -- WG tile BN x BM, both operands staged through LDS in fragment order (each lane's
//              16-byte pieces contiguous, so every LDS read is a conflict-free 1 KiB wave read),
//              double-buffered, one barrier per 64-column K step; workgroups are remapped so the
//              tiles that one XCD (own L2) runs share rows of X and S.
//   decode  -- few tokens: HBM-bound on S. A workgroup owns 16 rows of S; its waves take
//              interleaved 64-column K steps, stream S and its metadata straight into registers
//              (several steps of loads in flight), read X from L2, and combine their partial
//              accumulators through LDS in a fixed order.
#include "common.hpp"
#include "kernels.hpp"

namespace splr {
namespace {

// ---------------------------------------------------------------------------------------- shared

// Low-rank epilogue for one 16x16 accumulator block set.
// acc[i][j] (rows n = nrow0 + 16 i, tokens m = mrow0 + 16 j) += U[n][:] . T[m][:]
template <int NI, int NJ>
__device__ __forceinline__ void lowrank_epilogue(f32x4_t (&acc)[NI][NJ], const uint16_t* __restrict__ U,
                                                 const float* __restrict__ Tpart, int ksplit, int M, int n_out,
                                                 int r, int nrow0, int mrow0, int lane) {
  const int sub = lane & 15, koff = 8 * (lane >> 4);
  const size_t plane = (size_t)M * r;
  for (int j0 = 0; j0 < r; j0 += 32) {
    const int jj = j0 + koff;
    const bool j_ok = jj < r;  // r % 16 == 0: a lane's 8 ranks are all valid or all past the end
    bf16x8_t thi[NJ], tlo[NJ];
#pragma unroll
    for (int j = 0; j < NJ; ++j) {
      const int m = mrow0 + 16 * j + sub;
      float t[8] = {0, 0, 0, 0, 0, 0, 0, 0};
      if (m < M && j_ok) {
        const float* p = Tpart + (size_t)m * r + jj;
        for (int s = 0; s < ksplit; ++s) {
          const f32x4_t a = *(const f32x4_t*)(p + s * plane);
          const f32x4_t b = *(const f32x4_t*)(p + s * plane + 4);
          t[0] += a[0]; t[1] += a[1]; t[2] += a[2]; t[3] += a[3];
          t[4] += b[0]; t[5] += b[1]; t[6] += b[2]; t[7] += b[3];
        }
      }
      split_hi_lo(t, thi[j], tlo[j]);
    }
#pragma unroll
    for (int i = 0; i < NI; ++i) {
      const int n = nrow0 + 16 * i + sub;
      const u32x4_t zero = {0, 0, 0, 0};
      const bf16x8_t u = as_bf16x8((n < n_out && j_ok) ? *(const u32x4_t*)(U + (size_t)n * r + jj) : zero);
#pragma unroll
      for (int j = 0; j < NJ; ++j) {
        acc[i][j] = mfma16x16x32(u, thi[j], acc[i][j]);
        acc[i][j] = mfma16x16x32(u, tlo[j], acc[i][j]);
      }
    }
  }
}

// Store acc[i][j] (rows n = nrow0 + 16 i + 4*(lane/16) + 0..3, token m = mrow0 + 16 j + lane%16).
template <int NI, int NJ>
__device__ __forceinline__ void store_tile(const f32x4_t (&acc)[NI][NJ], float* __restrict__ Y, int M, int n_out,
                                           int nrow0, int mrow0, int lane) {
  const bool vec_ok = (n_out & 3) == 0;
#pragma unroll
  for (int j = 0; j < NJ; ++j) {
    const int m = mrow0 + 16 * j + (lane & 15);
    if (m >= M) continue;
    float* yrow = Y + (size_t)m * n_out;
#pragma unroll
    for (int i = 0; i < NI; ++i) {
      const int n = nrow0 + 16 * i + 4 * (lane >> 4);
      if (vec_ok && n + 3 < n_out) {
        *(f32x4_t*)(yrow + n) = acc[i][j];
      } else {
#pragma unroll
        for (int s = 0; s < 4; ++s)
          if (n + s < n_out) yrow[n + s] = acc[i][j][s];
      }
    }
  }
}

// ---------------------------------------------------------------------------------------- prefill

template <int BN, int BM, int WN, int WM>
struct PrefillCfg {
  static constexpr int kWavesN = BN / WN, kWavesM = BM / WM;
  static constexpr int kThreads = 64 * kWavesN * kWavesM;
  static constexpr int NI = WN / 16, NJ = WM / 16;
  // LDS stage, in 16-byte units: A fragments (BN/16 x 64 lanes), X fragments (BM/16 x 2 x 64),
  // then metadata (BN rows x 2 words = BN/2 units).
  static constexpr int kAUnits = BN * 4;
  static constexpr int kXUnits = BM * 8;
  static constexpr int kMUnits = BN / 2;
  static constexpr int kStageUnits = kAUnits + kXUnits + kMUnits;
  static constexpr int kAChunksPerThread = (kAUnits + kThreads - 1) / kThreads;
  static constexpr int kXChunksPerThread = (kXUnits + kThreads - 1) / kThreads;
  static constexpr int kMWordsPerThread = (BN * 2 + kThreads - 1) / kThreads;
};

template <int BN, int BM, int WN, int WM>
__global__ __launch_bounds__(64 * (BN / WN) * (BM / WM)) void linear_prefill_kernel(
    const uint16_t* __restrict__ X, const uint16_t* __restrict__ values, const uint32_t* __restrict__ meta,
    const uint16_t* __restrict__ U, const float* __restrict__ Tpart, float* __restrict__ Y, int M, int K,
    int n_out, int r, int ksplit, int tiles_n, int tiles_m, int tiles_per_xcd, int group_m) {
  using C = PrefillCfg<BN, BM, WN, WM>;
  __shared__ u32x4_t lds[2 * C::kStageUnits];

  // --- XCD-aware tile order: workgroup b runs on XCD b % 8; give each XCD a contiguous range of
  // logical tiles, and walk logical tiles in groups of `group_m` token tiles so that the tiles of
  // one XCD share X rows and S rows.
  const int b = blockIdx.x;
  const int logical = (b & 7) * tiles_per_xcd + (b >> 3);
  const int n_tiles = tiles_n * tiles_m;
  if (logical >= n_tiles) return;
  const int per_group = group_m * tiles_n;
  const int g = logical / per_group;
  const int first_m = g * group_m;
  const int gsize = min(group_m, tiles_m - first_m);
  const int in_group = logical - g * per_group;
  const int tile_m = first_m + in_group % gsize;
  const int tile_n = in_group / gsize;
  const int n0 = tile_n * BN, m0 = tile_m * BM;

  const int tid = threadIdx.x;
  const int lane = tid & 63, wave = tid >> 6;
  const int wn = wave % C::kWavesN, wm = wave / C::kWavesN;
  const int Kc = K / 2;          // kept values per row
  const int Kw = K / 32;         // metadata words per row
  const int nk = (K + 63) / 64;  // 64-column K steps (the last may be half)

  // global -> register staging for one K step
  u32x4_t ra[C::kAChunksPerThread], rx[C::kXChunksPerThread];
  uint32_t rm[C::kMWordsPerThread];
  const u32x4_t zero = {0, 0, 0, 0};

  auto load_stage = [&](int kc) {
#pragma unroll
    for (int c = 0; c < C::kAChunksPerThread; ++c) {
      const int q = tid + c * C::kThreads;
      const int row = q >> 2, part = q & 3;
      const int n = n0 + row;
      const int kv = kc * 32 + part * 8;  // kept-value column
      ra[c] = (q < C::kAUnits && n < n_out && kv < Kc) ? *(const u32x4_t*)(values + (size_t)n * Kc + kv) : zero;
    }
#pragma unroll
    for (int c = 0; c < C::kXChunksPerThread; ++c) {
      const int q = tid + c * C::kThreads;
      const int row = q >> 3, part = q & 7;
      const int m = m0 + row;
      const int k = kc * 64 + part * 8;
      rx[c] = (q < C::kXUnits && m < M && k < K) ? *(const u32x4_t*)(X + (size_t)m * K + k) : zero;
    }
#pragma unroll
    for (int c = 0; c < C::kMWordsPerThread; ++c) {
      const int q = tid + c * C::kThreads;
      const int row = q >> 1, w = q & 1;
      const int n = n0 + row;
      const int kw = kc * 2 + w;
      rm[c] = (q < BN * 2 && n < n_out && kw < Kw) ? meta[(size_t)n * Kw + kw] : 0u;
    }
  };
  auto store_stage = [&](int buf) {
    u32x4_t* st = lds + buf * C::kStageUnits;
#pragma unroll
    for (int c = 0; c < C::kAChunksPerThread; ++c) {
      const int q = tid + c * C::kThreads;
      if (q < C::kAUnits) {
        const int row = q >> 2, part = q & 3;
        st[(row >> 4) * 64 + (row & 15) + 16 * part] = ra[c];
      }
    }
#pragma unroll
    for (int c = 0; c < C::kXChunksPerThread; ++c) {
      const int q = tid + c * C::kThreads;
      if (q < C::kXUnits) {
        const int row = q >> 3, part = q & 7;
        st[C::kAUnits + ((row >> 4) * 2 + (part >> 2)) * 64 + (row & 15) + 16 * (part & 3)] = rx[c];
      }
    }
    uint32_t* sm = (uint32_t*)(st + C::kAUnits + C::kXUnits);
#pragma unroll
    for (int c = 0; c < C::kMWordsPerThread; ++c) {
      const int q = tid + c * C::kThreads;
      if (q < BN * 2) sm[q] = rm[c];
    }
  };

  f32x4_t acc[C::NI][C::NJ];
#pragma unroll
  for (int i = 0; i < C::NI; ++i)
#pragma unroll
    for (int j = 0; j < C::NJ; ++j) acc[i][j] = f32x4_t{0, 0, 0, 0};

  load_stage(0);
  store_stage(0);
  __syncthreads();

  const int sub = lane & 15, quad = lane >> 4;
  for (int kc = 0; kc < nk; ++kc) {
    const int cur = kc & 1;
    if (kc + 1 < nk) load_stage(kc + 1);
    const u32x4_t* st = lds + cur * C::kStageUnits;
    const uint32_t* sm = (const uint32_t*)(st + C::kAUnits + C::kXUnits);
    bf16x8_t a[C::NI];
    int idx[C::NI];
#pragma unroll
    for (int i = 0; i < C::NI; ++i) {
      const int rowblk = wn * C::NI + i;
      a[i] = as_bf16x8(st[rowblk * 64 + lane]);
      const uint32_t w = sm[(rowblk * 16 + sub) * 2 + (quad >> 1)];
      idx[i] = (int)(w >> (16 * (quad & 1)));
    }
#pragma unroll
    for (int j = 0; j < C::NJ; ++j) {
      const int colblk = wm * C::NJ + j;
      const bf16x16_t bx = cat16(as_bf16x8(st[C::kAUnits + (colblk * 2) * 64 + lane]),
                                 as_bf16x8(st[C::kAUnits + (colblk * 2 + 1) * 64 + lane]));
#pragma unroll
      for (int i = 0; i < C::NI; ++i) acc[i][j] = smfmac16x16x64(a[i], bx, acc[i][j], idx[i]);
    }
    if (kc + 1 < nk) store_stage(cur ^ 1);
    __syncthreads();
  }

  const int nrow0 = n0 + wn * WN, mrow0 = m0 + wm * WM;
  if (r > 0) lowrank_epilogue<C::NI, C::NJ>(acc, U, Tpart, ksplit, M, n_out, r, nrow0, mrow0, lane);
  store_tile<C::NI, C::NJ>(acc, Y, M, n_out, nrow0, mrow0, lane);
}

// ---------------------------------------------------------------------------------------- decode

template <int KW, int MB, int UNROLL>
__global__ __launch_bounds__(64 * KW) void linear_decode_kernel(
    const uint16_t* __restrict__ X, const uint16_t* __restrict__ values, const uint32_t* __restrict__ meta,
    const uint16_t* __restrict__ U, const float* __restrict__ Tpart, float* __restrict__ Y, int M, int K,
    int n_out, int r, int ksplit) {
  __shared__ f32x4_t red[(KW - 1) * MB * 64];
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int n0 = blockIdx.x * 16, m0 = blockIdx.y * 16 * MB;
  const int sub = lane & 15, quad = lane >> 4;
  const int Kc = K / 2, Kw = K / 32;
  const int nk = (K + 63) / 64;

  const int n = n0 + sub;
  const bool n_ok = n < n_out;
  const uint16_t* vrow = values + (size_t)(n_ok ? n : 0) * Kc + 8 * quad;
  const uint32_t* mrow = meta + (size_t)(n_ok ? n : 0) * Kw + (quad >> 1);
  const int mshift = 16 * (quad & 1);
  const uint16_t* xrow[MB];
  bool m_ok[MB];
#pragma unroll
  for (int j = 0; j < MB; ++j) {
    const int m = m0 + 16 * j + sub;
    m_ok[j] = m < M;
    xrow[j] = X + (size_t)(m_ok[j] ? m : 0) * K + 8 * quad;
  }

  f32x4_t acc[1][MB];
#pragma unroll
  for (int j = 0; j < MB; ++j) acc[0][j] = f32x4_t{0, 0, 0, 0};
  const u32x4_t zero = {0, 0, 0, 0};

  for (int kc0 = wave; kc0 < nk; kc0 += KW * UNROLL) {
    u32x4_t av[UNROLL], xv[UNROLL][MB][2];
    uint32_t mv[UNROLL];
#pragma unroll
    for (int u = 0; u < UNROLL; ++u) {
      const int kc = kc0 + u * KW;
      const bool in = kc < nk;
      const bool a_in = in && n_ok && kc * 32 + 8 * quad < Kc;
      av[u] = a_in ? __builtin_nontemporal_load((const u32x4_t*)(vrow + (size_t)kc * 32)) : zero;
      mv[u] = (in && n_ok && kc * 2 + (quad >> 1) < Kw) ? mrow[(size_t)kc * 2] : 0u;
#pragma unroll
      for (int j = 0; j < MB; ++j) {
        const size_t k = (size_t)kc * 64;
        const bool x0 = in && m_ok[j] && (int)k + 8 * quad < K;
        const bool x1 = in && m_ok[j] && (int)k + 32 + 8 * quad < K;
        xv[u][j][0] = x0 ? *(const u32x4_t*)(xrow[j] + k) : zero;
        xv[u][j][1] = x1 ? *(const u32x4_t*)(xrow[j] + k + 32) : zero;
      }
    }
#pragma unroll
    for (int u = 0; u < UNROLL; ++u) {
      const int idx = (int)(mv[u] >> mshift);
#pragma unroll
      for (int j = 0; j < MB; ++j)
        acc[0][j] = smfmac16x16x64(as_bf16x8(av[u]), cat16(as_bf16x8(xv[u][j][0]), as_bf16x8(xv[u][j][1])),
                                   acc[0][j], idx);
    }
  }

  // fixed-order combination of the waves' partial sums
  if (wave > 0) {
#pragma unroll
    for (int j = 0; j < MB; ++j) red[((wave - 1) * MB + j) * 64 + lane] = acc[0][j];
  }
  __syncthreads();
  if (wave != 0) return;
#pragma unroll
  for (int w = 1; w < KW; ++w)
#pragma unroll
    for (int j = 0; j < MB; ++j) acc[0][j] += red[((w - 1) * MB + j) * 64 + lane];

  if (r > 0) lowrank_epilogue<1, MB>(acc, U, Tpart, ksplit, M, n_out, r, n0, m0, lane);
  store_tile<1, MB>(acc, Y, M, n_out, n0, m0, lane);
}

template <int MB>
hipError_t launch_decode(const void* X, int64_t M, int64_t n_in, const void* values, const uint32_t* meta,
                         int64_t n_out, const void* U, int64_t r, const float* Tpart, int ksplit, float* Y,
                         hipStream_t stream) {
  constexpr int KW = 8, UNROLL = 2;
  dim3 grid((unsigned)ceil_div(n_out, 16), (unsigned)ceil_div(M, 16 * MB));
  linear_decode_kernel<KW, MB, UNROLL><<<grid, dim3(64 * KW), 0, stream>>>(
      (const uint16_t*)X, (const uint16_t*)values, meta, (const uint16_t*)U, Tpart, Y, (int)M, (int)n_in,
      (int)n_out, (int)r, ksplit);
  return hipGetLastError();
}

}  // namespace

hipError_t launch_linear_bf16(const void* X, int64_t M, int64_t n_in, const void* values, const uint32_t* meta,
                              int64_t n_out, const void* U, int64_t r, const float* Tpart, int ksplit, float* Y,
                              hipStream_t stream) {
  if (M <= 16) return launch_decode<1>(X, M, n_in, values, meta, n_out, U, r, Tpart, ksplit, Y, stream);
  if (M <= 32) return launch_decode<2>(X, M, n_in, values, meta, n_out, U, r, Tpart, ksplit, Y, stream);
  if (M <= kDecodeMaxTokens) return launch_decode<4>(X, M, n_in, values, meta, n_out, U, r, Tpart, ksplit, Y, stream);

  constexpr int BN = 128, BM = 128, WN = 64, WM = 64;
  using C = PrefillCfg<BN, BM, WN, WM>;
  const int tiles_n = (int)ceil_div(n_out, BN), tiles_m = (int)ceil_div(M, BM);
  const int n_tiles = tiles_n * tiles_m;
  const int per_xcd = (int)ceil_div(n_tiles, 8);
  const int group_m = 4;
  linear_prefill_kernel<BN, BM, WN, WM><<<dim3((unsigned)(8 * per_xcd)), dim3(C::kThreads), 0, stream>>>(
      (const uint16_t*)X, (const uint16_t*)values, meta, (const uint16_t*)U, Tpart, Y, (int)M, (int)n_in,
      (int)n_out, (int)r, ksplit, tiles_n, tiles_m, per_xcd, group_m);
  return hipGetLastError();
}

}  // namespace splr
