// Fused residual + 2:4 projection + pack on gfx950.
//
// The sparse step of the alternating-minimisation / ADMM decompositions acts on the weight minus
// the current low-rank part, R = W - U V (HASSLE-free page, §4 and §4.1.1), and projects it onto the
// 2:4 set (3BASiL article, "A three-block ADMM replaces alternating minimization"). This kernel
// forms R in registers and packs it, so R never goes to memory. The arithmetic is pinned so the
// result is bit-exact: per entry acc = W[n][k], then acc = fma(-U[n][j], V[j][k], acc) for
// j = 0, 1, ..., r-1 in binary32 (one rounding per step), then rounding to the storage type
// (bfloat16: to nearest even); a NaN result is stored as the canonical quiet NaN.
//
// Vector-ALU bound (r fused multiply-adds per weight; matrix cores cannot keep the sequential
// rounding order). A workgroup of 4 waves takes a run of 16-row tile rows; each wave owns 256
// columns (lane l: columns 4l .. 4l+3, one group of four), keeps V's 64 x 4 block of its columns in
// registers as float32 (for r <= 64 once per workgroup) and reads U (staged per tile row and rank
// block in LDS as float32, shared by the 4 waves) with broadcast LDS reads. Rows run one at a time;
// for r > 64 a row's running sums wait in LDS between rank blocks. Each rounded row is selected
// and written into a per-wave LDS image of the 4 packed tiles, which leaves with contiguous 16-byte
// stores.
#include <algorithm>

#include "common.hpp"
#include "kernels.hpp"

namespace splr {
namespace {

constexpr int kResWaves = 4;
constexpr int kRJ = 64;  // ranks whose V block a lane holds in registers at a time

template <bool BF16>
__device__ __forceinline__ float load_elem(const void* base, size_t i) {
  if constexpr (BF16) return __uint_as_float((uint32_t)((const uint16_t*)base)[i] << 16);
  else return ((const float*)base)[i];
}

// four consecutive elements starting at i (8- or 16-byte aligned)
template <bool BF16>
__device__ __forceinline__ void load4(const void* base, size_t i, float (&x)[4]) {
  if constexpr (BF16) {
    const u32x2_t w = *(const u32x2_t*)((const uint16_t*)base + i);
    x[0] = __uint_as_float(w[0] << 16);
    x[1] = __uint_as_float(w[0] & 0xFFFF0000u);
    x[2] = __uint_as_float(w[1] << 16);
    x[3] = __uint_as_float(w[1] & 0xFFFF0000u);
  } else {
    const f32x4_t w = *(const f32x4_t*)((const float*)base + i);
    x[0] = w[0];
    x[1] = w[1];
    x[2] = w[2];
    x[3] = w[3];
  }
}

// residual entry -> storage bits: NaN canonical, bfloat16 rounded to nearest even
template <bool BF16>
__device__ __forceinline__ uint32_t storage_bits(float acc) {
  const uint32_t u = __float_as_uint(acc);
  const bool nan = (u & 0x7FFFFFFFu) > 0x7F800000u;
  if constexpr (BF16) return nan ? 0x7FC0u : (u + 0x7FFFu + ((u >> 16) & 1u)) >> 16;
  else return nan ? 0x7FC00000u : u;
}

template <bool BF16>
__global__ __launch_bounds__(64 * kResWaves) void residual_pack_kernel(
    const void* __restrict__ W, const void* __restrict__ U, const void* __restrict__ V, int n_out, int K, int r,
    int TK, int TR, int tile_rows_per_wg, u32x4_t* __restrict__ values, uint32_t* __restrict__ meta) {
  constexpr int kTileU32 = BF16 ? 256 : 512;  // one packed tile's values in 32-bit words
  __shared__ f32x4_t us[16 * kRJ / 4];        // U rows of the tile row, one rank block, float32
  __shared__ uint32_t img[kResWaves][4 * kTileU32];
  __shared__ uint32_t mimg[kResWaves][4 * 32];
  __shared__ f32x4_t accl[kResWaves][16][64];  // running sums between rank blocks (r > kRJ)

  const int lane = threadIdx.x & 63, wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int col_block = (blockIdx.x * kResWaves + wave) * 256;  // this wave's first column
  const int c0 = col_block + 4 * lane;
  const bool col_ok = c0 < K;
  const int cc = col_ok ? c0 : 0;  // clamped column for loads
  const int tl = lane >> 4, gi = lane & 15;
  const int tr_begin = blockIdx.y * tile_rows_per_wg, tr_end = min(TR, tr_begin + tile_rows_per_wg);
  const bool single = r <= kRJ;

  float v[kRJ][4];
  auto load_v = [&](int jb) {
#pragma unroll
    for (int j = 0; j < kRJ; ++j) load4<BF16>(V, (size_t)min(jb + j, max(r - 1, 0)) * K + cc, v[j]);
  };
  // the fused multiply-adds of ranks jb .. jb + nj - 1 for row i of the staged block, in rank order
  auto fma_block = [&](float (&a)[4], int i, int nj) {
    if (nj == kRJ) {
#pragma unroll
      for (int j4 = 0; j4 < kRJ / 4; ++j4) {
        const f32x4_t u = us[i * (kRJ / 4) + j4];
#pragma unroll
        for (int t = 0; t < 4; ++t)
#pragma unroll
          for (int c = 0; c < 4; ++c) a[c] = __builtin_fmaf(-u[t], v[4 * j4 + t][c], a[c]);
      }
    } else {  // partial block: exactly nj steps (a padding step is not neutral)
#pragma unroll
      for (int j4 = 0; j4 < kRJ / 4; ++j4) {
        const f32x4_t u = us[i * (kRJ / 4) + j4];
#pragma unroll
        for (int t = 0; t < 4; ++t)
          if (4 * j4 + t < nj) {  // wave-uniform
#pragma unroll
            for (int c = 0; c < 4; ++c) a[c] = __builtin_fmaf(-u[t], v[4 * j4 + t][c], a[c]);
          }
      }
    }
  };
  // round row i, select the top two of each group, write it into this wave's LDS image of 4 tiles
  auto select_row = [&](const float (&a)[4], int i, bool row_ok) {
    const bool ok = col_ok && row_ok;
    uint32_t e[4];
#pragma unroll
    for (int c = 0; c < 4; ++c) e[c] = ok ? storage_bits<BF16>(a[c]) : 0u;
    const uint32_t m = BF16 ? 0x7FFFu : 0x7FFFFFFFu;
    uint32_t va, vb;
    uint32_t nib = top2_of_4(e[0] & m, e[1] & m, e[2] & m, e[3] & m, e[0], e[1], e[2], e[3], va, vb);
    if (!ok) nib = 0;
    const int slot = i + 16 * (gi >> 2);
    if constexpr (BF16) {
      img[wave][tl * kTileU32 + slot * 4 + (gi & 3)] = va | (vb << 16);
    } else {
      *(u32x2_t*)&img[wave][tl * kTileU32 + slot * 8 + 2 * (gi & 3)] = u32x2_t{va, vb};
    }
    // nibble gi % 8 of word gi / 8 of row i: the eight lanes gi % 8 = 0..7 share it
    uint32_t word = nib;
    word |= (uint32_t)__shfl_down((int)word, 1) << 4;
    word |= (uint32_t)__shfl_down((int)word, 2) << 8;
    word |= (uint32_t)__shfl_down((int)word, 4) << 16;
    if ((gi & 7) == 0) mimg[wave][tl * 32 + (gi >> 3) * 16 + i] = word;
  };

  if (r > 0 && single) load_v(0);
  for (int tr = tr_begin; tr < tr_end; ++tr) {
    if (r == 0) {
#pragma unroll 1
      for (int i = 0; i < 16; ++i) {
        float a[4];
        load4<BF16>(W, (size_t)min(tr * 16 + i, n_out - 1) * K + cc, a);
        select_row(a, i, tr * 16 + i < n_out);
      }
    }
    for (int jb = 0; jb < r; jb += kRJ) {
      const int nj = min(kRJ, r - jb);
      const bool last = jb + nj >= r;
      __syncthreads();  // every wave is done reading the previous block of U
      for (int q = threadIdx.x; q < 16 * kRJ; q += 64 * kResWaves) {
        const int i = q / kRJ, j = q % kRJ;
        ((float*)us)[q] = j < nj ? load_elem<BF16>(U, (size_t)min(tr * 16 + i, n_out - 1) * r + jb + j) : 0.0f;
      }
      __syncthreads();
      if (!single) load_v(jb);
#pragma unroll 1
      for (int i = 0; i < 16; ++i) {
        float a[4];
        if (jb == 0) {
          load4<BF16>(W, (size_t)min(tr * 16 + i, n_out - 1) * K + cc, a);
        } else {
          const f32x4_t p = accl[wave][i][lane];
          a[0] = p[0], a[1] = p[1], a[2] = p[2], a[3] = p[3];
        }
        fma_block(a, i, nj);
        if (last) select_row(a, i, tr * 16 + i < n_out);
        else accl[wave][i][lane] = f32x4_t{a[0], a[1], a[2], a[3]};
      }
    }

    // tiles (tr, col_block / 64 + t) are contiguous in the packed arrays; this wave's LDS writes
    // are complete before its own reads below (LDS operations of one wave execute in order)
    const int tk0 = col_block / 64;
    constexpr int kTileU4 = kTileU32 / 4;
#pragma unroll
    for (int q = lane; q < 4 * kTileU4; q += 64) {
      const int t = q / kTileU4;
      if (tk0 + t < TK) values[((size_t)tr * TK + tk0 + t) * kTileU4 + q % kTileU4] = ((const u32x4_t*)img[wave])[q];
    }
    if (lane < 32) {
      const int t = lane / 8;
      if (tk0 + t < TK) ((u32x4_t*)meta)[((size_t)tr * TK + tk0 + t) * 8 + lane % 8] = ((const u32x4_t*)mimg[wave])[lane];
    }
  }
}

// r <= 64 (one register block of V): the same arithmetic with the memory latency hidden. W of the
// next tile row (raw storage bits) and its U block are loaded while the current tile row computes;
// the 16 rows of a tile row are unrolled, each selected as soon as its sums are complete.
template <bool BF16>
__global__ __launch_bounds__(64 * kResWaves) void residual_pack_r64_kernel(
    const void* __restrict__ W, const void* __restrict__ U, const void* __restrict__ V, int n_out, int K, int r,
    int TK, int TR, int tile_rows_per_wg, u32x4_t* __restrict__ values, uint32_t* __restrict__ meta) {
  constexpr int kTileU32 = BF16 ? 256 : 512;
  constexpr int kWRaw = BF16 ? 2 : 4;                       // 32-bit words of one row's 4 entries
  constexpr int kUPer = 16 * kRJ / (64 * kResWaves);       // U elements each thread stages per tile row
  __shared__ f32x4_t us[16 * kRJ / 4];
  __shared__ uint32_t img[kResWaves][4 * kTileU32];
  __shared__ uint32_t mimg[kResWaves][4 * 32];

  const int lane = threadIdx.x & 63, wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int col_block = (blockIdx.x * kResWaves + wave) * 256;
  const int c0 = col_block + 4 * lane;
  const bool col_ok = c0 < K;
  const int cc = col_ok ? c0 : 0;
  const int tl = lane >> 4, gi = lane & 15;
  const int tr_begin = blockIdx.y * tile_rows_per_wg, tr_end = min(TR, tr_begin + tile_rows_per_wg);
  if (tr_begin >= tr_end) return;  // uniform over the workgroup

  float v[kRJ][4];
#pragma unroll
  for (int j = 0; j < kRJ; ++j) load4<BF16>(V, (size_t)min(j, r - 1) * K + cc, v[j]);

  uint32_t wraw[16][kWRaw];
  float unext[kUPer];
  auto load_w = [&](int tr) {
#pragma unroll
    for (int i = 0; i < 16; ++i) {
      const uint32_t* p = (const uint32_t*)W + ((size_t)min(tr * 16 + i, n_out - 1) * K + cc) * (BF16 ? 2 : 4) / 4;
      if constexpr (BF16) {
        const u32x2_t w = *(const u32x2_t*)p;
        wraw[i][0] = w[0], wraw[i][1] = w[1];
      } else {
        const u32x4_t w = *(const u32x4_t*)p;
        wraw[i][0] = w[0], wraw[i][1] = w[1], wraw[i][2] = w[2], wraw[i][3] = w[3];
      }
    }
  };
  auto load_u = [&](int tr) {
#pragma unroll
    for (int t = 0; t < kUPer; ++t) {
      const int q = threadIdx.x + t * 64 * kResWaves, i = q / kRJ, j = q % kRJ;
      unext[t] = j < r ? load_elem<BF16>(U, (size_t)min(tr * 16 + i, n_out - 1) * r + j) : 0.0f;
    }
  };
  auto stage_u = [&]() {
#pragma unroll
    for (int t = 0; t < kUPer; ++t) ((float*)us)[threadIdx.x + t * 64 * kResWaves] = unext[t];
  };

  load_u(tr_begin);
  stage_u();
  load_w(tr_begin);
  __syncthreads();
  for (int tr = tr_begin; tr < tr_end; ++tr) {
    const bool more = tr + 1 < tr_end;
    if (more) load_u(tr + 1);  // in flight during this tile row
#pragma unroll
    for (int i = 0; i < 16; ++i) {
      float a[4];
      if constexpr (BF16) {
        a[0] = __uint_as_float(wraw[i][0] << 16), a[1] = __uint_as_float(wraw[i][0] & 0xFFFF0000u);
        a[2] = __uint_as_float(wraw[i][1] << 16), a[3] = __uint_as_float(wraw[i][1] & 0xFFFF0000u);
      } else {
        a[0] = __uint_as_float(wraw[i][0]), a[1] = __uint_as_float(wraw[i][1]);
        a[2] = __uint_as_float(wraw[i][2]), a[3] = __uint_as_float(wraw[i][3]);
      }
      if (r == kRJ) {
#pragma unroll
        for (int j4 = 0; j4 < kRJ / 4; ++j4) {
          const f32x4_t u = us[i * (kRJ / 4) + j4];
#pragma unroll
          for (int t = 0; t < 4; ++t)
#pragma unroll
            for (int c = 0; c < 4; ++c) a[c] = __builtin_fmaf(-u[t], v[4 * j4 + t][c], a[c]);
        }
      } else {
#pragma unroll
        for (int j4 = 0; j4 < kRJ / 4; ++j4) {
          const f32x4_t u = us[i * (kRJ / 4) + j4];
#pragma unroll
          for (int t = 0; t < 4; ++t)
            if (4 * j4 + t < r) {  // wave-uniform
#pragma unroll
              for (int c = 0; c < 4; ++c) a[c] = __builtin_fmaf(-u[t], v[4 * j4 + t][c], a[c]);
            }
        }
      }
      const bool ok = col_ok && tr * 16 + i < n_out;
      uint32_t e[4];
#pragma unroll
      for (int c = 0; c < 4; ++c) e[c] = ok ? storage_bits<BF16>(a[c]) : 0u;
      const uint32_t m = BF16 ? 0x7FFFu : 0x7FFFFFFFu;
      uint32_t va, vb;
      uint32_t nib = top2_of_4(e[0] & m, e[1] & m, e[2] & m, e[3] & m, e[0], e[1], e[2], e[3], va, vb);
      if (!ok) nib = 0;
      const int slot = i + 16 * (gi >> 2);
      if constexpr (BF16) {
        img[wave][tl * kTileU32 + slot * 4 + (gi & 3)] = va | (vb << 16);
      } else {
        *(u32x2_t*)&img[wave][tl * kTileU32 + slot * 8 + 2 * (gi & 3)] = u32x2_t{va, vb};
      }
      uint32_t word = nib;
      word |= (uint32_t)__shfl_down((int)word, 1) << 4;
      word |= (uint32_t)__shfl_down((int)word, 2) << 8;
      word |= (uint32_t)__shfl_down((int)word, 4) << 16;
      if ((gi & 7) == 0) mimg[wave][tl * 32 + (gi >> 3) * 16 + i] = word;
    }
    if (more) load_w(tr + 1);  // the raw W of this tile row is consumed
    const int tk0 = col_block / 64;
    constexpr int kTileU4 = kTileU32 / 4;
#pragma unroll
    for (int q = lane; q < 4 * kTileU4; q += 64) {
      const int t = q / kTileU4;
      if (tk0 + t < TK) values[((size_t)tr * TK + tk0 + t) * kTileU4 + q % kTileU4] = ((const u32x4_t*)img[wave])[q];
    }
    if (lane < 32) {
      const int t = lane / 8;
      if (tk0 + t < TK) ((u32x4_t*)meta)[((size_t)tr * TK + tk0 + t) * 8 + lane % 8] = ((const u32x4_t*)mimg[wave])[lane];
    }
    __syncthreads();  // every wave is done with this tile row's U
    if (more) stage_u();
    __syncthreads();
  }
}

}  // namespace

hipError_t launch_prune24_pack_residual(const void* W, const void* U, const void* V, int64_t n_out, int64_t n_in,
                                        int64_t r, bool bf16, void* values, uint32_t* meta, hipStream_t stream) {
  const int TK = (int)ceil_div(n_in, 64), TR = (int)ceil_div(n_out, 16);
  const int col_groups = (int)ceil_div(n_in, 256 * kResWaves);
  // about 512 workgroups; each takes a run of tile rows (V stays in registers across the run)
  const int tile_rows = (int)std::max<int64_t>(1, ceil_div((int64_t)TR * col_groups, 512));
  dim3 grid((unsigned)col_groups, (unsigned)ceil_div(TR, tile_rows));
  if (r >= 1 && r <= kRJ) {
    if (bf16)
      residual_pack_r64_kernel<true><<<grid, dim3(64 * kResWaves), 0, stream>>>(
          W, U, V, (int)n_out, (int)n_in, (int)r, TK, TR, tile_rows, (u32x4_t*)values, meta);
    else
      residual_pack_r64_kernel<false><<<grid, dim3(64 * kResWaves), 0, stream>>>(
          W, U, V, (int)n_out, (int)n_in, (int)r, TK, TR, tile_rows, (u32x4_t*)values, meta);
  } else if (bf16) {
    residual_pack_kernel<true><<<grid, dim3(64 * kResWaves), 0, stream>>>(
        W, U, V, (int)n_out, (int)n_in, (int)r, TK, TR, tile_rows, (u32x4_t*)values, meta);
  } else {
    residual_pack_kernel<false><<<grid, dim3(64 * kResWaves), 0, stream>>>(
        W, U, V, (int)n_out, (int)n_in, (int)r, TK, TR, tile_rows, (u32x4_t*)values, meta);
  }
  return hipGetLastError();
}

}  // namespace splr
