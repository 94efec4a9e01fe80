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
// rounding order). Columns per lane: a wave owns kResColsPerLane 64-column packed tiles of one
// tile row (lane l: column l of each), a workgroup of 4 waves the neighbouring tiles. Each lane
// keeps its columns' 16 running sums and, per block of kRJ ranks, its columns of V in registers;
// U for the tile row and the rank block is staged in LDS as float32 and read with broadcast reads
// (one read feeds 4 ranks of every column of the lane). A broadcast 16-byte read still returns
// 1 KiB per wave through the LDS data path, so with one column per lane that path, not the FMAs,
// sets the pace; two columns halve the LDS bytes per FMA. Registers stay low enough for three
// waves per SIMD, which hide each other's LDS and memory latency.
// The rounded rows of a tile pass through LDS so that each lane selects whole groups (four rows'
// worth of groups per lane instead of every lane of a group repeating the selection); the kept
// pairs and nibbles form a per-wave LDS image of the packed tile, which leaves with contiguous
// 16-byte stores.
#include <algorithm>

#include "common.hpp"
#include "kernels.hpp"

namespace splr {
namespace {

constexpr int kResWaves = 4;
constexpr int kRJ = 32;   // ranks per block (a lane's column of V for the block sits in registers)
constexpr int kResColsPerLane = 2;  // columns (tiles) per lane (wave)

template <bool BF16>
__device__ __forceinline__ float load_elem(const void* base, size_t i) {
  if constexpr (BF16) return __uint_as_float((uint32_t)((const uint16_t*)base)[i] << 16);
  else return ((const float*)base)[i];
}

// residual entry -> storage bits: NaN canonical, bfloat16 rounded to nearest even
template <bool BF16>
__device__ __forceinline__ uint32_t storage_bits(float acc) {
  const uint32_t u = __float_as_uint(acc);
  const bool nan = (u & 0x7FFFFFFFu) > 0x7F800000u;
  if constexpr (BF16) return nan ? 0x7FC0u : (u + 0x7FFFu + ((u >> 16) & 1u)) >> 16;
  else return nan ? 0x7FC00000u : u;
}

// acc[s][i] = fma(-U[row i][j], V[j][column s], acc[s][i]) for j = 0 .. NJ-1 in order, U from the
// staged block `us` (16 rows x kRJ ranks, float32), V from registers
template <int NJ, int CPL>
__device__ __forceinline__ void fma_block(float (&acc)[CPL][16], const float (&v)[CPL][kRJ], const f32x4_t* us) {
#pragma unroll
  for (int i = 0; i < 16; ++i)
#pragma unroll
    for (int j4 = 0; j4 < NJ / 4; ++j4) {
      const f32x4_t u = us[i * (kRJ / 4) + j4];
#pragma unroll
      for (int q = 0; q < 4; ++q)
#pragma unroll
        for (int s = 0; s < CPL; ++s) acc[s][i] = __builtin_fmaf(-u[q], v[s][4 * j4 + q], acc[s][i]);
    }
}

// the same for ranks J0 .. J0 + nb - 1 (nb < 16)
template <int J0, int CPL>
__device__ __forceinline__ void fma_tail(float (&acc)[CPL][16], const float (&v)[CPL][kRJ], const f32x4_t* us,
                                         int nb) {
#pragma unroll
  for (int jj = 0; jj < 16; ++jj) {
    if (jj < nb) {  // uniform
#pragma unroll
      for (int i = 0; i < 16; ++i) {
        const float u = ((const float*)us)[i * kRJ + J0 + jj];
#pragma unroll
        for (int s = 0; s < CPL; ++s) acc[s][i] = __builtin_fmaf(-u, v[s][J0 + jj], acc[s][i]);
      }
    }
  }
}

// One-dimensional grid of tile rows x blocks of kResWaves * CPL tile columns, the column block
// varying fastest (workgroup b: column block b % col_blocks of tile row b / col_blocks). Lane l of
// wave w owns column l of tiles (column block * kResWaves + w) * CPL + s, s < CPL.
template <bool BF16, int CPL>
__global__ __launch_bounds__(64 * kResWaves) void residual_pack_kernel(
    const void* __restrict__ W, const void* __restrict__ U, const void* __restrict__ V, int n_out, int K, int r,
    int TK, int TKB, int col_blocks, u32x4_t* __restrict__ values, uint32_t* __restrict__ meta) {
  static_assert(kResWaves * CPL == 8, "a workgroup's tiles are one metadata block");
  constexpr int kTileU32 = BF16 ? 256 : 512;  // one packed tile's values in 32-bit words
  __shared__ f32x4_t us[16 * kRJ / 4];        // U rows of the tile row, one rank block, float32
  __shared__ uint32_t img[kResWaves][kTileU32];
  __shared__ uint16_t mimg[64 * 8];  // the block's metadata image: unit (slot L, tile t) at L * 8 + t
  __shared__ __align__(16) uint32_t ebuf[kResWaves][16 * 64];  // rounded rows of a tile (storage bits)

  const int lane = threadIdx.x & 63, wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int tr = blockIdx.x / col_blocks;
  const int tk0 = ((blockIdx.x - tr * col_blocks) * kResWaves + wave) * CPL;  // this wave's first tile column
  const size_t esz = BF16 ? 2 : 4;
  bool col_ok[CPL];
  int cc[CPL];
#pragma unroll
  for (int s = 0; s < CPL; ++s) {
    const int c = (tk0 + s) * 64 + lane;
    col_ok[s] = c < K;
    cc[s] = col_ok[s] ? c : K - 1;  // clamped column for loads
  }

  // running sums, initialised with W; row pointers advance by one row per step (rows past n_out
  // repeat the last)
  float acc[CPL][16];
  {
    const char* wp = (const char*)W + (size_t)min(tr * 16, n_out - 1) * K * esz;
#pragma unroll
    for (int i = 0; i < 16; ++i) {
#pragma unroll
      for (int s = 0; s < CPL; ++s) acc[s][i] = load_elem<BF16>(wp, cc[s]);
      if (tr * 16 + i + 1 < n_out) wp += (size_t)K * esz;
    }
  }

  for (int jb = 0; jb < r; jb += kRJ) {
    const int nj = min(kRJ, r - jb);
    __syncthreads();  // every wave is done reading the previous block of U
    for (int q = threadIdx.x; q < 16 * kRJ; q += 64 * kResWaves) {
      const int row = q / kRJ, j = q % kRJ;
      ((float*)us)[q] = j < nj ? load_elem<BF16>(U, (size_t)min(tr * 16 + row, n_out - 1) * r + jb + j) : 0.0f;
    }
    float v[CPL][kRJ];
    {
      const char* vp = (const char*)V + (size_t)jb * K * esz;
#pragma unroll
      for (int j = 0; j < kRJ; ++j) {
#pragma unroll
        for (int s = 0; s < CPL; ++s) v[s][j] = load_elem<BF16>(vp, cc[s]);
        if (j + 1 < nj) vp += (size_t)K * esz;  // ranks past r repeat the last (never used)
      }
    }
    __syncthreads();
    // exactly nj steps (a padding step is not neutral): whole 16-rank parts, then the rest
    const int nb = nj & 15;
    static_assert(kRJ == 32 || kRJ == 64, "rank block of 32 or 64");
    switch (nj >> 4) {
      case 4: if constexpr (kRJ == 64) fma_block<64, CPL>(acc, v, us); break;
      case 3: if constexpr (kRJ == 64) { fma_block<48, CPL>(acc, v, us); fma_tail<48, CPL>(acc, v, us, nb); } break;
      case 2: fma_block<32, CPL>(acc, v, us); if constexpr (kRJ == 64) fma_tail<32, CPL>(acc, v, us, nb); break;
      case 1: fma_block<16, CPL>(acc, v, us); fma_tail<16, CPL>(acc, v, us, nb); break;
      default: fma_tail<0, CPL>(acc, v, us, nb); break;
    }
  }

  // round, select the top two of each group, pack: tile (tr, tk0 + s) per column s. The rounded
  // rows go through the per-wave buffer `ebuf` so that each lane selects whole groups: item
  // m*64 + lane = row 4m + lane/16, group lane%16.
  constexpr uint32_t kMag = BF16 ? 0x7FFFu : 0x7FFFFFFFu;
  const int gg = lane & 15;
#pragma unroll
  for (int s = 0; s < CPL; ++s) {
#pragma unroll
    for (int i = 0; i < 16; ++i) {
      const bool ok = col_ok[s] && tr * 16 + i < n_out;
      ebuf[wave][i * 64 + lane] = ok ? storage_bits<BF16>(acc[s][i]) : 0u;
    }
    const bool gok = (tk0 + s) * 64 + 4 * gg < K;  // the group's columns exist (K is a multiple of 32)
#pragma unroll
    for (int m = 0; m < 4; ++m) {
      const int i = 4 * m + (lane >> 4);
      const u32x4_t e = *(const u32x4_t*)&ebuf[wave][i * 64 + 4 * gg];
      uint32_t va, vb;
      uint32_t nib = top2_of_4(e[0] & kMag, e[1] & kMag, e[2] & kMag, e[3] & kMag, e[0], e[1], e[2], e[3], va, vb);
      if (!gok || tr * 16 + i >= n_out) nib = 0;  // padding: zero entries (already zero) and zero nibbles
      const int slot = i + 16 * (gg >> 2);
      if constexpr (BF16) img[wave][slot * 4 + (gg & 3)] = va | (vb << 16);
      else *(u32x2_t*)&img[wave][slot * 8 + 2 * (gg & 3)] = u32x2_t{va, vb};
      // the unit of slot i + 16 (gg / 4) in this tile: nibble at bits 4 (gg % 4); the four lanes
      // gg % 4 = 0..3 share it
      uint32_t word = nib;
      word |= (uint32_t)__shfl_down((int)word, 1) << 4;
      word |= (uint32_t)__shfl_down((int)word, 2) << 8;
      if ((lane & 3) == 0) mimg[(i + 16 * (gg >> 2)) * 8 + wave * CPL + s] = (uint16_t)word;
    }
    // this wave's LDS writes are complete before its own reads below, and those before the next
    // tile's writes (LDS operations of one wave execute in order)
    const int tk = tk0 + s;
    if (tk < TK) {
      constexpr int kTileU4 = kTileU32 / 4;
#pragma unroll
      for (int q = lane; q < kTileU4; q += 64) values[((size_t)tr * TK + tk) * kTileU4 + q] = ((const u32x4_t*)img[wave])[q];
    }
  }
  // every wave's units are in the block image (tiles past TK hold zero nibbles); wave 0 stores
  // the block
  __syncthreads();
  if (wave == 0) {
    const int tb = (tk0 - wave * CPL) / 8;
    ((u32x4_t*)meta)[((size_t)tr * TKB + tb) * 64 + lane] = ((const u32x4_t*)mimg)[lane];
  }
}

}  // namespace

namespace {
int residual_col_blocks(int64_t n_in) { return (int)ceil_div(ceil_div(n_in, 64), kResWaves * kResColsPerLane); }
dim3 residual_grid(int64_t n_out, int64_t n_in) {
  return dim3((unsigned)(ceil_div(n_out, 16) * residual_col_blocks(n_in)));
}
}  // namespace

bool residual_grids_fit(int64_t n_out, int64_t n_in) {
  return grid_fits(residual_grid(n_out, n_in), 64 * kResWaves);
}

hipError_t launch_prune24_pack_residual(const void* W, const void* U, const void* V, int64_t n_out, int64_t n_in,
                                        int64_t r, bool bf16, void* values, uint32_t* meta, hipStream_t stream) {
  constexpr int CPL = kResColsPerLane;
  const int TK = (int)ceil_div(n_in, 64), TKB = (TK + 7) / 8, cb = residual_col_blocks(n_in);
  const dim3 grid = residual_grid(n_out, n_in);
  if (bf16)
    residual_pack_kernel<true, CPL><<<grid, dim3(64 * kResWaves), 0, stream>>>(W, U, V, (int)n_out, (int)n_in, (int)r,
                                                                              TK, TKB, cb, (u32x4_t*)values, meta);
  else
    residual_pack_kernel<false, CPL><<<grid, dim3(64 * kResWaves), 0, stream>>>(W, U, V, (int)n_out, (int)n_in,
                                                                               (int)r, TK, TKB, cb, (u32x4_t*)values, meta);
  return hipGetLastError();
}

}  // namespace splr
