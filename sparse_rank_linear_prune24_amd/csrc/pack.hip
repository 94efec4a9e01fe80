// 2:4 projection + pack on gfx950.
//
// Hard thresholding per group of four (HASSLE-free page, §4.1.1; the 2:4 constraint as in the
// 3BASiL article, "A three-block ADMM replaces alternating minimization"): keep the two entries of
// largest magnitude as bit copies, ties to the lower column.
//
// Activation-aware variant (HASSLE-free page, §4.1.2: with a diagonal Hessian the residual is
// hard-thresholded after scaling column k by d_k, Wanda's score): the keys are |x| * |d_k|, formed
// as a binary64 product, which is exact for binary32 (and bfloat16) factors; NaN scores are made
// one canonical value, so they tie and outrank every number. The kept entries are R's own.
//
// HBM streaming kernel. A workgroup owns 16 rows x 1 KiB of R (eight bf16 tiles or four fp32
// tiles of the packed layout). Each lane reads 16-byte chunks with row-contiguous, fully
// coalesced loads, ranks the four entries of each group with six integer compares of keys (the
// sign-cleared bit patterns, or the bit patterns of the exact binary64 scores: bit-exact either way),
// and scatters its kept pair into the tile image in LDS; the lanes that share a metadata word
// merge their nibbles with cross-lane shuffles. The finished tiles leave LDS as contiguous
// 16-byte stores.
#include "common.hpp"
#include "kernels.hpp"

namespace splr {
namespace {

constexpr int kPackThreads = 256;
constexpr int kPackChunksPerThread = 4;  // 16-byte chunks of R per thread

// Activation-aware key: |x| * |d| exactly (binary64; dmag = |d| as binary64), NaN canonical;
// compared as unsigned integers.
__device__ __forceinline__ uint64_t scaled_key(float x, double dmag) {
  const double p = (double)fabsf(x) * dmag;
  return p != p ? 0x7FF8000000000000ull : (uint64_t)__double_as_longlong(p);
}

template <bool BF16, bool SCALED, int CPT>
__global__ __launch_bounds__(kPackThreads) void prune24_pack_kernel(const uint8_t* __restrict__ R,
                                                                    const float* __restrict__ dscale, int n_out, int K,
                                                                    int TK, u32x4_t* __restrict__ values,
                                                                    uint32_t* __restrict__ meta) {
  constexpr int kEsz = BF16 ? 2 : 4;            // bytes per entry
  constexpr int kPerChunk = 16 / kEsz;          // entries per 16-byte chunk (8 bf16 = 2 groups, 4 fp32 = 1)
  constexpr int kRowChunks = 16 * CPT;          // 16-byte chunks per row: CPT per thread over 16 rows
  constexpr int kCols = kRowChunks * kPerChunk; // columns per workgroup
  constexpr int kTiles = kCols / 64;            // packed tiles per workgroup
  constexpr int kTileU4 = 512 * kEsz / 16;      // 16-byte units of values per tile (64 / 128)
  static_assert((kRowChunks & (kRowChunks - 1)) == 0 && kTiles >= 1, "power-of-two row chunks, whole tiles");
  __shared__ u32x4_t sv[kTiles * kTileU4];
  __shared__ uint32_t sm[kTiles * 32];

  const int tr = blockIdx.x;                    // tile row
  const int tk0 = blockIdx.y * kTiles;          // first tile column of this workgroup
  const int tid = threadIdx.x;

  // a thread's chunks are rows tid / kRowChunks + 4c of one column chunk (kPackThreads is a
  // multiple of kRowChunks), so they share their column scales
  static_assert(kPackThreads % kRowChunks == 0, "a thread's chunks share their columns");
  u32x4_t x[CPT];
  bool valid[CPT];
#pragma unroll
  for (int c = 0; c < CPT; ++c) {
    const int q = tid + c * kPackThreads;
    const int r = q / kRowChunks, ch = q % kRowChunks;
    const int n = tr * 16 + r;
    const int k = blockIdx.y * kCols + ch * kPerChunk;
    valid[c] = n < n_out && k < K;
    x[c] = valid[c] ? __builtin_nontemporal_load((const u32x4_t*)(R + ((size_t)n * K + k) * kEsz))
                    : u32x4_t{0, 0, 0, 0};
  }
  // column scales of the thread's chunk as float64 magnitudes (SCALED only)
  double dmag[kPerChunk];
  if constexpr (SCALED) {
    const int k = blockIdx.y * kCols + (tid % kRowChunks) * kPerChunk;
#pragma unroll
    for (int h = 0; h < kPerChunk / 4; ++h) {
      const f32x4_t d4 = k < K ? *(const f32x4_t*)(dscale + k + 4 * h) : f32x4_t{0, 0, 0, 0};
#pragma unroll
      for (int e = 0; e < 4; ++e) dmag[4 * h + e] = (double)fabsf(d4[e]);
    }
  }
#pragma unroll
  for (int c = 0; c < CPT; ++c) {
    const int q = tid + c * kPackThreads;
    const int r = q / kRowChunks, ch = q % kRowChunks;
    uint32_t word;  // this chunk's nibbles, merged below into metadata words
    if constexpr (BF16) {
      // chunk = groups gi0, gi0+1 of tile tkl (gi0 even)
      const int tkl = ch >> 3, gi0 = 2 * (ch & 7);
      uint32_t v[4];
      const uint32_t d0 = x[c][0], d1 = x[c][1], d2 = x[c][2], d3 = x[c][3];
      uint32_t n0, n1;
      if constexpr (SCALED) {
        auto key = [](uint32_t bits16, double s) { return scaled_key(__uint_as_float(bits16 << 16), s); };
        n0 = top2_of_4(key(d0 & 0xFFFFu, dmag[0]), key(d0 >> 16, dmag[1]), key(d1 & 0xFFFFu, dmag[2]),
                       key(d1 >> 16, dmag[3]), d0 & 0xFFFFu, d0 >> 16, d1 & 0xFFFFu, d1 >> 16, v[0], v[1]);
        n1 = top2_of_4(key(d2 & 0xFFFFu, dmag[4]), key(d2 >> 16, dmag[5]), key(d3 & 0xFFFFu, dmag[6]),
                       key(d3 >> 16, dmag[7]), d2 & 0xFFFFu, d2 >> 16, d3 & 0xFFFFu, d3 >> 16, v[2], v[3]);
      } else {
        n0 = top2_of_4(d0 & 0x7FFFu, (d0 >> 16) & 0x7FFFu, d1 & 0x7FFFu, (d1 >> 16) & 0x7FFFu, d0 & 0xFFFFu, d0 >> 16,
                       d1 & 0xFFFFu, d1 >> 16, v[0], v[1]);
        n1 = top2_of_4(d2 & 0x7FFFu, (d2 >> 16) & 0x7FFFu, d3 & 0x7FFFu, (d3 >> 16) & 0x7FFFu, d2 & 0xFFFFu, d2 >> 16,
                       d3 & 0xFFFFu, d3 >> 16, v[2], v[3]);
      }
      if (!valid[c]) n0 = n1 = 0;  // padding: zero entries (already zero) and zero nibbles
      const int slot = r + 16 * (gi0 >> 2);
      // 4 entries (8 bytes) at entry 2*(gi0 % 4) of the slot: half (gi0 % 4) / 2 of its 16 bytes
      u32x2_t* dst = (u32x2_t*)&sv[tkl * kTileU4 + slot] + ((gi0 & 3) >> 1);
      *dst = u32x2_t{v[0] | (v[1] << 16), v[2] | (v[3] << 16)};
      // byte (gi0 % 8) / 2 of word (gi0 / 8) of row r: the four lanes ch % 4 = 0..3 share it
      word = n0 | (n1 << 4);
      word |= (uint32_t)__shfl_down((int)word, 1) << 8;
      word |= (uint32_t)__shfl_down((int)word, 2) << 16;
      if ((ch & 3) == 0) sm[tkl * 32 + (gi0 >> 3) * 16 + r] = word;
    } else {
      // chunk = group gi of tile tkl
      const int tkl = ch >> 4, gi = ch & 15;
      const uint32_t e0 = x[c][0], e1 = x[c][1], e2 = x[c][2], e3 = x[c][3];
      uint32_t va, vb, nb;
      if constexpr (SCALED) {
        nb = top2_of_4(scaled_key(__uint_as_float(e0), dmag[0]), scaled_key(__uint_as_float(e1), dmag[1]),
                       scaled_key(__uint_as_float(e2), dmag[2]), scaled_key(__uint_as_float(e3), dmag[3]), e0, e1,
                       e2, e3, va, vb);
      } else {
        nb = top2_of_4(e0 & 0x7FFFFFFFu, e1 & 0x7FFFFFFFu, e2 & 0x7FFFFFFFu, e3 & 0x7FFFFFFFu, e0, e1, e2, e3, va, vb);
      }
      if (!valid[c]) nb = 0;
      const int slot = r + 16 * (gi >> 2);
      u32x2_t* dst = (u32x2_t*)&sv[tkl * kTileU4 + 2 * slot] + (gi & 3);
      *dst = u32x2_t{va, vb};
      // nibble gi % 8 of word gi / 8 of row r: the eight lanes ch % 8 = 0..7 share it
      word = nb;
      word |= (uint32_t)__shfl_down((int)word, 1) << 4;
      word |= (uint32_t)__shfl_down((int)word, 2) << 8;
      word |= (uint32_t)__shfl_down((int)word, 4) << 16;
      if ((ch & 7) == 0) sm[tkl * 32 + (gi >> 3) * 16 + r] = word;
    }
  }
  __syncthreads();
  // tiles (tr, tk0 .. tk0 + kTiles - 1) are contiguous in the packed arrays
  const size_t t0 = (size_t)tr * TK + tk0;
  const int n_tiles = min(kTiles, TK - tk0);
#pragma unroll
  for (int u = tid; u < kTiles * kTileU4; u += kPackThreads)
    if (u < n_tiles * kTileU4) values[t0 * kTileU4 + u] = sv[u];
  if (tid < n_tiles * 8) ((u32x4_t*)meta)[t0 * 8 + tid] = ((const u32x4_t*)sm)[tid];
}

template <bool SCALED>
hipError_t launch_pack(const void* R, const float* d, int64_t n_out, int64_t n_in, bool bf16, void* values,
                       uint32_t* meta, hipStream_t stream) {
  constexpr int CPT = kPackChunksPerThread;
  const int TK = (int)ceil_div(n_in, 64);
  const int cols = 16 * CPT * (bf16 ? 8 : 4);
  dim3 grid((unsigned)ceil_div(n_out, 16), (unsigned)ceil_div(n_in, cols));
  if (bf16)
    prune24_pack_kernel<true, SCALED, CPT><<<grid, dim3(kPackThreads), 0, stream>>>(
        (const uint8_t*)R, d, (int)n_out, (int)n_in, TK, (u32x4_t*)values, meta);
  else
    prune24_pack_kernel<false, SCALED, CPT><<<grid, dim3(kPackThreads), 0, stream>>>(
        (const uint8_t*)R, d, (int)n_out, (int)n_in, TK, (u32x4_t*)values, meta);
  return hipGetLastError();
}

}  // namespace

hipError_t launch_prune24_pack(const void* R, int64_t n_out, int64_t n_in, bool bf16, void* values,
                               uint32_t* meta, hipStream_t stream) {
  return launch_pack<false>(R, nullptr, n_out, n_in, bf16, values, meta, stream);
}

hipError_t launch_prune24_pack_scaled(const void* R, const float* d, int64_t n_out, int64_t n_in, bool bf16,
                                      void* values, uint32_t* meta, hipStream_t stream) {
  return launch_pack<true>(R, d, n_out, n_in, bf16, values, meta, stream);
}

}  // namespace splr
