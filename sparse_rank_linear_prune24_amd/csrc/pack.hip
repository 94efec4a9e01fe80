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
// N:M projection (HASSLE-free page, §1 and §2: N:M sparsity; 3BASiL article, "A three-block ADMM
// replaces alternating minimization": N:M structures such as 2:4, and the 2:8 configuration): in
// every group of M consecutive columns the n entries of largest magnitude are kept (ties to the
// lower column) and the rest become +0; the result then goes through the 2:4 selection and pack
// unchanged. For n <= 2 and 4 | M no aligned group of four holds more than two nonzeros, so the
// packed 2:4 operand is exactly the N:M matrix and the layer product runs on it as it is. A group
// that spans several 16-byte chunks lies in neighbouring lanes (a lane's chunk index along the row
// is its lane id), whose words are exchanged with cross-lane shuffles.
//
// HBM streaming kernel. A workgroup owns 16 rows x 1 KiB of R (eight bf16 tiles or four fp32
// tiles of the packed layout). Each lane reads 16-byte chunks with row-contiguous, fully
// coalesced loads, ranks the four entries of each group with six integer compares of keys (the
// sign-cleared bit patterns, or the bit patterns of the exact binary64 scores: bit-exact either way),
// and scatters its kept pair into the tile image in LDS; the lanes that share a 16-bit metadata
// unit merge their nibbles with cross-lane shuffles. A bf16 workgroup's 8 tiles are exactly one
// metadata block (8 tile columns of a tile row), an fp32 workgroup's 4 tiles half of one. The
// finished tiles and the block leave LDS as contiguous 16-byte (fp32 metadata: 8-byte) stores.
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

// N:M projection of one 16-byte chunk in place (group size M, n_keep kept per group). Every lane of
// the wave must call this (the shuffles read neighbouring lanes); `lane` is the chunk's index along
// its row within the wave's 64 chunks.
template <bool BF16, int M>
__device__ __forceinline__ void nm_project_chunk(u32x4_t& x, int n_keep, int lane) {
  constexpr int kPer = BF16 ? 8 : 4;                  // entries per chunk
  constexpr int kChunks = M > kPer ? M / kPer : 1;    // chunks (lanes) per group
  constexpr int kGroup = M < kPer ? M : kPer * kChunks;  // entries per group (= M)
  static_assert(kGroup == M && (kChunks & (kChunks - 1)) == 0 && 64 % kChunks == 0, "groups of whole lanes");
  // the group's words, in column order (this lane's own chunk at position lane % kChunks)
  uint32_t w[kChunks][4];
  const int base = lane & ~(kChunks - 1);
#pragma unroll
  for (int g = 0; g < kChunks; ++g)
#pragma unroll
    for (int i = 0; i < 4; ++i) w[g][i] = kChunks == 1 ? x[i] : (uint32_t)__shfl((int)x[i], base + g);
  auto key = [&](int g, int e) -> uint32_t {  // magnitude key of entry e of chunk g
    if constexpr (BF16) return (w[g][e >> 1] >> (16 * (e & 1))) & 0x7FFFu;
    else return w[g][e] & 0x7FFFFFFFu;
  };
  const int own = lane & (kChunks - 1);
  constexpr int kSeen = kChunks * kPer;  // entries the lane sees: its group, or the chunk's groups
  int above[kPer];                       // 0: outranks all others of its group; >= n_keep: dropped
  if constexpr (BF16) {
    // 15-bit keys: the value (key << 4) | (15 - position in the group) is unique within a group
    // and orders its entries exactly as "outranks" (larger key, then lower position), so the
    // first and second of a group are its largest and second-largest values
    static_assert(M <= 16, "4 position bits");
    uint32_t cv[kSeen];
#pragma unroll
    for (int t = 0; t < kSeen; ++t) cv[t] = (key(t / kPer, t % kPer) << 4) | (uint32_t)(15 - t % M);
#pragma unroll
    for (int e = 0; e < kPer; ++e) above[e] = 2;
#pragma unroll
    for (int g0 = 0; g0 < kSeen; g0 += M) {
      uint32_t m1 = cv[g0];
#pragma unroll
      for (int t = g0 + 1; t < g0 + M; ++t) m1 = max(m1, cv[t]);
      uint32_t m2 = 0;  // values are unique and a group has >= 4, so the second is > 0
#pragma unroll
      for (int t = g0; t < g0 + M; ++t) m2 = max(m2, cv[t] != m1 ? cv[t] : 0u);
      const uint32_t thr = n_keep == 1 ? m1 : m2;  // kept: the values >= the n-th largest
      // this lane's entries of the group
#pragma unroll
      for (int e = 0; e < kPer; ++e) {
        if (kChunks == 1 && (e < g0 || e >= g0 + M)) continue;  // compile-time
        const uint32_t c = (key(own, e) << 4) | (uint32_t)(15 - (kChunks == 1 ? e - g0 : own * kPer + e));
        above[e] = c >= thr ? 0 : 2;
      }
    }
  } else {
    // 31-bit keys: rank by one compare per unordered pair (the lower position i outranks j iff
    // k_i >= k_j, and the pair counts for one of the two)
    int rk[kSeen];
#pragma unroll
    for (int t = 0; t < kSeen; ++t) rk[t] = 0;
#pragma unroll
    for (int g0 = 0; g0 < kSeen; g0 += M)
#pragma unroll
      for (int i = g0; i < g0 + M; ++i)
#pragma unroll
        for (int j = i + 1; j < g0 + M; ++j) {
          const int c = key(i / kPer, i % kPer) >= key(j / kPer, j % kPer) ? 1 : 0;
          rk[j] += c;
          rk[i] += 1 - c;
        }
#pragma unroll
    for (int e = 0; e < kPer; ++e) {
      above[e] = rk[e];
#pragma unroll
      for (int g = 1; g < kChunks; ++g) above[e] = own == g ? rk[g * kPer + e] : above[e];
    }
  }
  uint32_t out[4] = {x[0], x[1], x[2], x[3]};
#pragma unroll
  for (int e = 0; e < kPer; ++e) {
    if (above[e] >= n_keep) {  // dropped: +0
      if constexpr (BF16) out[e >> 1] &= (e & 1) ? 0x0000FFFFu : 0xFFFF0000u;
      else out[e] = 0u;
    }
  }
  x = u32x4_t{out[0], out[1], out[2], out[3]};
}

// NM: 0 for the 2:4 projection, else the group size M of an N:M projection applied first
// (n_keep kept per group).
template <bool BF16, bool SCALED, int CPT, int NM = 0>
__global__ __launch_bounds__(kPackThreads) void prune24_pack_kernel(const uint8_t* __restrict__ R,
                                                                    const float* __restrict__ dscale, int n_out, int K,
                                                                    int TK, int TKB, u32x4_t* __restrict__ values,
                                                                    uint32_t* __restrict__ meta, int n_keep = 2) {
  constexpr int kEsz = BF16 ? 2 : 4;            // bytes per entry
  constexpr int kPerChunk = 16 / kEsz;          // entries per 16-byte chunk (8 bf16 = 2 groups, 4 fp32 = 1)
  constexpr int kRowChunks = 16 * CPT;          // 16-byte chunks per row: CPT per thread over 16 rows
  constexpr int kCols = kRowChunks * kPerChunk; // columns per workgroup
  constexpr int kTiles = kCols / 64;            // packed tiles per workgroup
  constexpr int kTileU4 = 512 * kEsz / 16;      // 16-byte units of values per tile (64 / 128)
  static_assert((kRowChunks & (kRowChunks - 1)) == 0 && kTiles >= 1, "power-of-two row chunks, whole tiles");
  static_assert(kTiles == 8 || kTiles == 4, "a metadata block or half of one per workgroup");
  __shared__ u32x4_t sv[kTiles * kTileU4];
  // metadata image: slot L's units for this workgroup's tiles, unit (L, t) at sm[L * kTiles + t]
  __shared__ uint16_t sm[64 * kTiles];

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
  if constexpr (NM > 0) {
    static_assert(!SCALED && kPackThreads % 64 == 0 && kRowChunks == 64, "a lane's chunk index is its lane id");
#pragma unroll
    for (int c = 0; c < CPT; ++c) nm_project_chunk<BF16, NM>(x[c], n_keep, tid & 63);
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
      // the unit of slot r + 16 (gi0 / 4) in tile tkl: groups 4q .. 4q+3, this chunk's two at
      // bits 4 (gi0 % 4); the lanes ch, ch + 1 (gi0 % 4 = 0, 2) share it
      word = n0 | (n1 << 4);
      word |= (uint32_t)__shfl_down((int)word, 1) << 8;
      if ((ch & 1) == 0) sm[(r + 16 * (gi0 >> 2)) * kTiles + tkl] = (uint16_t)word;
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
      // the unit of slot r + 16 (gi / 4) in tile tkl: nibble at bits 4 (gi % 4); the four lanes
      // ch % 4 = 0..3 share it
      word = nb;
      word |= (uint32_t)__shfl_down((int)word, 1) << 4;
      word |= (uint32_t)__shfl_down((int)word, 2) << 8;
      if ((ch & 3) == 0) sm[(r + 16 * (gi >> 2)) * kTiles + tkl] = (uint16_t)word;
    }
  }
  __syncthreads();
  // tiles (tr, tk0 .. tk0 + kTiles - 1) are contiguous in the packed arrays
  const size_t t0 = (size_t)tr * TK + tk0;
  const int n_tiles = min(kTiles, TK - tk0);
#pragma unroll
  for (int u = tid; u < kTiles * kTileU4; u += kPackThreads)
    if (u < n_tiles * kTileU4) values[t0 * kTileU4 + u] = sv[u];
  // metadata block (tr, tk0 / 8): slot tid's 16 bytes (bf16), or the half of them for tiles
  // tk0 .. tk0 + 3 (fp32: with zeros for the other half when no workgroup covers it)
  uint8_t* mblock = (uint8_t*)meta + ((size_t)tr * TKB + tk0 / 8) * 1024;
  if (tid < 64) {
    if constexpr (kTiles == 8) {
      *(u32x4_t*)(mblock + tid * 16) = ((const u32x4_t*)sm)[tid];
    } else {
      const u32x2_t half = ((const u32x2_t*)sm)[tid];
      if (tk0 % 8 == 0 && tk0 + 4 >= TK) *(u32x4_t*)(mblock + tid * 16) = u32x4_t{half[0], half[1], 0u, 0u};
      else *(u32x2_t*)(mblock + tid * 16 + (tk0 % 8) * 2) = half;
    }
  }
}

dim3 pack_grid(int64_t n_out, int64_t n_in, bool bf16) {
  const int cols = 16 * kPackChunksPerThread * (bf16 ? 8 : 4);
  return dim3((unsigned)ceil_div(n_out, 16), (unsigned)ceil_div(n_in, cols));
}

template <bool SCALED, int NM = 0>
hipError_t launch_pack(const void* R, const float* d, int64_t n_out, int64_t n_in, bool bf16, void* values,
                       uint32_t* meta, hipStream_t stream, int n_keep = 2) {
  constexpr int CPT = kPackChunksPerThread;
  const int TK = (int)ceil_div(n_in, 64), TKB = (TK + 7) / 8;
  const dim3 grid = pack_grid(n_out, n_in, bf16);
  if (bf16)
    prune24_pack_kernel<true, SCALED, CPT, NM><<<grid, dim3(kPackThreads), 0, stream>>>(
        (const uint8_t*)R, d, (int)n_out, (int)n_in, TK, TKB, (u32x4_t*)values, meta, n_keep);
  else
    prune24_pack_kernel<false, SCALED, CPT, NM><<<grid, dim3(kPackThreads), 0, stream>>>(
        (const uint8_t*)R, d, (int)n_out, (int)n_in, TK, TKB, (u32x4_t*)values, meta, n_keep);
  return hipGetLastError();
}

}  // namespace

bool pack_grids_fit(int64_t n_out, int64_t n_in, bool bf16) {
  return grid_fits(pack_grid(n_out, n_in, bf16), kPackThreads);
}

hipError_t launch_prune24_pack(const void* R, int64_t n_out, int64_t n_in, bool bf16, void* values,
                               uint32_t* meta, hipStream_t stream) {
  return launch_pack<false>(R, nullptr, n_out, n_in, bf16, values, meta, stream);
}

hipError_t launch_prune_nm_pack(const void* R, int64_t n_out, int64_t n_in, int n, int m, bool bf16, void* values,
                                uint32_t* meta, hipStream_t stream) {
  if (n == 2 && m == 4) return launch_pack<false>(R, nullptr, n_out, n_in, bf16, values, meta, stream);
  switch (m) {
    case 4: return launch_pack<false, 4>(R, nullptr, n_out, n_in, bf16, values, meta, stream, n);
    case 8: return launch_pack<false, 8>(R, nullptr, n_out, n_in, bf16, values, meta, stream, n);
    case 16: return launch_pack<false, 16>(R, nullptr, n_out, n_in, bf16, values, meta, stream, n);
    default: return hipErrorInvalidValue;
  }
}

hipError_t launch_prune24_pack_scaled(const void* R, const float* d, int64_t n_out, int64_t n_in, bool bf16,
                                      void* values, uint32_t* meta, hipStream_t stream) {
  return launch_pack<true>(R, d, n_out, n_in, bf16, values, meta, stream);
}

}  // namespace splr
