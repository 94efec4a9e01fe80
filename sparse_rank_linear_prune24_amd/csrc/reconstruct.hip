// W_hat = S + U V as a dense float32 matrix (LoSparse page, §3: the weight is approximated by the
// sum of the sparse and the low-rank part).  One lane per group of four columns: the two stored
// entries are widened exactly to float32 at their columns (+0 elsewhere); when r > 0 the rank-r
// sum, accumulated in float32 over j in order, is added once.
#include <algorithm>

#include "common.hpp"
#include "kernels.hpp"

namespace splr {
namespace {

template <bool BF16>
__device__ __forceinline__ float load_elem(const void* p, size_t i) {
  if (BF16) return bf16_bits_to_float(((const uint16_t*)p)[i]);
  return ((const float*)p)[i];
}

// group g (columns 4g .. 4g+3) of row n
template <bool BF16>
__device__ __forceinline__ void reconstruct_group(const void* __restrict__ values, const uint32_t* __restrict__ meta,
                                                  const void* __restrict__ U, const void* __restrict__ V, int K, int r,
                                                  float* __restrict__ W, int64_t n, int g) {
  // packed tiles of 16 rows x 64 columns: tile (n / 16, g / 16), slot n % 16 + 16 * (gi / 4)
  const int TK = (K + 63) / 64, gi = g % 16;
  const size_t tile = (size_t)(n / 16) * TK + g / 16;
  const uint32_t nib = (meta_unit(meta, meta_blocks(TK), n / 16, g / 16, (int)(n % 16) + 16 * (gi / 4)) >> (4 * (gi % 4))) & 0xFu;
  const int a = (int)(nib & 3u), b = (int)(nib >> 2);
  const size_t e = (tile * 64 + (size_t)(n % 16) + 16 * (gi / 4)) * 8 + 2 * (gi % 4);
  float out[4] = {0.0f, 0.0f, 0.0f, 0.0f};
  out[a] = load_elem<BF16>(values, e);
  out[b] = load_elem<BF16>(values, e + 1);
  if (r > 0) {
    float lr[4] = {0.0f, 0.0f, 0.0f, 0.0f};
    for (int j = 0; j < r; ++j) {
      const float u = load_elem<BF16>(U, (size_t)n * r + j);
#pragma unroll
      for (int q = 0; q < 4; ++q) lr[q] = fmaf(u, load_elem<BF16>(V, (size_t)j * K + 4 * g + q), lr[q]);
    }
#pragma unroll
    for (int q = 0; q < 4; ++q) out[q] += lr[q];
  }
  *(f32x4_t*)(W + (size_t)n * K + 4 * g) = f32x4_t{out[0], out[1], out[2], out[3]};
}

// Grid-stride over groups t = n * (K / 4) + g (64-bit; the grid is capped)
template <bool BF16>
__global__ __launch_bounds__(256) void dense_reconstruct_kernel(const void* __restrict__ values,
                                                               const uint32_t* __restrict__ meta,
                                                               const void* __restrict__ U, const void* __restrict__ V,
                                                               int64_t n_out, int K, int r, float* __restrict__ W) {
  const int groups = K / 4;
  for (int64_t t = (int64_t)blockIdx.x * 256 + threadIdx.x; t < n_out * groups; t += (int64_t)gridDim.x * 256)
    reconstruct_group<BF16>(values, meta, U, V, K, r, W, t / groups, (int)(t % groups));
}

constexpr int64_t kMaxBlocks = int64_t(1) << 20;
dim3 reconstruct_grid(int64_t n_out, int64_t n_in) {
  return dim3((unsigned)std::min(ceil_div(n_out * (n_in / 4), 256), kMaxBlocks));
}

}  // namespace

bool reconstruct_grids_fit(int64_t n_out, int64_t n_in) { return grid_fits(reconstruct_grid(n_out, n_in), 256); }

hipError_t launch_dense_reconstruct(const void* values, const uint32_t* meta, const void* U, const void* V,
                                    int64_t n_out, int64_t n_in, int64_t r, bool bf16, float* W_hat,
                                    hipStream_t stream) {
  const dim3 grid = reconstruct_grid(n_out, n_in);
  if (bf16)
    dense_reconstruct_kernel<true><<<grid, dim3(256), 0, stream>>>(values, meta, U, V, n_out, (int)n_in, (int)r, W_hat);
  else
    dense_reconstruct_kernel<false><<<grid, dim3(256), 0, stream>>>(values, meta, U, V, n_out, (int)n_in, (int)r, W_hat);
  return hipGetLastError();
}

}  // namespace splr
