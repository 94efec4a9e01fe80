// Y = X S^T + T U^T for float32 operands (T = X V^T from the first low-rank stage), float32
// arithmetic throughout (LoSparse page, §3.2: the two products summed).  One lane per output;
// the sparse sum walks the row's groups in order (through the packed tiles of 16 rows x 64
// columns), two fused multiply-adds per group.  This path exists for exact-type float32 layers
// (small, latency-bound); bf16 layers use the MFMA kernels.
#include <algorithm>

#include "common.hpp"
#include "kernels.hpp"

namespace splr {
namespace {

// one output Y[m][n]
__device__ __forceinline__ void linear_f32_output(const float* __restrict__ X, const float* __restrict__ values,
                                                  const uint32_t* __restrict__ meta, const float* __restrict__ U,
                                                  const float* __restrict__ T, void* __restrict__ Y, int y_bf16, int K,
                                                  int n_out, int r, int n, int m) {
  const float* x = X + (size_t)m * K;
  const int TK = (K + 63) / 64;
  const float* v = values + (size_t)(n / 16) * TK * 512;  // this row's tile row
  const int TKB = meta_blocks(TK);
  float acc = 0.0f;
  // unrolled so that the metadata, value and X loads of 16 groups are in flight together (measured
  // at 32 tokens x 512 x 512: 36 -> 13 us; loading each group's four X values at once and picking
  // two in registers instead of the indexed loads ran 29 us); the sum still runs over the groups in
  // order
#pragma unroll 16
  for (int grp = 0; grp < K / 4; ++grp) {
    const int tk = grp / 16, gi = grp % 16;
    const uint32_t nib = (meta_unit(meta, TKB, n / 16, tk, n % 16 + 16 * (gi / 4)) >> (4 * (gi % 4))) & 0xFu;
    const float* kept = v + (size_t)tk * 512 + ((n % 16) + 16 * (gi / 4)) * 8 + 2 * (gi % 4);
    acc = fmaf(x[4 * grp + (nib & 3u)], kept[0], acc);
    acc = fmaf(x[4 * grp + (nib >> 2)], kept[1], acc);
  }
  float lr = 0.0f;
#pragma unroll 8
  for (int j = 0; j < r; ++j) lr = fmaf(T[(size_t)m * r + j], U[(size_t)n * r + j], lr);
  const float y = acc + lr;
  if (y_bf16) ((uint16_t*)Y)[(size_t)m * n_out + n] = (uint16_t)float_to_bf16_bits(y);
  else ((float*)Y)[(size_t)m * n_out + n] = y;
}

__global__ __launch_bounds__(256) void linear_f32_kernel(const float* __restrict__ X, const float* __restrict__ values,
                                                        const uint32_t* __restrict__ meta,
                                                        const float* __restrict__ U, const float* __restrict__ T,
                                                        void* __restrict__ Y, int y_bf16, int M, int K, int n_out,
                                                        int r) {
  // workgroup tiles of 64 outputs x 4 tokens, numbered with the output block varying fastest; the
  // grid strides over them (it is capped, so large layers fit the dispatch limits)
  const int64_t nb = (n_out + 63) / 64, tiles = nb * ((M + 3) / 4);
  for (int64_t t = blockIdx.x; t < tiles; t += gridDim.x) {
    const int n = (int)(t % nb) * 64 + (threadIdx.x & 63);
    const int m = (int)(t / nb) * 4 + (threadIdx.x >> 6);
    if (n < n_out && m < M) linear_f32_output(X, values, meta, U, T, Y, y_bf16, K, n_out, r, n, m);
  }
}

}  // namespace

dim3 linear_f32_grid(int64_t M, int64_t n_out) {
  constexpr int64_t kMaxBlocks = int64_t(1) << 20;
  return dim3((unsigned)std::min(ceil_div(n_out, 64) * ceil_div(M, 4), kMaxBlocks));
}

hipError_t launch_linear_f32(const float* X, int64_t M, int64_t n_in, const float* values, const uint32_t* meta,
                             int64_t n_out, const float* U, int64_t r, const float* T, void* Y, bool y_bf16,
                             hipStream_t stream) {
  const dim3 grid = linear_f32_grid(M, n_out);
  linear_f32_kernel<<<grid, dim3(256), 0, stream>>>(X, values, meta, U, T, Y, y_bf16 ? 1 : 0, (int)M, (int)n_in,
                                                    (int)n_out, (int)r);
  return hipGetLastError();
}

}  // namespace splr
