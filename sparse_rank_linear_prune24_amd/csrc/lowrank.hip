// First stage of the low-rank product, T = X V^T (LoSparse page, §3.2: the input is multiplied by
// the thin factors; in the orientation used here X [M x n_in] times V^T [n_in x r]).
//
// bf16: dense MFMA 16x16x32 with float32 accumulation. One wave owns 16 tokens x 64 ranks over one
// slice of K; K is split across waves when there are few token blocks (decode shapes) so enough
// waves stream X and V, and the slices' partial sums are written as separate float32 planes which
// the consumer adds in a fixed order (no atomics: bitwise reproducible).
// fp32: one wave per output, lanes stride over K, fixed-order butterfly reduction.
#include "common.hpp"
#include "kernels.hpp"

namespace splr {
namespace {

constexpr int kRankBlocks = 4;  // 16-wide rank blocks per wave (64 ranks)
constexpr int kStepUnroll = 4;  // K steps (32 columns each) whose loads are issued together

__global__ __launch_bounds__(64) void lowrank_bf16_kernel(const uint16_t* __restrict__ X,
                                                         const uint16_t* __restrict__ V, int M, int K,
                                                         int r, int steps_per_split,
                                                         float* __restrict__ Tpart) {
  const int lane = threadIdx.x;
  const int m0 = blockIdx.x * 16;
  const int j0 = blockIdx.y * 16 * kRankBlocks;
  const int split = blockIdx.z;
  const int nsteps = K / 32;
  const int s_begin = split * steps_per_split;
  const int s_end = min(nsteps, s_begin + steps_per_split);

  const int row = lane & 15;       // A row (token) / B column (rank) owned by this lane
  const int koff = 8 * (lane >> 4);  // this lane's 8-column slice of a 32-column K step
  const bool m_ok = m0 + row < M;
  const uint16_t* xrow = X + (size_t)(m_ok ? m0 + row : 0) * K + koff;
  const uint16_t* vrow[kRankBlocks];
  bool j_ok[kRankBlocks];
#pragma unroll
  for (int b = 0; b < kRankBlocks; ++b) {
    const int j = j0 + 16 * b + row;
    j_ok[b] = j < r;
    vrow[b] = V + (size_t)(j_ok[b] ? j : 0) * K + koff;
  }
  f32x4_t acc[kRankBlocks];
#pragma unroll
  for (int b = 0; b < kRankBlocks; ++b) acc[b] = f32x4_t{0, 0, 0, 0};

  const u32x4_t zero = {0, 0, 0, 0};
  for (int s = s_begin; s < s_end; s += kStepUnroll) {
    u32x4_t xa[kStepUnroll], vb[kStepUnroll][kRankBlocks];
#pragma unroll
    for (int u = 0; u < kStepUnroll; ++u) {
      const bool in = s + u < s_end;
      const size_t k = (size_t)(s + u) * 32;
      xa[u] = (in && m_ok) ? *(const u32x4_t*)(xrow + k) : zero;
#pragma unroll
      for (int b = 0; b < kRankBlocks; ++b) vb[u][b] = (in && j_ok[b]) ? *(const u32x4_t*)(vrow[b] + k) : zero;
    }
#pragma unroll
    for (int u = 0; u < kStepUnroll; ++u)
#pragma unroll
      for (int b = 0; b < kRankBlocks; ++b) acc[b] = mfma16x16x32(as_bf16x8(xa[u]), as_bf16x8(vb[u][b]), acc[b]);
  }

  float* out = Tpart + (size_t)split * M * r;
#pragma unroll
  for (int b = 0; b < kRankBlocks; ++b) {
    const int j = j0 + 16 * b + (lane & 15);
    if (j >= r) continue;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int m = m0 + 4 * (lane >> 4) + i;
      if (m < M) out[(size_t)m * r + j] = acc[b][i];
    }
  }
}

__global__ __launch_bounds__(256) void lowrank_f32_kernel(const float* __restrict__ X, const float* __restrict__ V,
                                                         int M, int K, int r, float* __restrict__ T) {
  const int wave = blockIdx.x * 4 + (threadIdx.x >> 6);
  const int lane = threadIdx.x & 63;
  if (wave >= M * r) return;
  const int m = wave / r, j = wave % r;
  const float* x = X + (size_t)m * K;
  const float* v = V + (size_t)j * K;
  float t = 0.0f;
  for (int k = lane; k < K; k += 64) t = fmaf(x[k], v[k], t);
#pragma unroll
  for (int off = 32; off > 0; off >>= 1) t += __shfl_xor(t, off);
  if (lane == 0) T[(size_t)m * r + j] = t;
}

}  // namespace

int lowrank_ksplit(int64_t M, int64_t n_in, int64_t r, bool bf16) {
  if (!bf16 || r == 0) return 1;
  const int64_t waves = ceil_div(M, 16) * ceil_div(r, 16 * kRankBlocks);
  const int64_t nsteps = n_in / 32;
  int64_t ks = ceil_div(512, waves);
  ks = ks < 16 ? ks : 16;
  const int64_t max_by_k = nsteps / 8 > 1 ? nsteps / 8 : 1;  // keep >= 8 steps (256 columns) per slice
  ks = ks < max_by_k ? ks : max_by_k;
  return (int)(ks > 0 ? ks : 1);
}

hipError_t launch_lowrank(const void* X, const void* V, int64_t M, int64_t n_in, int64_t r, bool bf16, int ksplit,
                          float* Tpart, hipStream_t stream) {
  if (r == 0) return hipSuccess;
  if (bf16) {
    const int nsteps = (int)(n_in / 32);
    const int per = (int)ceil_div(nsteps, ksplit);
    dim3 grid((unsigned)ceil_div(M, 16), (unsigned)ceil_div(r, 16 * kRankBlocks), (unsigned)ksplit);
    lowrank_bf16_kernel<<<grid, dim3(64), 0, stream>>>((const uint16_t*)X, (const uint16_t*)V, (int)M, (int)n_in,
                                                      (int)r, per, Tpart);
  } else {
    const int64_t waves = M * r;
    lowrank_f32_kernel<<<dim3((unsigned)ceil_div(waves, 4)), dim3(256), 0, stream>>>(
        (const float*)X, (const float*)V, (int)M, (int)n_in, (int)r, Tpart);
  }
  return hipGetLastError();
}

}  // namespace splr
