// Small dense factorisations for the subspace iteration of the low-rank step (HASSLE-free page, §4.2:
// the low-rank update is the rank-r truncated SVD of W - S). The iteration keeps a k-column basis
// (k = r + oversampling, at most kMaxCholK) orthonormal by Cholesky QR: G = Y^T Y in float64, then
// G = R^T R and Y R^-1. Both run here so that a step of the loop needs no host round trip for them:
//
//   gram_partial_kernel / gram_reduce_kernel: G = Y^T Y (float64) for float32 Y [n][k]; products of
//     float32 values are exact in float64, each workgroup sums its rows in row order, and the
//     partials are added in workgroup order (deterministic).
//   chol_rinv_kernel: R^-1 (float32, upper triangular) for G = R^T R, one workgroup: Cholesky
//     G = L L^T by block columns (L = R^T), then X = L^-1 by block rows (forward substitution on
//     the identity), written transposed; 4 x 4 blocks of the lower triangle held in registers,
//     L and one block row of X shared through LDS.
#include <algorithm>
#include <cmath>

#include "common.hpp"
#include "kernels.hpp"

namespace splr {
namespace {

constexpr int kGramThreads = 1024;
constexpr int kGramRows = 32;    // rows staged in LDS at a time
constexpr int kGramMaxBlocks = 128;
constexpr int kCholThreads = 512;

// 4 x 4 block index t of the lower (ib >= jb) triangle, t = ib (ib + 1) / 2 + jb
__device__ __forceinline__ void tri_block(int t, int& ib, int& jb) {
  int i = (int)((sqrtf(8.0f * (float)t + 1.0f) - 1.0f) * 0.5f);
  while (i * (i + 1) / 2 > t) --i;
  while ((i + 1) * (i + 2) / 2 <= t) ++i;
  ib = i;
  jb = t - i * (i + 1) / 2;
}

// Block b sums rows [b * rows_per_block, ...) of Y; thread t accumulates 4 x 4 blocks t and t + 1024
// of G's lower triangle (float64), over kGramRows-row chunks staged in LDS as float32.
__global__ __launch_bounds__(kGramThreads) void gram_partial_kernel(const float* __restrict__ Y, int64_t n, int k,
                                                                    int64_t rows_per_block,
                                                                    double* __restrict__ partial) {
  __shared__ __align__(16) float ys[kGramRows * kMaxCholK];
  const int kb = (k + 3) / 4, nblk = kb * (kb + 1) / 2;
  const int64_t r0 = (int64_t)blockIdx.x * rows_per_block;
  const int64_t r1 = std::min<int64_t>(n, r0 + rows_per_block);
  double acc[2][4][4] = {};
  int ib[2], jb[2];
#pragma unroll
  for (int m = 0; m < 2; ++m) {
    const int t = threadIdx.x + m * kGramThreads;
    if (t < nblk) tri_block(t, ib[m], jb[m]);
    else ib[m] = jb[m] = -1;
  }
  for (int64_t c0 = r0; c0 < r1; c0 += kGramRows) {
    const int rows = (int)std::min<int64_t>(kGramRows, r1 - c0);
    __syncthreads();  // the previous chunk's reads are done
    // columns past k read as zero (the 4 x 4 blocks of the last block column overhang)
    for (int e = threadIdx.x; e < kGramRows * 4 * kb; e += kGramThreads) {
      const int row = e / (4 * kb), col = e % (4 * kb);
      ys[row * (4 * kb) + col] = (row < rows && col < k) ? Y[(c0 + row) * k + col] : 0.0f;
    }
    __syncthreads();
#pragma unroll
    for (int m = 0; m < 2; ++m) {
      if (ib[m] < 0) continue;
      for (int row = 0; row < rows; ++row) {
        const float4 a = *(const float4*)&ys[row * (4 * kb) + 4 * ib[m]];
        const float4 c = *(const float4*)&ys[row * (4 * kb) + 4 * jb[m]];
        const double av[4] = {a.x, a.y, a.z, a.w}, cv[4] = {c.x, c.y, c.z, c.w};
#pragma unroll
        for (int x = 0; x < 4; ++x)
#pragma unroll
          for (int y = 0; y < 4; ++y) acc[m][x][y] = fma(av[x], cv[y], acc[m][x][y]);
      }
    }
  }
  // partial[block][4 ib + x][4 jb + y], k x k row-major, only the lower-triangle blocks written
  double* out = partial + (size_t)blockIdx.x * k * k;
#pragma unroll
  for (int m = 0; m < 2; ++m) {
    if (ib[m] < 0) continue;
#pragma unroll
    for (int x = 0; x < 4; ++x)
#pragma unroll
      for (int y = 0; y < 4; ++y) {
        const int i = 4 * ib[m] + x, j = 4 * jb[m] + y;
        if (i < k && j < k && j <= i) out[(size_t)i * k + j] = acc[m][x][y];
      }
  }
}

// G[i][j] = G[j][i] = sum over blocks, in block order, of partial[b][i][j] (i >= j)
__global__ __launch_bounds__(256) void gram_reduce_kernel(const double* __restrict__ partial, int blocks, int k,
                                                          double* __restrict__ G) {
  const int e = blockIdx.x * 256 + threadIdx.x;
  if (e >= k * k) return;
  const int i = e / k, j = e % k;
  if (j > i) return;
  double s = 0.0;
  for (int b = 0; b < blocks; ++b) s += partial[(size_t)b * k * k + e];
  G[(size_t)i * k + j] = s;
  G[(size_t)j * k + i] = s;
}

using Blk = double[4][4];

// 1 / sqrt(d) and 1 / a from the hardware approximations plus Newton steps (a few ulps; the
// factorisation's own rounding is larger): short dependency chains for the serial parts of the
// blocked factorisation. d <= 0 gives NaN or infinity, which propagates.
__device__ __forceinline__ double rsqrt_nr(double d) {
  double y = __builtin_amdgcn_rsq(d);
#pragma unroll
  for (int it = 0; it < 2; ++it) {
    const double e = fma(-d * y, y, 1.0);
    y = fma(0.5 * y, e, y);
  }
  return y;
}
__device__ __forceinline__ double rcp_nr(double a) {
  double y = __builtin_amdgcn_rcp(a);
#pragma unroll
  for (int it = 0; it < 2; ++it) y = fma(y, fma(-a, y, 1.0), y);
  return y;
}

// L (lower triangular 4 x 4) = chol(A) of a symmetric positive definite 4 x 4 block (lower part read)
__device__ __forceinline__ void chol4(const Blk& A, Blk& L) {
#pragma unroll
  for (int c = 0; c < 4; ++c) {
    double d = A[c][c];
#pragma unroll
    for (int m = 0; m < c; ++m) d -= L[c][m] * L[c][m];
    const double inv = rsqrt_nr(d);
    L[c][c] = d * inv;
#pragma unroll
    for (int i = c + 1; i < 4; ++i) {
      double v = A[i][c];
#pragma unroll
      for (int m = 0; m < c; ++m) v -= L[i][m] * L[c][m];
      L[i][c] = v * inv;
    }
#pragma unroll
    for (int i = 0; i < c; ++i) L[i][c] = 0.0;
  }
}

// Xi = L^-1 of a lower triangular 4 x 4 block (forward substitution on the identity)
__device__ __forceinline__ void trinv4(const Blk& L, Blk& Xi) {
  double rd[4];
#pragma unroll
  for (int i = 0; i < 4; ++i) rd[i] = rcp_nr(L[i][i]);
#pragma unroll
  for (int c = 0; c < 4; ++c)
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      if (i < c) {
        Xi[i][c] = 0.0;
        continue;
      }
      double v = (i == c) ? 1.0 : 0.0;
#pragma unroll
      for (int m = c; m < i; ++m) v -= L[i][m] * Xi[m][c];
      Xi[i][c] = v * rd[i];
    }
}

__device__ __forceinline__ void load_blk(const double* p, Blk& b) {
#pragma unroll
  for (int x = 0; x < 4; ++x)
#pragma unroll
    for (int y = 0; y < 4; ++y) b[x][y] = p[4 * x + y];
}
__device__ __forceinline__ void store_blk(double* p, const Blk& b) {
#pragma unroll
  for (int x = 0; x < 4; ++x)
#pragma unroll
    for (int y = 0; y < 4; ++y) p[4 * x + y] = b[x][y];
}

// One workgroup; the matrix is padded to 4 kb rows with the identity and cut into 4 x 4 blocks;
// thread t owns lower-triangle blocks t + 512 m (m < MAXB) in registers. Blocked right-looking
// Cholesky, one block column per step (two barriers): the diagonal block's factor L_cc (computed
// by its owner at the end of the previous step) is in LDS; the owners of the panel below solve
// L_ic = A_ic L_cc^-T and publish it; every owner of a trailing block subtracts L_ic L_jc^T, and
// the owner of the next diagonal block factors it. Then X = L^-1 by block rows (one barrier per
// step, double-buffered): X_rc = L_rr^-1 B_rc for the row's blocks, published, and B_ic -= L_ir X_rc
// below it. L is kept in LDS as 4 x 4 blocks in triangle order.
template <int MAXB>
__global__ __launch_bounds__(kCholThreads) void chol_rinv_kernel(const double* __restrict__ G, int k,
                                                                 float* __restrict__ Rinv) {
  constexpr int kMaxKb = (kMaxCholK + 3) / 4;
  __shared__ double lblk[kMaxKb * (kMaxKb + 1) / 2 * 16];  // L, block t at 16 t
  __shared__ double xrow[2][kMaxKb * 16];                   // a block row of X
  const int kb = (k + 3) / 4, nblk = kb * (kb + 1) / 2;
  Blk a[MAXB];
  int ib[MAXB], jb[MAXB];
#pragma unroll
  for (int m = 0; m < MAXB; ++m) {
    const int t = threadIdx.x + m * kCholThreads;
    if (t < nblk) tri_block(t, ib[m], jb[m]);
    else ib[m] = jb[m] = -1;
#pragma unroll
    for (int x = 0; x < 4; ++x)
#pragma unroll
      for (int y = 0; y < 4; ++y) {
        const int i = 4 * ib[m] + x, j = 4 * jb[m] + y;
        a[m][x][y] = (ib[m] < 0) ? 0.0 : (i < k && j < k) ? G[(size_t)i * k + j] : (i == j ? 1.0 : 0.0);
      }
  }
  auto tri = [](int i, int j) { return i * (i + 1) / 2 + j; };
  // step 0's diagonal factor
#pragma unroll
  for (int m = 0; m < MAXB; ++m)
    if (ib[m] == 0 && jb[m] == 0) {
      Blk L;
      chol4(a[m], L);
      store_blk(lblk, L);
#pragma unroll
      for (int x = 0; x < 4; ++x)
#pragma unroll
        for (int y = 0; y < 4; ++y) a[m][x][y] = L[x][y];
    }
  for (int cb = 0; cb < kb; ++cb) {
    __syncthreads();  // L_cc in LDS
#pragma unroll
    for (int m = 0; m < MAXB; ++m) {
      if (jb[m] != cb || ib[m] <= cb) continue;
      Blk Lc;
      load_blk(lblk + 16 * tri(cb, cb), Lc);
      double rd[4];
#pragma unroll
      for (int c = 0; c < 4; ++c) rd[c] = rcp_nr(Lc[c][c]);
      // row x of L_ic solves l L_cc^T = a (forward over the columns)
#pragma unroll
      for (int x = 0; x < 4; ++x)
#pragma unroll
        for (int c = 0; c < 4; ++c) {
          double v = a[m][x][c];
#pragma unroll
          for (int q = 0; q < c; ++q) v -= a[m][x][q] * Lc[c][q];
          a[m][x][c] = v * rd[c];
        }
      store_blk(lblk + 16 * tri(ib[m], cb), a[m]);
    }
    __syncthreads();  // the panel in LDS
#pragma unroll
    for (int m = 0; m < MAXB; ++m) {
      if (jb[m] <= cb) continue;  // finished (or not owned)
      Blk Li, Lj;
      load_blk(lblk + 16 * tri(ib[m], cb), Li);
      load_blk(lblk + 16 * tri(jb[m], cb), Lj);
#pragma unroll
      for (int x = 0; x < 4; ++x)
#pragma unroll
        for (int y = 0; y < 4; ++y) {
          double v = a[m][x][y];
#pragma unroll
          for (int q = 0; q < 4; ++q) v -= Li[x][q] * Lj[y][q];
          a[m][x][y] = v;
        }
      if (ib[m] == cb + 1 && jb[m] == cb + 1) {
        Blk L;
        chol4(a[m], L);
        store_blk(lblk + 16 * tri(cb + 1, cb + 1), L);
#pragma unroll
        for (int x = 0; x < 4; ++x)
#pragma unroll
          for (int y = 0; y < 4; ++y) a[m][x][y] = L[x][y];
      }
    }
  }
  __syncthreads();  // all of L in LDS

  // X = L^-1 by block rows; a[] becomes B (the identity, then the running right-hand side)
#pragma unroll
  for (int m = 0; m < MAXB; ++m)
#pragma unroll
    for (int x = 0; x < 4; ++x)
#pragma unroll
      for (int y = 0; y < 4; ++y) a[m][x][y] = (ib[m] >= 0 && ib[m] == jb[m] && x == y) ? 1.0 : 0.0;
  for (int rb = 0; rb < kb; ++rb) {
    double* xr = xrow[rb % 2];
#pragma unroll
    for (int m = 0; m < MAXB; ++m) {
      if (ib[m] != rb) continue;
      Blk Lr, Xi, out;
      load_blk(lblk + 16 * tri(rb, rb), Lr);
      trinv4(Lr, Xi);
#pragma unroll
      for (int x = 0; x < 4; ++x)
#pragma unroll
        for (int y = 0; y < 4; ++y) {
          double v = 0.0;
#pragma unroll
          for (int q = 0; q <= x; ++q) v += Xi[x][q] * a[m][q][y];
          out[x][y] = v;
        }
#pragma unroll
      for (int x = 0; x < 4; ++x)
#pragma unroll
        for (int y = 0; y < 4; ++y) a[m][x][y] = out[x][y];
      store_blk(xr + 16 * jb[m], out);
    }
    __syncthreads();  // the block row of X in LDS
#pragma unroll
    for (int m = 0; m < MAXB; ++m) {
      if (ib[m] <= rb || jb[m] > rb) continue;
      Blk Li, Xr;
      load_blk(lblk + 16 * tri(ib[m], rb), Li);
      load_blk(xr + 16 * jb[m], Xr);
#pragma unroll
      for (int x = 0; x < 4; ++x)
#pragma unroll
        for (int y = 0; y < 4; ++y) {
          double v = a[m][x][y];
#pragma unroll
          for (int q = 0; q < 4; ++q) v -= Li[x][q] * Xr[q][y];
          a[m][x][y] = v;
        }
    }
  }
  // Rinv = X^T: Rinv[c][i] = X[i][c] (i >= c), zero below the diagonal
#pragma unroll
  for (int m = 0; m < MAXB; ++m) {
    if (ib[m] < 0) continue;
#pragma unroll
    for (int x = 0; x < 4; ++x)
#pragma unroll
      for (int y = 0; y < 4; ++y) {
        const int i = 4 * ib[m] + x, c = 4 * jb[m] + y;
        if (i >= k || c >= k) continue;
        if (c <= i) {
          Rinv[(size_t)c * k + i] = (float)a[m][x][y];
          if (c < i) Rinv[(size_t)i * k + c] = 0.0f;
        }
      }
  }
}

int gram_blocks(int64_t n) { return (int)std::min<int64_t>(kGramMaxBlocks, ceil_div(n, kGramRows)); }

}  // namespace

size_t gram_workspace_bytes(int64_t n, int64_t k) { return (size_t)gram_blocks(n) * k * k * sizeof(double); }

hipError_t launch_gram_f64(const float* Y, int64_t n, int64_t k, double* G, void* workspace, hipStream_t stream) {
  const int blocks = gram_blocks(n);
  const int64_t rows_per_block = ceil_div(n, blocks);
  double* partial = (double*)workspace;
  gram_partial_kernel<<<dim3(blocks), dim3(kGramThreads), 0, stream>>>(Y, n, (int)k, rows_per_block, partial);
  gram_reduce_kernel<<<dim3((unsigned)ceil_div(k * k, 256)), dim3(256), 0, stream>>>(partial, blocks, (int)k, G);
  return hipGetLastError();
}

hipError_t launch_chol_rinv(const double* G, int64_t k, float* Rinv, hipStream_t stream) {
  const int64_t kb = (k + 3) / 4, nblk = kb * (kb + 1) / 2;
  if (nblk <= kCholThreads)
    chol_rinv_kernel<1><<<dim3(1), dim3(kCholThreads), 0, stream>>>(G, (int)k, Rinv);
  else if (nblk <= 2 * kCholThreads)
    chol_rinv_kernel<2><<<dim3(1), dim3(kCholThreads), 0, stream>>>(G, (int)k, Rinv);
  else
    chol_rinv_kernel<3><<<dim3(1), dim3(kCholThreads), 0, stream>>>(G, (int)k, Rinv);
  return hipGetLastError();
}

}  // namespace splr
