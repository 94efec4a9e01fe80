// Internal launchers of libsplr (argument checking happens in api.hip before these are called).
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

namespace splr {

// Dispatch limits of one launch (HIP on gfx9): fewer than 2^32 work-items along x, at most 65535
// workgroups along y and z. Every entry point checks the grids of all the launches it will make
// against these limits before its first HIP call (the *_grids_fit functions below compute those
// grids exactly as the launchers do).
inline bool grid_fits(dim3 g, unsigned threads) {
  return g.x >= 1 && g.y >= 1 && g.z >= 1 && (uint64_t)g.x * threads < (uint64_t(1) << 32) && g.y <= 65535u &&
         g.z <= 65535u;
}
bool pack_grids_fit(int64_t n_out, int64_t n_in, bool bf16);
bool residual_grids_fit(int64_t n_out, int64_t n_in);
bool lowrank_grids_fit(int64_t M, int64_t n_in, int64_t r, bool bf16);
bool linear_grids_fit(int64_t M, int64_t n_in, int64_t n_out, int64_t r, bool bf16);
bool reconstruct_grids_fit(int64_t n_out, int64_t n_in);
dim3 linear_f32_grid(int64_t M, int64_t n_out);

hipError_t launch_prune24_pack(const void* R, int64_t n_out, int64_t n_in, bool bf16, void* values,
                               uint32_t* meta, hipStream_t stream);
// Fused residual R = W - U V (pinned binary32 fused multiply-add order, then rounding) + pack.
hipError_t launch_prune24_pack_residual(const void* W, const void* U, const void* V, int64_t n_out, int64_t n_in,
                                        int64_t r, bool bf16, void* values, uint32_t* meta, hipStream_t stream);
// N:M projection (n in {1, 2}, m in {4, 8, 16}), then the 2:4 pack of the result.
hipError_t launch_prune_nm_pack(const void* R, int64_t n_out, int64_t n_in, int n, int m, bool bf16, void* values,
                                uint32_t* meta, hipStream_t stream);
// The same with keys |R[n][k]| * |d[k]| (d: float32 [n_in]).
hipError_t launch_prune24_pack_scaled(const void* R, const float* d, int64_t n_out, int64_t n_in, bool bf16,
                                      void* values, uint32_t* meta, hipStream_t stream);

// First low-rank stage T = X V^T, written to the workspace as float32 partial sums over `slices`
// slices of K: part[z][M][r], z = 0 .. slices-1 (T = sum of the slices in slice order; the fp32 path
// always uses one slice).
constexpr int kMaxLowrankSlices = 16;
int lowrank_slices(int64_t M, int64_t n_in, int64_t r, bool bf16);
size_t lowrank_workspace_bytes(int64_t M, int64_t n_in, int64_t r, bool bf16);
hipError_t launch_lowrank(const void* X, const void* V, int64_t M, int64_t n_in, int64_t r, bool bf16,
                          void* workspace, hipStream_t stream);

// Y (float32, or bfloat16 when y_bf16, rounded to nearest even) = X S^T + T U^T, T given as
// `slices` float32 partial sums [slices][M][r] (r == 0: no low-rank term). The partials are added
// in slice order and T enters the MFMAs as a bfloat16 pair hi = RNE(T), lo = RNE(T - hi).
hipError_t launch_linear_bf16(const void* X, int64_t M, int64_t n_in, const void* values, const uint32_t* meta,
                              int64_t n_out, const void* U, int64_t r, const float* Tpart, int slices, void* Y,
                              bool y_bf16, hipStream_t stream);
// The same for `layers` (1 .. kMaxGroup) layers of one shape in one launch, their tiles in one grid
// (each layer's Y bit-identical to its own launch_linear_bf16); M > kDecodeMaxTokens.
constexpr int kMaxGroup = 4;
bool linear_group_grid_fits(int64_t M, int64_t n_out, int layers);
hipError_t launch_linear_bf16_group(int layers, const void* const* X, int64_t M, int64_t n_in,
                                    const void* const* values, const uint32_t* const* meta, int64_t n_out,
                                    const void* const* U, int64_t r, const float* const* Tpart, int slices,
                                    void* const* Y, bool y_bf16, hipStream_t stream);
// Stage 2 with S decompressed to dense bfloat16 in registers and dense MFMA (the alternative to the
// structured-sparse instruction, any M; same tiles and pipeline as the prefill kernels' 512-row
// design: 512 rows and eight waves when that gives every CU a tile, else 256 rows and four).
bool linear_dense_grids_fit(int64_t M, int64_t n_out);
hipError_t launch_linear_bf16_dense(const void* X, int64_t M, int64_t n_in, const void* values, const uint32_t* meta,
                                    int64_t n_out, const void* U, int64_t r, const float* Tpart, int slices, void* Y,
                                    hipStream_t stream);
// The same for M <= kDecodeMaxTokens (decode kernel).
bool decode_grids_fit(int64_t M, int64_t n_out);
hipError_t launch_linear_decode(const void* X, int64_t M, int64_t n_in, const void* values, const uint32_t* meta,
                                int64_t n_out, const void* U, int64_t r, const float* Tpart, int slices, void* Y,
                                bool y_bf16, hipStream_t stream);
hipError_t launch_linear_f32(const float* X, int64_t M, int64_t n_in, const float* values, const uint32_t* meta,
                             int64_t n_out, const float* U, int64_t r, const float* T, void* Y, bool y_bf16,
                             hipStream_t stream);

hipError_t launch_dense_reconstruct(const void* values, const uint32_t* meta, const void* U, const void* V,
                                    int64_t n_out, int64_t n_in, int64_t r, bool bf16, float* W_hat,
                                    hipStream_t stream);

// Cholesky QR building blocks of the low-rank step's subspace iteration (k <= kMaxCholK):
// G = Y^T Y in float64 for float32 Y [n][k] (workspace: gram_workspace_bytes), and R^-1 (float32,
// upper triangular, k x k) for G = R^T R.
constexpr int kMaxCholK = 192;
size_t gram_workspace_bytes(int64_t n, int64_t k);
hipError_t launch_gram_f64(const float* Y, int64_t n, int64_t k, double* G, void* workspace, hipStream_t stream);
hipError_t launch_chol_rinv(const double* G, int64_t k, float* Rinv, hipStream_t stream);

// Token count up to which splr_linear takes the HBM-streaming (decode) kernel.
constexpr int64_t kDecodeMaxTokens = 64;

}  // namespace splr
