// Internal launchers of libsplr (argument checking happens in api.hip before these are called).
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

namespace splr {

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
hipError_t launch_linear_f32(const float* X, int64_t M, int64_t n_in, const float* values, const uint32_t* meta,
                             int64_t n_out, const float* U, int64_t r, const float* T, void* Y, bool y_bf16,
                             hipStream_t stream);

hipError_t launch_dense_reconstruct(const void* values, const uint32_t* meta, const void* U, const void* V,
                                    int64_t n_out, int64_t n_in, int64_t r, bool bf16, float* W_hat,
                                    hipStream_t stream);

// Token count up to which splr_linear takes the HBM-streaming (decode) kernel.
constexpr int64_t kDecodeMaxTokens = 64;

}  // namespace splr
