// C ABI of libsplr (declared in include/splr.h): argument validation, workspace sizing and
// kernel dispatch.  Every check runs before the first HIP call, so a rejected call enqueues
// nothing; the library holds no mutable state and never allocates device memory.
#include "splr.h"

#include "kernels.hpp"

namespace {

// Size limits keep every index the kernels form inside their integer types.
constexpr int64_t kMaxRows = int64_t(1) << 24;      // n_out and M
constexpr int64_t kMaxCols = int64_t(1) << 20;      // n_in
constexpr int64_t kMaxElems = int64_t(1) << 36;     // n_out * n_in, M * n_in, M * n_out
constexpr int64_t kMaxRank = 1024;

bool aligned16(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }
bool dtype_ok(splr_dtype_t d) { return d == SPLR_FP32 || d == SPLR_BF16; }

splr_status_t check_in(int64_t n_in) {
  return (n_in >= 32 && n_in <= kMaxCols && n_in % 32 == 0) ? SPLR_OK : SPLR_ERR_SHAPE;
}

splr_status_t check_rows(int64_t rows, int64_t n_in) {
  if (rows < 1 || rows > kMaxRows) return SPLR_ERR_SHAPE;
  if (rows * n_in > kMaxElems) return SPLR_ERR_SHAPE;
  return SPLR_OK;
}

splr_status_t check_rank(int64_t r) {
  return (r >= 0 && r <= kMaxRank && r % 16 == 0) ? SPLR_OK : SPLR_ERR_SHAPE;
}

size_t round_up(size_t x, size_t a) { return (x + a - 1) / a * a; }

size_t workspace_bytes(int64_t M, int64_t n_in, int64_t r, splr_dtype_t dtype) {
  if (r == 0) return 0;
  return round_up(splr::lowrank_workspace_bytes(M, n_in, r, dtype == SPLR_BF16), 256);
}

splr_status_t from_hip(hipError_t e) { return e == hipSuccess ? SPLR_OK : SPLR_ERR_HIP; }

}  // namespace

extern "C" {

splr_status_t splr_prune24_pack(const void* R, int64_t n_out, int64_t n_in, splr_dtype_t dtype, void* values,
                                uint32_t* meta, hipStream_t stream) {
  if (!R || !values || !meta) return SPLR_ERR_NULL;
  splr_status_t s = check_in(n_in);
  if (s == SPLR_OK) s = check_rows(n_out, n_in);
  if (s != SPLR_OK) return s;
  if (!dtype_ok(dtype)) return SPLR_ERR_DTYPE;
  if (!aligned16(R) || !aligned16(values) || !aligned16(meta)) return SPLR_ERR_ALIGN;
  return from_hip(splr::launch_prune24_pack(R, n_out, n_in, dtype == SPLR_BF16, values, meta, stream));
}

splr_status_t splr_prune_nm_pack(const void* R, int64_t n_out, int64_t n_in, int32_t n, int32_t m,
                                 splr_dtype_t dtype, void* values, uint32_t* meta, hipStream_t stream) {
  if (!R || !values || !meta) return SPLR_ERR_NULL;
  splr_status_t s = check_in(n_in);
  if (s == SPLR_OK) s = check_rows(n_out, n_in);
  if (s == SPLR_OK && !((n == 1 || n == 2) && (m == 4 || m == 8 || m == 16))) s = SPLR_ERR_SHAPE;
  if (s != SPLR_OK) return s;  // n_in % 32 == 0, so every m above divides n_in
  if (!dtype_ok(dtype)) return SPLR_ERR_DTYPE;
  if (!aligned16(R) || !aligned16(values) || !aligned16(meta)) return SPLR_ERR_ALIGN;
  return from_hip(splr::launch_prune_nm_pack(R, n_out, n_in, n, m, dtype == SPLR_BF16, values, meta, stream));
}

splr_status_t splr_prune24_pack_residual(const void* W, const void* U, const void* V, int64_t n_out, int64_t n_in,
                                         int64_t r, splr_dtype_t dtype, void* values, uint32_t* meta,
                                         hipStream_t stream) {
  if (!W || !values || !meta) return SPLR_ERR_NULL;
  if (r > 0 && (!U || !V)) return SPLR_ERR_NULL;
  splr_status_t s = check_in(n_in);
  if (s == SPLR_OK) s = check_rows(n_out, n_in);
  if (s == SPLR_OK && (r < 0 || r > kMaxRank)) s = SPLR_ERR_SHAPE;
  if (s != SPLR_OK) return s;
  if (!dtype_ok(dtype)) return SPLR_ERR_DTYPE;
  if (!aligned16(W) || !aligned16(values) || !aligned16(meta)) return SPLR_ERR_ALIGN;
  if (r > 0 && (!aligned16(U) || !aligned16(V))) return SPLR_ERR_ALIGN;
  return from_hip(
      splr::launch_prune24_pack_residual(W, U, V, n_out, n_in, r, dtype == SPLR_BF16, values, meta, stream));
}

splr_status_t splr_prune24_pack_scaled(const void* R, const float* d, int64_t n_out, int64_t n_in, splr_dtype_t dtype,
                                       void* values, uint32_t* meta, hipStream_t stream) {
  if (!R || !d || !values || !meta) return SPLR_ERR_NULL;
  splr_status_t s = check_in(n_in);
  if (s == SPLR_OK) s = check_rows(n_out, n_in);
  if (s != SPLR_OK) return s;
  if (!dtype_ok(dtype)) return SPLR_ERR_DTYPE;
  if (!aligned16(R) || !aligned16(d) || !aligned16(values) || !aligned16(meta)) return SPLR_ERR_ALIGN;
  return from_hip(
      splr::launch_prune24_pack_scaled(R, d, n_out, n_in, dtype == SPLR_BF16, values, meta, stream));
}

splr_status_t splr_packed_bytes(int64_t n_out, int64_t n_in, splr_dtype_t dtype, size_t* values_bytes,
                                size_t* meta_bytes) {
  if (!values_bytes || !meta_bytes) return SPLR_ERR_NULL;
  splr_status_t s = check_in(n_in);
  if (s == SPLR_OK) s = check_rows(n_out, n_in);
  if (s != SPLR_OK) return s;
  if (!dtype_ok(dtype)) return SPLR_ERR_DTYPE;
  const size_t tiles = (size_t)((n_out + 15) / 16) * (size_t)((n_in + 63) / 64);
  *values_bytes = tiles * 512 * (dtype == SPLR_BF16 ? 2 : 4);
  *meta_bytes = tiles * 32 * sizeof(uint32_t);
  return SPLR_OK;
}

size_t splr_linear_workspace_bytes(int64_t M, int64_t n_out, int64_t n_in, int64_t r, splr_dtype_t dtype) {
  (void)n_out;
  if (M < 1 || check_in(n_in) != SPLR_OK || check_rank(r) != SPLR_OK || !dtype_ok(dtype)) return 0;
  return workspace_bytes(M, n_in, r, dtype);
}

namespace {

// Argument checks shared by splr_linear and its two stages. V is checked only when need_v.
splr_status_t check_linear(const void* X, int64_t M, int64_t n_in, const void* values, const uint32_t* meta,
                           int64_t n_out, const void* U, const void* V, int64_t r, splr_dtype_t dtype, const void* Y,
                           const void* workspace, size_t ws_bytes, bool need_sparse, bool need_v) {
  if (!X) return SPLR_ERR_NULL;
  if (need_sparse && (!values || !meta || !Y || (r > 0 && !U))) return SPLR_ERR_NULL;
  if (need_v && r > 0 && !V) return SPLR_ERR_NULL;
  splr_status_t s = check_in(n_in);
  if (s == SPLR_OK) s = check_rows(M, n_in);
  if (s == SPLR_OK && need_sparse) s = check_rows(n_out, n_in);
  if (s == SPLR_OK) s = check_rank(r);
  if (s == SPLR_OK && need_sparse && M * n_out > kMaxElems) s = SPLR_ERR_SHAPE;
  if (s != SPLR_OK) return s;
  if (!dtype_ok(dtype)) return SPLR_ERR_DTYPE;
  if (!aligned16(X)) return SPLR_ERR_ALIGN;
  if (need_sparse && (!aligned16(values) || !aligned16(meta) || !aligned16(Y) || (r > 0 && !aligned16(U))))
    return SPLR_ERR_ALIGN;
  if (need_v && r > 0 && !aligned16(V)) return SPLR_ERR_ALIGN;
  const size_t need = workspace_bytes(M, n_in, r, dtype);
  if (need > 0 && (!workspace || ws_bytes < need)) return SPLR_ERR_WORKSPACE;
  if (need > 0 && !aligned16(workspace)) return SPLR_ERR_ALIGN;
  return SPLR_OK;
}

splr_status_t run_stage2(const void* X, int64_t M, int64_t n_in, const void* values, const uint32_t* meta,
                         int64_t n_out, const void* U, int64_t r, splr_dtype_t dtype, void* Y, bool y_bf16,
                         void* workspace, hipStream_t stream) {
  if (dtype == SPLR_BF16)
    return from_hip(splr::launch_linear_bf16(X, M, n_in, values, meta, n_out, U, r, (const float*)workspace,
                                             splr::lowrank_slices(M, n_in, r, true), Y, y_bf16, stream));
  return from_hip(splr::launch_linear_f32((const float*)X, M, n_in, (const float*)values, meta, n_out,
                                          (const float*)U, r, (const float*)workspace, Y, y_bf16, stream));
}

}  // namespace

splr_status_t splr_linear(const void* X, int64_t M, int64_t n_in, const void* values, const uint32_t* meta,
                          int64_t n_out, const void* U, const void* V, int64_t r, splr_dtype_t dtype, float* Y,
                          void* workspace, size_t ws_bytes, hipStream_t stream) {
  const splr_status_t s =
      check_linear(X, M, n_in, values, meta, n_out, U, V, r, dtype, Y, workspace, ws_bytes, true, true);
  if (s != SPLR_OK) return s;
  if (splr::launch_lowrank(X, V, M, n_in, r, dtype == SPLR_BF16, workspace, stream) != hipSuccess)
    return SPLR_ERR_HIP;
  return run_stage2(X, M, n_in, values, meta, n_out, U, r, dtype, Y, false, workspace, stream);
}

splr_status_t splr_linear_ex(const void* X, int64_t M, int64_t n_in, const void* values, const uint32_t* meta,
                             int64_t n_out, const void* U, const void* V, int64_t r, splr_dtype_t dtype,
                             splr_dtype_t y_dtype, void* Y, void* workspace, size_t ws_bytes, hipStream_t stream) {
  const splr_status_t s =
      check_linear(X, M, n_in, values, meta, n_out, U, V, r, dtype, Y, workspace, ws_bytes, true, true);
  if (s != SPLR_OK) return s;
  if (!dtype_ok(y_dtype)) return SPLR_ERR_DTYPE;
  if (splr::launch_lowrank(X, V, M, n_in, r, dtype == SPLR_BF16, workspace, stream) != hipSuccess)
    return SPLR_ERR_HIP;
  return run_stage2(X, M, n_in, values, meta, n_out, U, r, dtype, Y, y_dtype == SPLR_BF16, workspace, stream);
}

splr_status_t splr_linear_stage1(const void* X, int64_t M, int64_t n_in, const void* V, int64_t r,
                                 splr_dtype_t dtype, void* workspace, size_t ws_bytes, hipStream_t stream) {
  const splr_status_t s =
      check_linear(X, M, n_in, nullptr, nullptr, 0, nullptr, V, r, dtype, nullptr, workspace, ws_bytes, false, true);
  if (s != SPLR_OK) return s;
  return from_hip(splr::launch_lowrank(X, V, M, n_in, r, dtype == SPLR_BF16, workspace, stream));
}

splr_status_t splr_linear_stage2(const void* X, int64_t M, int64_t n_in, const void* values, const uint32_t* meta,
                                 int64_t n_out, const void* U, int64_t r, splr_dtype_t dtype, float* Y,
                                 const void* workspace, size_t ws_bytes, hipStream_t stream) {
  const splr_status_t s =
      check_linear(X, M, n_in, values, meta, n_out, U, nullptr, r, dtype, Y, workspace, ws_bytes, true, false);
  if (s != SPLR_OK) return s;
  return run_stage2(X, M, n_in, values, meta, n_out, U, r, dtype, Y, false, const_cast<void*>(workspace), stream);
}

splr_status_t splr_dense_reconstruct(const void* values, const uint32_t* meta, const void* U, const void* V,
                                     int64_t n_out, int64_t n_in, int64_t r, splr_dtype_t dtype, float* W_hat,
                                     hipStream_t stream) {
  if (!values || !meta || !W_hat) return SPLR_ERR_NULL;
  if (r > 0 && (!U || !V)) return SPLR_ERR_NULL;
  splr_status_t s = check_in(n_in);
  if (s == SPLR_OK) s = check_rows(n_out, n_in);
  if (s == SPLR_OK) s = check_rank(r);
  if (s != SPLR_OK) return s;
  if (!dtype_ok(dtype)) return SPLR_ERR_DTYPE;
  if (!aligned16(values) || !aligned16(meta) || !aligned16(W_hat)) return SPLR_ERR_ALIGN;
  if (r > 0 && (!aligned16(U) || !aligned16(V))) return SPLR_ERR_ALIGN;
  return from_hip(splr::launch_dense_reconstruct(values, meta, U, V, n_out, n_in, r, dtype == SPLR_BF16, W_hat,
                                                 stream));
}

const char* splr_status_string(splr_status_t status) {
  switch (status) {
    case SPLR_OK: return "SPLR_OK";
    case SPLR_ERR_NULL: return "SPLR_ERR_NULL: a required pointer is NULL";
    case SPLR_ERR_SHAPE: return "SPLR_ERR_SHAPE: a size is out of range";
    case SPLR_ERR_DTYPE: return "SPLR_ERR_DTYPE: unknown dtype";
    case SPLR_ERR_ALIGN: return "SPLR_ERR_ALIGN: a pointer is not 16-byte aligned";
    case SPLR_ERR_HIP: return "SPLR_ERR_HIP: the HIP runtime reported an error";
    case SPLR_ERR_WORKSPACE: return "SPLR_ERR_WORKSPACE: workspace missing or too small";
  }
  return "SPLR_ERR_UNKNOWN";
}

const char* splr_version(void) { return "0.1.0"; }

}  // extern "C"
