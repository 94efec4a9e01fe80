// C ABI of libsplr (declared in include/splr.h): argument validation, workspace sizing and
// kernel dispatch.  Every check runs before the first HIP call, so a rejected call enqueues
// nothing; the library holds no mutable state and never allocates device memory.
#include "splr.h"

#include <mutex>

#include "common.hpp"
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
  if (!splr::pack_grids_fit(n_out, n_in, dtype == SPLR_BF16)) return SPLR_ERR_SHAPE;
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
  if (!splr::pack_grids_fit(n_out, n_in, dtype == SPLR_BF16)) return SPLR_ERR_SHAPE;
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
  if (!splr::residual_grids_fit(n_out, n_in)) return SPLR_ERR_SHAPE;
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
  if (!splr::pack_grids_fit(n_out, n_in, dtype == SPLR_BF16)) return SPLR_ERR_SHAPE;
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
  const size_t TR = (size_t)((n_out + 15) / 16), TK = (size_t)((n_in + 63) / 64);
  *values_bytes = TR * TK * 512 * (dtype == SPLR_BF16 ? 2 : 4);
  *meta_bytes = TR * (size_t)splr::meta_blocks((int)TK) * 1024;
  return SPLR_OK;
}

size_t splr_linear_workspace_bytes(int64_t M, int64_t n_out, int64_t n_in, int64_t r, splr_dtype_t dtype) {
  (void)n_out;
  if (M < 1 || check_in(n_in) != SPLR_OK || check_rank(r) != SPLR_OK || !dtype_ok(dtype)) return 0;
  return workspace_bytes(M, n_in, r, dtype);
}

namespace {

// Argument checks shared by splr_linear and its two stages. V is checked only when need_v, the
// caller's workspace only when check_ws.
splr_status_t check_linear(const void* X, int64_t M, int64_t n_in, const void* values, const uint32_t* meta,
                           int64_t n_out, const void* U, const void* V, int64_t r, splr_dtype_t dtype, const void* Y,
                           const void* workspace, size_t ws_bytes, bool need_sparse, bool need_v,
                           bool check_ws = true) {
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
  // every launch of the call fits the dispatch limits (stage 2 only when it runs)
  if (need_sparse ? !splr::linear_grids_fit(M, n_in, n_out, r, dtype == SPLR_BF16)
                  : !splr::lowrank_grids_fit(M, n_in, r, dtype == SPLR_BF16))
    return SPLR_ERR_SHAPE;
  if (!aligned16(X)) return SPLR_ERR_ALIGN;
  if (need_sparse && (!aligned16(values) || !aligned16(meta) || !aligned16(Y) || (r > 0 && !aligned16(U))))
    return SPLR_ERR_ALIGN;
  if (need_v && r > 0 && !aligned16(V)) return SPLR_ERR_ALIGN;
  if (!check_ws) return SPLR_OK;
  const size_t need = workspace_bytes(M, n_in, r, dtype);
  if (need > 0 && (!workspace || ws_bytes < need)) return SPLR_ERR_WORKSPACE;
  if (need > 0 && !aligned16(workspace)) return SPLR_ERR_ALIGN;
  return SPLR_OK;
}

splr_status_t run_stage2(const void* X, int64_t M, int64_t n_in, const void* values, const uint32_t* meta,
                         int64_t n_out, const void* U, int64_t r, splr_dtype_t dtype, void* Y, bool y_bf16,
                         void* workspace, hipStream_t stream) {
  if (dtype == SPLR_BF16 && M <= splr::kDecodeMaxTokens)
    return from_hip(splr::launch_linear_decode(X, M, n_in, values, meta, n_out, U, r, (const float*)workspace,
                                               splr::lowrank_slices(M, n_in, r, true), Y, y_bf16, stream));
  if (dtype == SPLR_BF16)
    return from_hip(splr::launch_linear_bf16(X, M, n_in, values, meta, n_out, U, r, (const float*)workspace,
                                             splr::lowrank_slices(M, n_in, r, true), Y, y_bf16, stream));
  return from_hip(splr::launch_linear_f32((const float*)X, M, n_in, (const float*)values, meta, n_out,
                                          (const float*)U, r, (const float*)workspace, Y, y_bf16, stream));
}

// Layers of one shape: every layer is checked as splr_linear (or its stage 2) checks it before the
// first HIP call; with stage 1 (with_stage1) each layer's T goes to its own workspace, then the
// stage-2 products run as one launch when the prefill kernel takes them, else layer by layer.
splr_status_t run_group(int32_t count, const void* const* X, int64_t M, int64_t n_in, const void* const* values,
                        const uint32_t* const* meta, int64_t n_out, const void* const* U, const void* const* V,
                        int64_t r, splr_dtype_t dtype, float* const* Y, const void* const* workspace,
                        size_t ws_bytes, bool with_stage1, hipStream_t stream) {
  static_assert(SPLR_GROUP_MAX == splr::kMaxGroup, "header and library agree");
  if (count < 1 || count > splr::kMaxGroup) return SPLR_ERR_SHAPE;
  if (!X || !values || !meta || !Y || !workspace || (r > 0 && !U) || (with_stage1 && r > 0 && !V))
    return SPLR_ERR_NULL;
  for (int32_t i = 0; i < count; ++i) {
    const splr_status_t s =
        check_linear(X[i], M, n_in, values[i], meta[i], n_out, r > 0 ? U[i] : nullptr,
                     with_stage1 && r > 0 ? V[i] : nullptr, r, dtype, Y[i], workspace[i], ws_bytes, true, with_stage1);
    if (s != SPLR_OK) return s;
  }
  const bool grouped = dtype == SPLR_BF16 && M > splr::kDecodeMaxTokens;
  if (grouped && !splr::linear_group_grid_fits(M, n_out, count)) return SPLR_ERR_SHAPE;
  if (with_stage1)
    for (int32_t i = 0; i < count; ++i)
      if (splr::launch_lowrank(X[i], V ? V[i] : nullptr, M, n_in, r, dtype == SPLR_BF16, const_cast<void*>(workspace[i]),
                               stream) != hipSuccess)
        return SPLR_ERR_HIP;
  if (!grouped) {
    for (int32_t i = 0; i < count; ++i) {
      const splr_status_t s = run_stage2(X[i], M, n_in, values[i], meta[i], n_out, r > 0 ? U[i] : nullptr, r, dtype,
                                         Y[i], false, const_cast<void*>(workspace[i]), stream);
      if (s != SPLR_OK) return s;
    }
    return SPLR_OK;
  }
  const void* u[splr::kMaxGroup];
  const float* t[splr::kMaxGroup];
  void* y[splr::kMaxGroup];
  for (int32_t i = 0; i < count; ++i) {
    u[i] = r > 0 ? U[i] : nullptr;
    t[i] = (const float*)workspace[i];
    y[i] = Y[i];
  }
  return from_hip(splr::launch_linear_bf16_group(count, X, M, n_in, values, meta, n_out, u, r, t,
                                                 splr::lowrank_slices(M, n_in, r, true), y, false, stream));
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

splr_status_t splr_linear_stage2_dense(const void* X, int64_t M, int64_t n_in, const void* values,
                                       const uint32_t* meta, int64_t n_out, const void* U, int64_t r,
                                       splr_dtype_t dtype, float* Y, const void* workspace, size_t ws_bytes,
                                       hipStream_t stream) {
  const splr_status_t s =
      check_linear(X, M, n_in, values, meta, n_out, U, nullptr, r, dtype, Y, workspace, ws_bytes, true, false);
  if (s != SPLR_OK) return s;
  if (dtype != SPLR_BF16) return SPLR_ERR_DTYPE;
  if (!splr::linear_dense_grids_fit(M, n_out)) return SPLR_ERR_SHAPE;
  return from_hip(splr::launch_linear_bf16_dense(X, M, n_in, values, meta, n_out, U, r, (const float*)workspace,
                                                 splr::lowrank_slices(M, n_in, r, true), Y, stream));
}

splr_status_t splr_linear_stage2_group(int32_t count, const void* const* X, int64_t M, int64_t n_in,
                                       const void* const* values, const uint32_t* const* meta, int64_t n_out,
                                       const void* const* U, int64_t r, splr_dtype_t dtype, float* const* Y,
                                       const void* const* workspace, size_t ws_bytes, hipStream_t stream) {
  return run_group(count, X, M, n_in, values, meta, n_out, U, nullptr, r, dtype, Y, workspace, ws_bytes, false,
                   stream);
}

splr_status_t splr_linear_group(int32_t count, const void* const* X, int64_t M, int64_t n_in,
                                const void* const* values, const uint32_t* const* meta, int64_t n_out,
                                const void* const* U, const void* const* V, int64_t r, splr_dtype_t dtype,
                                float* const* Y, void* const* workspace, size_t ws_bytes, hipStream_t stream) {
  return run_group(count, X, M, n_in, values, meta, n_out, U, V, r, dtype, Y, (const void* const*)workspace,
                   ws_bytes, true, stream);
}

}  // extern "C"

// ---------------------------------------------------------------- splr_linear_noalloc
// For callers that cannot allocate: the first-stage workspace lives in a file-scope device array.
// Each GPU the library runs on holds its own copy (from the first call on it until the process
// ends), at its own address, found once per device with hipGetSymbolAddress. In host code the
// array's name is only a stand-in for the symbol; kernels get the looked-up device address.
namespace {

constexpr size_t kScratchBytes = size_t(32) << 20;  // SPLR_LINEAR_NOALLOC_MAX_WORKSPACE in splr.h
static_assert(kScratchBytes == SPLR_LINEAR_NOALLOC_MAX_WORKSPACE, "header and library agree");
__device__ __align__(256) uint8_t scratch[kScratchBytes];

constexpr int kMaxDevices = 64;
std::mutex g_scratch_mu;
void* g_scratch_ptr[kMaxDevices];

// This device's copy of `scratch`, looked up on the first call with that device current.
hipError_t device_scratch(void** out) {
  int dev = -1;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return e;
  if (dev < 0 || dev >= kMaxDevices) return hipErrorInvalidDevice;
  std::lock_guard<std::mutex> lock(g_scratch_mu);
  if (!g_scratch_ptr[dev]) {
    void* p = nullptr;
    e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    if (e != hipSuccess) return e;
    if (!p) return hipErrorInvalidSymbol;
    g_scratch_ptr[dev] = p;
  }
  *out = g_scratch_ptr[dev];
  return hipSuccess;
}

}  // namespace

extern "C" {

splr_status_t splr_linear_noalloc(const void* X, int64_t M, int64_t n_in, const void* values, const uint32_t* meta,
                                  int64_t n_out, const void* U, const void* V, int64_t r, splr_dtype_t dtype, float* Y,
                                  hipStream_t stream) {
  const splr_status_t s =
      check_linear(X, M, n_in, values, meta, n_out, U, V, r, dtype, Y, nullptr, 0, true, true, false);
  if (s != SPLR_OK) return s;
  const size_t need = workspace_bytes(M, n_in, r, dtype);
  if (need > kScratchBytes) return SPLR_ERR_SCRATCH;
  void* ws = nullptr;
  if (need > 0 && device_scratch(&ws) != hipSuccess) return SPLR_ERR_HIP;
  // the same kernels as splr_linear; the workspace needs no clearing (every byte the second stage
  // reads is written by the first stage of this call)
  if (splr::launch_lowrank(X, V, M, n_in, r, dtype == SPLR_BF16, ws, stream) != hipSuccess) return SPLR_ERR_HIP;
  return run_stage2(X, M, n_in, values, meta, n_out, U, r, dtype, Y, false, ws, stream);
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
  if (!splr::reconstruct_grids_fit(n_out, n_in)) return SPLR_ERR_SHAPE;
  if (!aligned16(values) || !aligned16(meta) || !aligned16(W_hat)) return SPLR_ERR_ALIGN;
  if (r > 0 && (!aligned16(U) || !aligned16(V))) return SPLR_ERR_ALIGN;
  return from_hip(splr::launch_dense_reconstruct(values, meta, U, V, n_out, n_in, r, dtype == SPLR_BF16, W_hat,
                                                 stream));
}

size_t splr_gram_workspace_bytes(int64_t n, int64_t k) {
  if (n < 1 || n > kMaxCols || k < 1 || k > splr::kMaxCholK) return 0;
  return round_up(splr::gram_workspace_bytes(n, k), 256);
}

splr_status_t splr_gram_f64(const float* Y, int64_t n, int64_t k, double* G, void* workspace,
                            size_t workspace_bytes, hipStream_t stream) {
  if (!Y || !G) return SPLR_ERR_NULL;
  if (n < 1 || n > kMaxCols || k < 1 || k > splr::kMaxCholK) return SPLR_ERR_SHAPE;
  if (!workspace || workspace_bytes < splr_gram_workspace_bytes(n, k)) return SPLR_ERR_WORKSPACE;
  if ((reinterpret_cast<uintptr_t>(Y) & 3u) || (reinterpret_cast<uintptr_t>(G) & 7u) ||
      (reinterpret_cast<uintptr_t>(workspace) & 7u))
    return SPLR_ERR_ALIGN;
  return from_hip(splr::launch_gram_f64(Y, n, k, G, workspace, stream));
}

splr_status_t splr_chol_rinv(const double* G, int64_t k, float* Rinv, hipStream_t stream) {
  if (!G || !Rinv) return SPLR_ERR_NULL;
  if (k < 1 || k > splr::kMaxCholK) return SPLR_ERR_SHAPE;
  if ((reinterpret_cast<uintptr_t>(G) & 7u) || (reinterpret_cast<uintptr_t>(Rinv) & 3u)) return SPLR_ERR_ALIGN;
  return from_hip(splr::launch_chol_rinv(G, k, Rinv, stream));
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
    case SPLR_ERR_SCRATCH:
      return "SPLR_ERR_SCRATCH: the call needs more workspace than splr_linear_noalloc's built-in buffer holds";
  }
  return "SPLR_ERR_UNKNOWN";
}

// The library version, followed by the first 16 hex digits of the SHA-256 of the sources it was
// built from (the build passes it in), so a loaded binary can be matched to a source tree.
#ifndef SPLR_SOURCE_SHA
#define SPLR_SOURCE_SHA "unknown"
#endif
const char* splr_version(void) { return "0.2.0+" SPLR_SOURCE_SHA; }

}  // extern "C"
