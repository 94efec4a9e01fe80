/*
 * splr.h -- C ABI of libsplr.so: the 2:4 sparse + rank-r linear layer on AMD MI355X (gfx950).
 *
 * The layer approximates a weight W [n_out x n_in] by S + U V, where S keeps at most two of every
 * four consecutive weights along the input dimension and U [n_out x r], V [r x n_in] are thin
 * factors (LoSparse page, §3; 3BASiL article, "Splitting each weight matrix into two parts" and
 * "A three-block ADMM replaces alternating minimization").  The forward pass evaluates the sparse
 * product and the low-rank product side by side and adds them (LoSparse §3.2); in the orientation
 * used here that is  Y = X S^T + (X V^T) U^T.
 *
 * General rules for every entry point
 * -----------------------------------
 *  - Array arguments are DEVICE pointers (hipMalloc / torch CUDA tensors), row-major, contiguous,
 *    16-byte aligned.  The caller owns every buffer; the library never allocates or frees device
 *    memory (its one buffer, splr_linear_noalloc's workspace, is a static device array, see
 *    there).  Outputs must not alias inputs.
 *  - Work is enqueued on `stream` (0 = the null stream) and the call returns without waiting.
 *  - Arguments are validated before any HIP call: on a validation error nothing is enqueued and
 *    the error code is returned.  A failed launch returns SPLR_ERR_HIP.  No C++ exception crosses
 *    the boundary.
 *  - Storage types: SPLR_FP32 = IEEE binary32, SPLR_BF16 = bfloat16 (upper half of a binary32).
 *    The same dtype applies to every floating-point input of one call; Y and W_hat are float32.
 *  - n_in must be a positive multiple of 32 (a metadata word covers 32 input columns).
 *
 * Packed 2:4 layout (shared by every entry point)
 * -----------------------------------------------
 * The pages fix no storage format; this one is laid out for gfx950's structured-sparse MFMA
 * (v_smfmac_f32_16x16x64_bf16), so that one wave reads one operand fragment as 1 KiB of
 * contiguous memory. S is cut into tiles of 16 rows x 64 input columns, TR = ceil(n_out/16) tile
 * rows by TK = ceil(n_in/64) tile columns, tile (tr, tk) at index t = tr*TK + tk.
 *  values: t-major, 64 slots of 8 entries per tile (TR*TK*512 entries of dtype). Row n, group g
 *          (columns 4g..4g+3): gi = g % 16, slot L = n % 16 + 16*(gi / 4); its two kept entries,
 *          in ascending column order, are entries 2*(gi % 4) and 2*(gi % 4)+1 of slot L.
 *  meta:   blocks of 8 consecutive tile columns of one tile row, TKB = ceil(TK/8) per tile row,
 *          block (tr, tb) at index tr*TKB + tb, 1 KiB (256 uint32 words) each: TR*TKB*256 words.
 *          Slot L of a block owns words 4L .. 4L+3, i.e. eight 16-bit units; unit u is the low
 *          (u even) or high (u odd) half of word 4L + u/2 and belongs to tile column 8*tb + u.
 *          The unit of slot L = n % 16 + 16*(gi / 4) in tile (tr, tk) holds the nibbles of
 *          groups gi with gi / 4 = L / 16 of row n, group gi at bits 4*(gi % 4); a nibble is
 *          (a | b << 2), where a < b in {0,1,2,3} are the kept positions. Valid nibbles: 0x4 0x8
 *          0xC 0x9 0xD 0xE. (One 16-byte load gives a lane the indices of 8 tiles, and a 32-bit
 *          word is the index operand of two steps of the structured-sparse MFMA.)
 *  Entries and nibbles outside the matrix (row padding n >= n_out, column padding k >= n_in)
 *  are zero. splr_packed_bytes() gives both buffer sizes. Metadata not produced by
 *  splr_prune24_pack gives unspecified results (it is not validated).
 */
#ifndef SPLR_H_
#define SPLR_H_

#include <stddef.h>
#include <stdint.h>

#include <hip/hip_runtime_api.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum { SPLR_FP32 = 0, SPLR_BF16 = 1 } splr_dtype_t;

typedef enum {
  SPLR_OK = 0,
  SPLR_ERR_NULL = 1,      /* a required pointer is NULL                                         */
  SPLR_ERR_SHAPE = 2,     /* a size is out of range (see each entry point)                      */
  SPLR_ERR_DTYPE = 3,     /* unknown splr_dtype_t                                               */
  SPLR_ERR_ALIGN = 4,     /* a pointer is not 16-byte aligned                                   */
  SPLR_ERR_HIP = 5,       /* the HIP runtime reported an error while enqueueing                 */
  SPLR_ERR_WORKSPACE = 6, /* workspace NULL or smaller than splr_linear_workspace_bytes()      */
  SPLR_ERR_SCRATCH = 7    /* splr_linear_noalloc: the call needs more than its built-in buffer  */
} splr_status_t;

/*
 * splr_prune24_pack -- Euclidean projection of a dense matrix onto the 2:4 set, then packing.
 *
 * This is the sparse step of the alternating-minimisation / ADMM decompositions: with an identity
 * Hessian, hard thresholding solves it exactly (HASSLE-free page, §4.1.1); the constraint allows at
 * most two nonzeros in every four consecutive weights (3BASiL article, "A three-block ADMM replaces
 * alternating minimization").  R is typically the residual W - U V.
 *
 * For each row and each group of four consecutive columns the two entries of largest magnitude
 * are kept as bit copies.  Magnitude is compared as the bit pattern with the sign cleared: +0 and
 * -0 tie, subnormals are ordered exactly, infinities outrank finite values, NaNs outrank
 * infinities (by payload).  Equal magnitudes go to the lower column.  The result is bit-exact and
 * deterministic.
 *
 *   R      [n_out][n_in] dtype, row-major       input
 *   values, meta                               output, packed layout above (every entry written,
 *                                              padding included)
 * Errors: NULL pointer -> SPLR_ERR_NULL; n_out < 1, n_in < 32 or n_in % 32 != 0 -> SPLR_ERR_SHAPE;
 *         bad dtype -> SPLR_ERR_DTYPE; misaligned pointer -> SPLR_ERR_ALIGN.
 */
splr_status_t splr_prune24_pack(const void* R, int64_t n_out, int64_t n_in, splr_dtype_t dtype,
                                void* values, uint32_t* meta, hipStream_t stream);

/*
 * splr_prune_nm_pack -- Euclidean projection onto an N:M set, stored in the 2:4 packed layout.
 *
 * N:M sparsity keeps at most n of every m consecutive weights (HASSLE-free page, §1 and §2: the
 * framework targets N:M sparsity; 3BASiL article, "A three-block ADMM replaces alternating
 * minimization": N:M structures such as 2:4, and the 2:8 + rank-64 configuration after LoRA
 * fine-tuning); with an identity Hessian the projection is hard thresholding (HASSLE-free §4.1.1).
 * For each row and each group of m consecutive columns the n entries of largest magnitude are kept
 * as bit copies (magnitude and ties exactly as in splr_prune24_pack: equal magnitudes go to the
 * lower column) and the others become +0; the result is then packed exactly as splr_prune24_pack
 * packs it.  With n <= 2 and m a multiple of 4, no aligned group of four holds more than two
 * nonzeros, so the packed S is exactly the N:M matrix and splr_linear computes with it unchanged
 * (patterns denser than 2:4 somewhere, e.g. 4:8, do not fit the 2:4 operand and are rejected).
 * n = 2, m = 4 is splr_prune24_pack itself.  Bit-exact and deterministic.
 *
 *   R      [n_out][n_in] dtype, row-major       input
 *   n, m   n in {1, 2}, m in {4, 8, 16}
 *   values, meta                               output, packed layout above
 * Errors: NULL pointer -> SPLR_ERR_NULL; n_out < 1, n_in < 32, n_in % 32 != 0, or (n, m) outside
 *         the sets above -> SPLR_ERR_SHAPE; bad dtype -> SPLR_ERR_DTYPE; misaligned pointer ->
 *         SPLR_ERR_ALIGN.
 */
splr_status_t splr_prune_nm_pack(const void* R, int64_t n_out, int64_t n_in, int32_t n, int32_t m,
                                 splr_dtype_t dtype, void* values, uint32_t* meta, hipStream_t stream);

/*
 * splr_prune24_pack_residual -- residual R = W - U V formed in the kernel, then projected and packed
 * exactly as splr_prune24_pack does (R never goes to memory).
 *
 * The sparse step of the alternating-minimisation / ADMM decompositions acts on the weight minus
 * the current low-rank part (HASSLE-free page, §4 and §4.1.1), and repeats at every iteration.
 * Pinned arithmetic (bit-exact): per entry acc = W[n][k] as binary32, then for j = 0, 1, ..., r-1
 * in that order acc = fma(-U[n][j], V[j][k], acc) (one rounding per step), then the storage type
 * (bfloat16: round to nearest even).  A NaN result is stored as the canonical quiet NaN
 * (0x7FC00000 / 0x7FC0).  r == 0 packs W itself.
 *
 *   W      [n_out][n_in] dtype    U [n_out][r] dtype    V [r][n_in] dtype (U, V NULL iff r == 0)
 *   values, meta                  output, packed layout above
 * Vector-ALU bound: r fused multiply-adds per weight.
 * Errors: NULL pointer -> SPLR_ERR_NULL; n_out < 1, n_in < 32, n_in % 32 != 0, r < 0 or r > 1024 ->
 *         SPLR_ERR_SHAPE; bad dtype -> SPLR_ERR_DTYPE; misaligned pointer -> SPLR_ERR_ALIGN.
 */
splr_status_t splr_prune24_pack_residual(const void* W, const void* U, const void* V, int64_t n_out,
                                         int64_t n_in, int64_t r, splr_dtype_t dtype, void* values,
                                         uint32_t* meta, hipStream_t stream);

/*
 * splr_prune24_pack_scaled -- activation-aware (diagonal-Hessian) 2:4 projection, then packing.
 *
 * With a diagonal Hessian the sparse step hard-thresholds the residual after scaling input column
 * k by d_k, which gives Wanda's score |W_ij| * ||X_j|| (HASSLE-free page, §4.1.2); the entries kept
 * are the residual's own.  Typically d_k is the 2-norm of column k of the calibration activations.
 *
 * For each row and each group of four consecutive columns the two entries of largest score
 * |R[n][k]| * |d[k]| are kept as bit copies.  The score is the exact product (formed in binary64,
 * which holds the product of two binary32 values exactly), so no rounding decides a choice; equal
 * scores go to the lower column; NaN scores (NaN entry or scale, infinity times zero) all tie and
 * outrank every number.  With d == 1 everywhere the result equals splr_prune24_pack's for inputs
 * with at most one NaN per group.  Bit-exact and deterministic.
 *
 *   R      [n_out][n_in] dtype, row-major       input
 *   d      [n_in] float32                        per-column scales (any sign; |d| is used)
 *   values, meta                                output, packed layout above
 * Errors: as splr_prune24_pack; d NULL -> SPLR_ERR_NULL, misaligned d -> SPLR_ERR_ALIGN.
 */
splr_status_t splr_prune24_pack_scaled(const void* R, const float* d, int64_t n_out, int64_t n_in,
                                       splr_dtype_t dtype, void* values, uint32_t* meta,
                                       hipStream_t stream);

/*
 * splr_packed_bytes -- sizes of the packed values and metadata buffers for an n_out x n_in S.
 * Returns SPLR_ERR_SHAPE / SPLR_ERR_DTYPE / SPLR_ERR_NULL like the other entry points.
 */
splr_status_t splr_packed_bytes(int64_t n_out, int64_t n_in, splr_dtype_t dtype, size_t* values_bytes,
                                size_t* meta_bytes);

/*
 * splr_linear_workspace_bytes -- device workspace that splr_linear needs for these sizes
 * (0 when none).  It holds the first low-rank stage T = X V^T as float32 partial sums over at most
 * 16 slices of n_in (one slice for fp32).  Everything a call reads from it is written by the same
 * call, so it needs no initialisation and may be reused by calls of any shape that fit.
 */
size_t splr_linear_workspace_bytes(int64_t M, int64_t n_out, int64_t n_in, int64_t r,
                                   splr_dtype_t dtype);

/*
 * splr_linear -- Y = X S^T + (X V^T) U^T  (LoSparse §3.2: both products, summed).
 *
 *   X      [M][n_in] dtype                       activations
 *   values, meta                                 packed S (layout above)
 *   U      [n_out][r] dtype, V [r][n_in] dtype   thin factors; both may be NULL iff r == 0
 *   Y      [M][n_out] float32                    output, written once
 *   workspace / workspace_bytes                  device scratch of at least
 *                                                splr_linear_workspace_bytes(...) bytes (may be
 *                                                NULL when that is 0); contents need not be
 *                                                initialised and are clobbered.
 * Arithmetic: products of dtype operands accumulated in float32.  With SPLR_BF16 the first
 * low-rank stage T is kept to about 16 significant bits (a bfloat16 high part plus a bfloat16
 * correction), never rounded to a single bfloat16.  Results are bitwise reproducible run to run
 * (fixed reduction order, no floating-point atomics).
 * Errors: NULL pointer -> SPLR_ERR_NULL; M < 1, n_out < 1, n_in < 32, n_in % 32 != 0, r < 0,
 *         r > 1024 or r % 16 != 0 -> SPLR_ERR_SHAPE; bad dtype -> SPLR_ERR_DTYPE; misaligned
 *         pointer -> SPLR_ERR_ALIGN; workspace too small -> SPLR_ERR_WORKSPACE.
 */
splr_status_t splr_linear(const void* X, int64_t M, int64_t n_in, const void* values,
                          const uint32_t* meta, int64_t n_out, const void* U, const void* V,
                          int64_t r, splr_dtype_t dtype, float* Y, void* workspace,
                          size_t workspace_bytes, hipStream_t stream);

/*
 * splr_linear_ex -- splr_linear with a choice of output type: y_dtype SPLR_FP32 gives splr_linear's
 * Y; SPLR_BF16 stores each float32 result rounded to bfloat16 (to nearest even; NaN stays a quiet
 * NaN), so Y [M][n_out] is 2-byte entries and half the bytes to write.  The rounding is the only
 * difference: a bfloat16 Y is, bit for bit, the round-to-nearest-even of the float32 Y of the same
 * call.
 * Errors: as splr_linear; unknown y_dtype -> SPLR_ERR_DTYPE.
 */
splr_status_t splr_linear_ex(const void* X, int64_t M, int64_t n_in, const void* values,
                             const uint32_t* meta, int64_t n_out, const void* U, const void* V,
                             int64_t r, splr_dtype_t dtype, splr_dtype_t y_dtype, void* Y,
                             void* workspace, size_t workspace_bytes, hipStream_t stream);

/*
 * splr_linear_stage1 / splr_linear_stage2 -- the two stages of splr_linear, for callers that want
 * to schedule them apart (for example stage 1 on another stream while the residual is packed).
 * splr_linear(...) is exactly stage1 followed by stage2 on one stream with one workspace.
 *
 *   stage1: T = X V^T into `workspace` (the first low-rank stage; nothing else is read or
 *           written).  No-op when r == 0.
 *   stage2: Y = X S^T + T U^T, reading T from `workspace` as left there by stage1 with the same
 *           X, M, n_in, r and dtype (stage2 does not read V).
 * The workspace must stay untouched between the two stages, and stage2 must be ordered after
 * stage1 (same stream, or an event).  Arguments mean what they mean for splr_linear; V may be NULL
 * for stage2 and values, meta, U, Y are not used by stage1.
 * Errors: as splr_linear, for the arguments that stage uses.
 */
splr_status_t splr_linear_stage1(const void* X, int64_t M, int64_t n_in, const void* V, int64_t r,
                                 splr_dtype_t dtype, void* workspace, size_t workspace_bytes,
                                 hipStream_t stream);
splr_status_t splr_linear_stage2(const void* X, int64_t M, int64_t n_in, const void* values,
                                 const uint32_t* meta, int64_t n_out, const void* U, int64_t r,
                                 splr_dtype_t dtype, float* Y, const void* workspace,
                                 size_t workspace_bytes, hipStream_t stream);

/*
 * splr_linear_stage2_dense -- splr_linear_stage2 with the sparse product X S^T computed the other
 * way gfx950 can run it: each lane expands its packed S operand (the two kept values of every group
 * of four and their positions) to dense bfloat16 in registers, and dense MFMAs
 * (v_mfma_f32_16x16x32_bf16, twice as many as structured-sparse ones) multiply it with the same
 * LDS-staged X tiles; S is decompressed on chip only, never written out.  Tiles, loads, rank-r
 * epilogue and Y store are those of the prefill kernel with the 512-row tile (its 256-row form,
 * four waves, when 512-row tiles would leave CUs idle), for every M.  The layer product itself is
 * the one splr_linear computes (LoSparse page, §3.2); this entry exists as the measured alternative
 * to the structured-sparse instruction, which splr_linear uses.
 *
 *   Arguments: as splr_linear_stage2 (T from splr_linear_stage1 in `workspace`).
 *   Arithmetic: the same bfloat16 products accumulated in float32, summed in another order than
 *          splr_linear_stage2, so the two agree to rounding (bit for bit where every partial sum is
 *          exact, e.g. small-integer inputs).  Bitwise reproducible run to run.
 * Errors: as splr_linear_stage2; dtype other than SPLR_BF16 -> SPLR_ERR_DTYPE.
 */
splr_status_t splr_linear_stage2_dense(const void* X, int64_t M, int64_t n_in, const void* values,
                                       const uint32_t* meta, int64_t n_out, const void* U, int64_t r,
                                       splr_dtype_t dtype, float* Y, const void* workspace,
                                       size_t workspace_bytes, hipStream_t stream);

/*
 * splr_linear_group / splr_linear_stage2_group -- splr_linear (or its stage 2) for `count` layers
 * of one shape at once, e.g. the two 1024-output projections of an attention block, whose forward
 * passes are each the sum of the sparse and the low-rank product (LoSparse page, §3.2).  Stage 2
 * of all the layers runs as one launch of the prefill kernel whose grid holds every layer's tiles,
 * so layers too small to give each compute unit a 512-row tile on their own can still use that
 * tile (k_proj and v_proj of a Llama-3-8B block at 8192 tokens: 128 tiles each, 256 together).
 *
 *   Arguments: host arrays of `count` device pointers (X, values, meta, U, V, Y, workspace), entry
 *          i belonging to layer i; the sizes M, n_in, n_out, r and the dtype are shared, and each
 *          layer's buffers mean what they mean for splr_linear.  U and V may be NULL (the arrays)
 *          iff r == 0.  Every layer has its own workspace of at least `workspace_bytes`
 *          (splr_linear_workspace_bytes of the shared sizes); the stage-2 form reads T there as
 *          splr_linear_stage1 of that layer left it.  Outputs must not alias each other or any
 *          input.
 *   Results: Y[i] bit for bit what splr_linear (or splr_linear_stage2) gives for layer i alone.
 *          splr_linear_group runs stage 1 of each layer in turn, then the grouped stage 2.  For
 *          M <= 64 tokens and for float32 the layers run one after the other (the decode and
 *          float32 kernels take a layer per launch).
 * Errors: count outside 1..SPLR_GROUP_MAX -> SPLR_ERR_SHAPE; a NULL array -> SPLR_ERR_NULL;
 *         otherwise as splr_linear for each layer (every layer checked before any HIP call).
 */
#define SPLR_GROUP_MAX 4
splr_status_t splr_linear_group(int32_t count, const void* const* X, int64_t M, int64_t n_in,
                                const void* const* values, const uint32_t* const* meta, int64_t n_out,
                                const void* const* U, const void* const* V, int64_t r, splr_dtype_t dtype,
                                float* const* Y, void* const* workspace, size_t workspace_bytes,
                                hipStream_t stream);
splr_status_t splr_linear_stage2_group(int32_t count, const void* const* X, int64_t M, int64_t n_in,
                                       const void* const* values, const uint32_t* const* meta, int64_t n_out,
                                       const void* const* U, int64_t r, splr_dtype_t dtype, float* const* Y,
                                       const void* const* workspace, size_t workspace_bytes,
                                       hipStream_t stream);

/*
 * splr_linear_noalloc -- splr_linear without a workspace argument, for callers that cannot
 * allocate device memory (code under HIP graph capture, allocation-free serving loops, harnesses
 * that forbid hipMalloc).  The first-stage workspace lives in a device array inside the library,
 * SPLR_LINEAR_NOALLOC_MAX_WORKSPACE bytes on each GPU it runs on, held from the first call on that
 * GPU until the process ends.  The call allocates nothing (no hipMalloc / hipFree, no allocating
 * library routine); its first call on a GPU looks up that GPU's copy of the array.
 *
 *   Arguments and results: as splr_linear (same kernels, so Y is bit for bit splr_linear's).
 *   Limit: splr_linear_workspace_bytes(M, n_out, n_in, r, dtype) must not exceed
 *          SPLR_LINEAR_NOALLOC_MAX_WORKSPACE (e.g. 8192 tokens at rank 128 need 8 MiB).
 *   Sharing: every call on one GPU uses that GPU's single array, which keeps the last call's
 *          contents (nothing in it needs clearing: each call writes every byte it reads).  Calls
 *          that overlap in time on one GPU (different streams or host threads) race on it; order
 *          them on one stream or with events.
 * Errors: as splr_linear, minus SPLR_ERR_WORKSPACE; workspace need above the limit ->
 *         SPLR_ERR_SCRATCH (checked before any HIP call); a failed symbol lookup -> SPLR_ERR_HIP.
 */
#define SPLR_LINEAR_NOALLOC_MAX_WORKSPACE ((size_t)32 << 20)
splr_status_t splr_linear_noalloc(const void* X, int64_t M, int64_t n_in, const void* values,
                                  const uint32_t* meta, int64_t n_out, const void* U, const void* V,
                                  int64_t r, splr_dtype_t dtype, float* Y, hipStream_t stream);

/*
 * splr_dense_reconstruct -- W_hat = S + U V as a dense float32 matrix (LoSparse §3: the weight is
 * approximated by the sum of the sparse and the low-rank part).  A verification aid.
 *
 *   values, meta : packed S [n_out x n_in];  U [n_out][r], V [r][n_in] (NULL iff r == 0)
 *   W_hat [n_out][n_in] float32 output: stored entries widened exactly at their columns, +0
 *         elsewhere, plus the rank-r product accumulated in float32.
 * Errors: as splr_linear (no workspace).
 */
splr_status_t splr_dense_reconstruct(const void* values, const uint32_t* meta, const void* U,
                                     const void* V, int64_t n_out, int64_t n_in, int64_t r,
                                     splr_dtype_t dtype, float* W_hat, hipStream_t stream);

/*
 * Cholesky QR building blocks of the low-rank step of the data-free alternating minimisation
 * (HASSLE-free page, §4.2: the low-rank update is the rank-r truncated SVD of W - S, computed here
 * by subspace iteration on a k-column basis, k = r + oversampling). One orthonormalisation of a
 * float32 basis Y [n][k] is G = Y^T Y (splr_gram_f64), G = R^T R and Y R^-1 (splr_chol_rinv, then
 * a float32 matrix product); both stay on the device, so the loop synchronises with the host once
 * per step at most.
 *
 * splr_gram_workspace_bytes -- device workspace splr_gram_f64 needs for (n, k) (0 if out of range).
 *
 * splr_gram_f64 -- G = Y^T Y in float64 (every product of two float32 values is exact in float64;
 * rows are summed in a fixed order, so the result is deterministic).
 *   Y         [n][k] float32, row-major (device), 4-byte aligned
 *   G         [k][k] float64 output, both triangles written (device), 8-byte aligned
 *   workspace device memory of at least splr_gram_workspace_bytes(n, k) bytes, 8-byte aligned;
 *             its contents on entry do not matter
 * Errors: NULL Y or G -> SPLR_ERR_NULL; n < 1, n > 2^20, k < 1 or k > 192 -> SPLR_ERR_SHAPE;
 *         workspace NULL or too small -> SPLR_ERR_WORKSPACE; misaligned pointer -> SPLR_ERR_ALIGN.
 *
 * splr_chol_rinv -- R^-1 for the Cholesky factor of G = R^T R (R upper triangular, positive
 * diagonal), computed in float64 and written as float32.
 *   G    [k][k] float64 symmetric positive definite (device); only its lower triangle is read
 *   Rinv [k][k] float32 output (device): upper triangular, zeros below the diagonal
 * A G that is not numerically positive definite gives NaN entries (no error is reported).
 * Errors: NULL pointer -> SPLR_ERR_NULL; k < 1 or k > 192 -> SPLR_ERR_SHAPE; misaligned pointer
 *         (G 8 bytes, Rinv 4 bytes) -> SPLR_ERR_ALIGN.
 */
size_t splr_gram_workspace_bytes(int64_t n, int64_t k);
splr_status_t splr_gram_f64(const float* Y, int64_t n, int64_t k, double* G, void* workspace,
                            size_t workspace_bytes, hipStream_t stream);
splr_status_t splr_chol_rinv(const double* G, int64_t k, float* Rinv, hipStream_t stream);

/* Human-readable name of a status code (static storage; never NULL). */
const char* splr_status_string(splr_status_t status);

/* Library version as "major.minor.patch+<source hash>" (static storage): the first 16 hex digits of
   the SHA-256 of the sources the library was built from. */
const char* splr_version(void);

#ifdef __cplusplus
}
#endif

#endif /* SPLR_H_ */
