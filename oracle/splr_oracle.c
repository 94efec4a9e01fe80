/*
 * CPU oracle for the 2:4 sparse + rank-r linear layer.  TEST INFRASTRUCTURE ONLY.
 *
 * This file is the plain, slow, obviously-correct definition that the GPU library is checked
 * against.  Only the tests, the package's smoke check and the benchmark's CPU-baseline leg load
 * it; the GPU library never links, includes or calls it, and it includes nothing from the GPU
 * library.  Every sum is a sequential float64 loop in index order; OpenMP only splits independent
 * outputs between threads, so the result does not depend on the thread count.
 *
 * Layouts (contiguous):
 *   R, W_hat : [n_out][n_in] row-major
 *   X        : [M][n_in]   U : [n_out][r]   V : [r][n_in]   Y : [rows][n_out] (float64)
 *   packed S : tiles of 16 rows x 64 input columns, tile (tr, tk) at index tr * TK + tk with
 *              TR = ceil(n_out / 16), TK = ceil(n_in / 64). Row n, group g (columns 4g..4g+3)
 *              has tile (n / 16, g / 16); within the tile gi = g % 16, q = gi / 4, slot
 *              L = n % 16 + 16 q. Its two kept entries a < b (positions 0..3 in the group) are
 *              values[((tile * 64 + L) * 8) + 2 (gi % 4) + {0, 1}].
 *              Metadata comes in blocks of 8 consecutive tile columns of one tile row: block
 *              (tr, tb) at index tr * TKB + tb, TKB = ceil(TK / 8), 1 KiB = 256 uint32 words each.
 *              Within a block, slot L owns words 4 L .. 4 L + 3, i.e. eight 16-bit units, unit
 *              u = tk % 8 being the low (u even) or high (u odd) half of word 4 L + u / 2. Unit u
 *              of slot L holds the nibbles (a | b << 2) of groups 4 q .. 4 q + 3 of row n in tile
 *              (n / 16, 8 tb + u), group gi at bits 4 (gi % 4) of the unit.
 *              values holds TR * TK * 512 entries, meta TR * TKB * 256 uint32 words; entries and
 *              nibbles outside the matrix (row or column padding) are zero.
 * dtype 0 = float32 storage, 1 = bfloat16 storage (uint16 bit patterns).
 *
 * Functions and the passages they follow:
 *   splr_ref_prune24_pack     -- the sparse subproblem with identity Hessian is solved exactly by
 *                                hard thresholding (HASSLE-free page, §4.1.1); under the 2:4
 *                                constraint, at most two of every four consecutive weights may be
 *                                nonzero (3BASiL article, "A three-block ADMM replaces alternating
 *                                minimization").  Hard thresholding per group = keep the two
 *                                largest magnitudes unchanged, zero the rest.
 *   splr_ref_prune24_pack_scaled
 *                             -- the sparse subproblem with a diagonal Hessian: hard thresholding is
 *                                applied to the residual scaled column by column by D, which gives
 *                                Wanda's score |W_ij| * ||X_j|| (HASSLE-free page, §4.1.2); the kept
 *                                entries are the unscaled residual (scaling, thresholding, unscaling).
 *   splr_ref_residual, splr_ref_prune24_pack_residual
 *                             -- the sparse step of the alternating-minimisation / ADMM
 *                                decompositions acts on the weight minus the current low-rank part,
 *                                R = W - U V (HASSLE-free page, §4 and §4.1.1, the sparse subproblem
 *                                (P1)); the fused pack forms R entry by entry and projects it.
 *   splr_ref_prune_nm         -- N:M projection: in every group of M consecutive input columns keep
 *                                the N entries of largest magnitude and zero the rest, the same
 *                                hard thresholding under an N:M constraint (HASSLE-free page, §1 and
 *                                §2: the framework targets N:M sparsity; 3BASiL article, "A
 *                                three-block ADMM replaces alternating minimization": N:M structures
 *                                such as 2:4, and the 2:8 + rank-64 configuration after LoRA).
 *   splr_ref_linear           -- the compressed forward pass sums the sparse product and the
 *                                low-rank product, computed side by side (LoSparse page, §3 and
 *                                §3.2), here as Y = X S^T + (X V^T) U^T.
 *   splr_ref_dense_reconstruct-- the weight is approximated by the sum S + U V (LoSparse §3).
 *
 * Readings where the pages are silent (ties, special values, layout) are the ones listed at the
 * top of each function.
 */
#include <math.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>

#define SPLR_REF_FP32 0
#define SPLR_REF_BF16 1

#define SPLR_REF_OK 0
#define SPLR_REF_EINVAL 1
#define SPLR_REF_ENOMEM 2

static double load_f64(const void *base, int dtype, size_t i) {
  if (dtype == SPLR_REF_BF16) {
    uint32_t bits = (uint32_t)((const uint16_t *)base)[i] << 16;
    float f;
    memcpy(&f, &bits, 4);
    return (double)f;
  }
  return (double)((const float *)base)[i];
}

/* Unsigned magnitude key: the IEEE bit pattern with the sign cleared.  For finite values it orders
   by |x| exactly (subnormals included, +0 and -0 equal); infinities sort above every finite value
   and NaNs above infinities (by payload). */
static uint32_t magnitude_key(const void *base, int dtype, size_t i) {
  if (dtype == SPLR_REF_BF16) return (uint32_t)(((const uint16_t *)base)[i] & 0x7FFFu);
  return ((const uint32_t *)base)[i] & 0x7FFFFFFFu;
}

static void copy_elem(void *dst, size_t di, const void *src, size_t si, int dtype) {
  if (dtype == SPLR_REF_BF16)
    ((uint16_t *)dst)[di] = ((const uint16_t *)src)[si];
  else
    ((uint32_t *)dst)[di] = ((const uint32_t *)src)[si];
}

/* Activation-aware key of entry i (column k): |R| * |d_k| as a binary64 value.  Both factors have
   at most 24 significant bits and binary32 range, so the product is exact (no rounding, no
   overflow, no underflow) and keys order entries by the exact score.  NaN scores (a NaN entry or
   scale, or infinity times zero) are all equal and rank above every number.  Keys are compared as
   unsigned integers: for non-negative binary64 values that is the numeric order. */
static uint64_t scaled_key(const void *base, int dtype, size_t i, float dk) {
  const double p = fabs(load_f64(base, dtype, i)) * fabs((double)dk);
  if (p != p) return 0x7FF8000000000000ull;
  uint64_t u;
  memcpy(&u, &p, 8);
  return u;
}

/* Position i of a group outranks position j when its key is larger, or equal with i < j. */
static int outranks(const uint64_t key[4], int i, int j) {
  return key[i] > key[j] || (key[i] == key[j] && i < j);
}

/* ---- packed layout (see the header comment) ---- */
static int64_t tiles_rows(int64_t n_out) { return (n_out + 15) / 16; }
static int64_t tiles_cols(int64_t n_in) { return (n_in + 63) / 64; }

/* index of kept slot s (0 or 1) of group g in row n */
static size_t value_index(int64_t n, int64_t g, int s, int64_t n_in) {
  const int64_t gi = g % 16, q = gi / 4;
  const size_t tile = (size_t)(n / 16) * (size_t)tiles_cols(n_in) + (size_t)(g / 16);
  return (tile * 64 + (size_t)(n % 16 + 16 * q)) * 8 + (size_t)(2 * (gi % 4) + s);
}

static int64_t meta_blocks(int64_t n_in) { return (tiles_cols(n_in) + 7) / 8; }

/* metadata word holding the nibble of group g of row n, and the nibble's bit position in it */
static size_t meta_index(int64_t n, int64_t g, int64_t n_in, int *shift) {
  const int64_t tk = g / 16, gi = g % 16;
  const int64_t slot = n % 16 + 16 * (gi / 4), unit = tk % 8;
  const size_t block = (size_t)(n / 16) * (size_t)meta_blocks(n_in) + (size_t)(tk / 8);
  *shift = (int)(16 * (unit % 2) + 4 * (gi % 4));
  return block * 256 + (size_t)(4 * slot + unit / 2);
}

size_t splr_ref_packed_values(int64_t n_out, int64_t n_in) {
  return (size_t)tiles_rows(n_out) * (size_t)tiles_cols(n_in) * 512;
}

size_t splr_ref_packed_meta(int64_t n_out, int64_t n_in) {
  return (size_t)tiles_rows(n_out) * (size_t)meta_blocks(n_in) * 256;
}

/*
 * Shared selection of both packs: for every row and every group of four consecutive input columns,
 * keep the entry that outranks the other three and the entry that outranks the remaining two,
 * unchanged (bit copies); store them in ascending position order and record their positions.  The
 * key is the magnitude (d == NULL) or the activation-aware score (d = per-column scales).
 * Readings: ties go to the lower position; groups with fewer than two nonzeros still store two
 * slots (zeros included), so the output layout is fixed.
 */
static int pack_by_keys(const void *R, const float *d, int64_t n_out, int64_t n_in, int dtype, void *values,
                        uint32_t *meta) {
  if (!R || !values || !meta) return SPLR_REF_EINVAL;
  if (n_out < 0 || n_in < 0 || n_in % 32 != 0) return SPLR_REF_EINVAL;
  if (dtype != SPLR_REF_FP32 && dtype != SPLR_REF_BF16) return SPLR_REF_EINVAL;
  const int64_t groups = n_in / 4;
  const size_t nv = splr_ref_packed_values(n_out, n_in), nm = splr_ref_packed_meta(n_out, n_in);
  memset(values, 0, nv * (dtype == SPLR_REF_BF16 ? 2 : 4));
  memset(meta, 0, nm * sizeof(uint32_t));
#pragma omp parallel for schedule(static)
  for (int64_t n = 0; n < n_out; ++n) {
    for (int64_t g = 0; g < groups; ++g) {
      const size_t base = (size_t)n * (size_t)n_in + 4 * (size_t)g;
      uint64_t key[4];
      for (int i = 0; i < 4; ++i)
        key[i] = d ? scaled_key(R, dtype, base + i, d[4 * g + i]) : (uint64_t)magnitude_key(R, dtype, base + i);
      int first = 0;
      for (int i = 1; i < 4; ++i)
        if (outranks(key, i, first)) first = i;
      int second = -1;
      for (int i = 0; i < 4; ++i) {
        if (i == first) continue;
        if (second < 0 || outranks(key, i, second)) second = i;
      }
      const int a = first < second ? first : second;
      const int b = first < second ? second : first;
      copy_elem(values, value_index(n, g, 0, n_in), R, base + a, dtype);
      copy_elem(values, value_index(n, g, 1, n_in), R, base + b, dtype);
      int shift;
      const size_t w = meta_index(n, g, n_in, &shift);
      meta[w] |= (uint32_t)(a | (b << 2)) << shift;
    }
  }
  return SPLR_REF_OK;
}

/* 2:4 projection and pack (identity Hessian): keys are the magnitudes. */
int splr_ref_prune24_pack(const void *R, int64_t n_out, int64_t n_in, int dtype, void *values,
                          uint32_t *meta) {
  return pack_by_keys(R, NULL, n_out, n_in, dtype, values, meta);
}

/* Activation-aware 2:4 projection and pack (diagonal Hessian): keys are |R[n][k]| * |d[k]|; the
   stored entries are R's own.  d: float32 [n_in]. */
int splr_ref_prune24_pack_scaled(const void *R, const float *d, int64_t n_out, int64_t n_in, int dtype,
                                 void *values, uint32_t *meta) {
  if (!d) return SPLR_REF_EINVAL;
  return pack_by_keys(R, d, n_out, n_in, dtype, values, meta);
}

/*
 * N:M projection of R [n_out x n_in] into Rp (same storage type): in every group of m consecutive
 * columns of a row, entry i is kept (bit copy) when fewer than n entries of the group outrank it
 * (larger magnitude key, or an equal key at a lower position); every other entry becomes +0.
 * Readings: ties go to the lower position, as in the 2:4 projection; a dropped entry is stored as
 * +0 (the projection sets it to zero, and zero has no sign to keep).  Requires 1 <= n <= m and m | n_in.
 */
int splr_ref_prune_nm(const void *R, int64_t n_out, int64_t n_in, int n, int m, int dtype, void *Rp) {
  if (!R || !Rp) return SPLR_REF_EINVAL;
  if (n_out < 0 || n_in < 0 || m < 1 || n < 1 || n > m || n_in % m != 0) return SPLR_REF_EINVAL;
  if (dtype != SPLR_REF_FP32 && dtype != SPLR_REF_BF16) return SPLR_REF_EINVAL;
#pragma omp parallel for schedule(static)
  for (int64_t row = 0; row < n_out; ++row) {
    for (int64_t g0 = 0; g0 < n_in; g0 += m) {
      const size_t base = (size_t)row * (size_t)n_in + (size_t)g0;
      for (int i = 0; i < m; ++i) {
        const uint32_t ki = magnitude_key(R, dtype, base + i);
        int above = 0;
        for (int j = 0; j < m; ++j) {
          const uint32_t kj = magnitude_key(R, dtype, base + j);
          if (kj > ki || (kj == ki && j < i)) ++above;
        }
        if (above < n)
          copy_elem(Rp, base + i, R, base + i, dtype);
        else if (dtype == SPLR_REF_BF16)
          ((uint16_t *)Rp)[base + i] = 0;
        else
          ((uint32_t *)Rp)[base + i] = 0;
      }
    }
  }
  return SPLR_REF_OK;
}

/* binary32 (not NaN) -> bfloat16 bits, round to nearest even. */
static uint16_t to_bf16_rne(float f) {
  uint32_t u;
  memcpy(&u, &f, 4);
  return (uint16_t)((u + 0x7FFFu + ((u >> 16) & 1u)) >> 16);
}

static float load_f32(const void *base, int dtype, size_t i) { return (float)load_f64(base, dtype, i); }

/*
 * Residual with the pinned arithmetic of the fused pack.  For every entry: acc = W[n][k] (binary32),
 * then for j = 0, 1, ..., r-1 in that order acc = fmaf(-U[n][j], V[j][k], acc) -- one rounding per
 * step -- and R[n][k] = acc stored in the storage type (bfloat16: round to nearest even).  A NaN
 * result is stored as the canonical quiet NaN (binary32 0x7FC00000, bfloat16 0x7FC0): processors
 * differ in the sign and payload of the NaNs they produce.  Reading: the pages define R = W - U V
 * but fix no arithmetic; this order is the plainest one a bit-exact kernel can follow.
 */
int splr_ref_residual(const void *W, const void *U, const void *V, int64_t n_out, int64_t n_in, int64_t r, int dtype,
                      void *R) {
  if (!W || !R || (r > 0 && (!U || !V))) return SPLR_REF_EINVAL;
  if (n_out < 0 || n_in < 0 || r < 0) return SPLR_REF_EINVAL;
  if (dtype != SPLR_REF_FP32 && dtype != SPLR_REF_BF16) return SPLR_REF_EINVAL;
#pragma omp parallel for schedule(static)
  for (int64_t n = 0; n < n_out; ++n) {
    for (int64_t k = 0; k < n_in; ++k) {
      float acc = load_f32(W, dtype, (size_t)n * (size_t)n_in + (size_t)k);
      for (int64_t j = 0; j < r; ++j)
        acc = fmaf(-load_f32(U, dtype, (size_t)n * (size_t)r + (size_t)j),
                   load_f32(V, dtype, (size_t)j * (size_t)n_in + (size_t)k), acc);
      const size_t i = (size_t)n * (size_t)n_in + (size_t)k;
      if (acc != acc) {
        if (dtype == SPLR_REF_BF16)
          ((uint16_t *)R)[i] = 0x7FC0u;
        else
          ((uint32_t *)R)[i] = 0x7FC00000u;
      } else if (dtype == SPLR_REF_BF16) {
        ((uint16_t *)R)[i] = to_bf16_rne(acc);
      } else {
        ((float *)R)[i] = acc;
      }
    }
  }
  return SPLR_REF_OK;
}

/* Fused residual + 2:4 projection + pack: the plain pack of splr_ref_residual's R. */
int splr_ref_prune24_pack_residual(const void *W, const void *U, const void *V, int64_t n_out, int64_t n_in, int64_t r,
                                   int dtype, void *values, uint32_t *meta) {
  if (n_out < 0 || n_in < 0) return SPLR_REF_EINVAL;
  const size_t esz = dtype == SPLR_REF_BF16 ? 2 : 4;
  void *R = malloc((size_t)n_out * (size_t)n_in * esz + 1);
  if (!R) return SPLR_REF_ENOMEM;
  int rc = splr_ref_residual(W, U, V, n_out, n_in, r, dtype, R);
  if (rc == SPLR_REF_OK) rc = splr_ref_prune24_pack(R, n_out, n_in, dtype, values, meta);
  free(R);
  return rc;
}

static void decode_nibble(const uint32_t *meta, int64_t n, int64_t g, int64_t n_in, int *a, int *b) {
  int shift;
  const size_t w = meta_index(n, g, n_in, &shift);
  const uint32_t nib = (meta[w] >> shift) & 0xFu;
  *a = (int)(nib & 3u);
  *b = (int)(nib >> 2);
}

/*
 * The logical view of a packed matrix: kept[n][2g + s] (storage dtype) and the nibble of every
 * group, nib[n][g].  Layout bookkeeping only; it takes no decision.
 */
int splr_ref_unpack(const void *values, const uint32_t *meta, int64_t n_out, int64_t n_in, int dtype,
                    void *kept, uint8_t *nib) {
  if (!values || !meta || !kept || !nib) return SPLR_REF_EINVAL;
  if (n_out < 0 || n_in < 0 || n_in % 32 != 0) return SPLR_REF_EINVAL;
  if (dtype != SPLR_REF_FP32 && dtype != SPLR_REF_BF16) return SPLR_REF_EINVAL;
  const int64_t groups = n_in / 4;
  for (int64_t n = 0; n < n_out; ++n)
    for (int64_t g = 0; g < groups; ++g) {
      for (int s = 0; s < 2; ++s)
        copy_elem(kept, (size_t)n * (size_t)(n_in / 2) + 2 * (size_t)g + s, values, value_index(n, g, s, n_in), dtype);
      int shift;
      const size_t w = meta_index(n, g, n_in, &shift);
      nib[(size_t)n * (size_t)groups + g] = (uint8_t)((meta[w] >> shift) & 0xFu);
    }
  return SPLR_REF_OK;
}

/*
 * Y[i][n] = sum_g ( X[m][4g+a] * S_a(n, g) + X[m][4g+b] * S_b(n, g) )
 *         + sum_j T[i][j] * U[n][j],      T[i][j] = sum_k X[m][k] * V[j][k],
 * for m = rows[i] (every m in 0..M-1 in order when rows is NULL), all in float64.
 * U and V may be NULL when r == 0.
 */
int splr_ref_linear(const void *X, int64_t M, int64_t n_in, const void *values,
                    const uint32_t *meta, int64_t n_out, const void *U, const void *V, int64_t r,
                    int dtype, const int64_t *rows, int64_t n_rows, double *Y) {
  if (!X || !values || !meta || !Y) return SPLR_REF_EINVAL;
  if (r > 0 && (!U || !V)) return SPLR_REF_EINVAL;
  if (M < 0 || n_in < 0 || n_in % 32 != 0 || n_out < 0 || r < 0) return SPLR_REF_EINVAL;
  if (dtype != SPLR_REF_FP32 && dtype != SPLR_REF_BF16) return SPLR_REF_EINVAL;
  if (!rows) n_rows = M;
  for (int64_t i = 0; i < (rows ? n_rows : 0); ++i)
    if (rows[i] < 0 || rows[i] >= M) return SPLR_REF_EINVAL;
  const int64_t groups = n_in / 4;

  double *xrows = (double *)malloc(sizeof(double) * (size_t)(n_rows > 0 ? n_rows : 1) * (size_t)(n_in > 0 ? n_in : 1));
  double *T = (double *)malloc(sizeof(double) * (size_t)(n_rows > 0 ? n_rows : 1) * (size_t)(r > 0 ? r : 1));
  if (!xrows || !T) {
    free(xrows);
    free(T);
    return SPLR_REF_ENOMEM;
  }
#pragma omp parallel for schedule(static)
  for (int64_t i = 0; i < n_rows; ++i) {
    const int64_t m = rows ? rows[i] : i;
    for (int64_t k = 0; k < n_in; ++k) xrows[i * n_in + k] = load_f64(X, dtype, (size_t)m * (size_t)n_in + k);
  }
  /* first low-rank stage: T = X V^T */
#pragma omp parallel for collapse(2) schedule(static)
  for (int64_t i = 0; i < n_rows; ++i)
    for (int64_t j = 0; j < r; ++j) {
      double t = 0.0;
      for (int64_t k = 0; k < n_in; ++k) t += xrows[i * n_in + k] * load_f64(V, dtype, (size_t)j * (size_t)n_in + k);
      T[i * r + j] = t;
    }
  /* sparse product plus second low-rank stage */
#pragma omp parallel for collapse(2) schedule(static)
  for (int64_t i = 0; i < n_rows; ++i)
    for (int64_t n = 0; n < n_out; ++n) {
      const double *x = xrows + i * n_in;
      double sparse = 0.0;
      for (int64_t g = 0; g < groups; ++g) {
        int a, b;
        decode_nibble(meta, n, g, n_in, &a, &b);
        sparse += x[4 * g + a] * load_f64(values, dtype, value_index(n, g, 0, n_in));
        sparse += x[4 * g + b] * load_f64(values, dtype, value_index(n, g, 1, n_in));
      }
      double lowrank = 0.0;
      for (int64_t j = 0; j < r; ++j) lowrank += T[i * r + j] * load_f64(U, dtype, (size_t)n * (size_t)r + j);
      Y[i * n_out + n] = sparse + lowrank;
    }
  free(xrows);
  free(T);
  return SPLR_REF_OK;
}

/*
 * W_hat[n][k] = S[n][k] + sum_j U[n][j] * V[j][k] in float64, where S is the dense matrix
 * scattered from (values, meta): the two stored entries at their positions, +0 elsewhere.
 * Without a low-rank part (r = 0) W_hat is S itself, entry for entry: a stored -0 stays -0 (adding
 * an empty sum, +0, would turn it into +0).  With r > 0 the rank-r sum is added to every entry.
 */
int splr_ref_dense_reconstruct(const void *values, const uint32_t *meta, const void *U,
                               const void *V, int64_t n_out, int64_t n_in, int64_t r, int dtype,
                               double *W_hat) {
  if (!values || !meta || !W_hat) return SPLR_REF_EINVAL;
  if (r > 0 && (!U || !V)) return SPLR_REF_EINVAL;
  if (n_out < 0 || n_in < 0 || n_in % 32 != 0 || r < 0) return SPLR_REF_EINVAL;
  if (dtype != SPLR_REF_FP32 && dtype != SPLR_REF_BF16) return SPLR_REF_EINVAL;
  const int64_t groups = n_in / 4;
#pragma omp parallel for schedule(static)
  for (int64_t n = 0; n < n_out; ++n) {
    double *w = W_hat + n * n_in;
    for (int64_t k = 0; k < n_in; ++k) w[k] = 0.0;
    for (int64_t g = 0; g < groups; ++g) {
      int a, b;
      decode_nibble(meta, n, g, n_in, &a, &b);
      w[4 * g + a] = load_f64(values, dtype, value_index(n, g, 0, n_in));
      w[4 * g + b] = load_f64(values, dtype, value_index(n, g, 1, n_in));
    }
    if (r == 0) continue;
    for (int64_t k = 0; k < n_in; ++k) {
      double lowrank = 0.0;
      for (int64_t j = 0; j < r; ++j)
        lowrank += load_f64(U, dtype, (size_t)n * (size_t)r + j) * load_f64(V, dtype, (size_t)j * (size_t)n_in + k);
      w[k] += lowrank;
    }
  }
  return SPLR_REF_OK;
}
