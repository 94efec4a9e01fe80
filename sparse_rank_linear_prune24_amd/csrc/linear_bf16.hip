// Y = X S^T + (X V^T) U^T for bfloat16 operands, float32 accumulation and output (LoSparse page,
// §3.2: the sparse product and the low-rank product are evaluated side by side and summed).
//
// The sparse product runs on gfx950's structured-sparse MFMA, v_smfmac_f32_16x16x64_bf16, as
// Y^T tiles = S_tile * X_tile^T: S is the sparse A operand, X^T the dense B operand. Lane layouts:
//   A (S):  lane l -> row l%16, dense columns 16*(l/16) .. +15 (kept values 8*(l/16) .. +7), index
//           operand = the 4 nibbles of those groups in bits [15:0]
//   B (X):  lane l -> token l%16, columns 8*(l/16)+0..7 and 32+8*(l/16)+0..7
//   D:      lane l -> rows (n) 4*(l/16)+0..3, token l%16
// The packed layout stores each 16-row x 64-column tile in exactly this A order, so a wave reads
// its S fragment as 1 KiB of contiguous memory and its metadata as 128 contiguous bytes. X is
// row-major: it is loaded with row-contiguous (coalesced) 16-byte loads and staged in LDS with a
// padded 160-byte row pitch, from which the B fragments are read without bank conflicts.
//
// The rank-r term is folded into the same accumulators with the same instruction (its first 128
// ranks before the main loop, so that they overlap the loop's first loads; further blocks of 64
// after it): dense U is the sum of two 2:4 matrices with fixed patterns (positions 0,1 and 2,3 of
// every group of four ranks), so acc += U_tile T_tile^T is two structured-sparse MFMAs per 64
// ranks with constant index operands. T (float32) enters as a bfloat16 high part plus a bfloat16
// correction. Y is stored once.
//
// One kernel template for M > 64 tokens (fewer tokens take the decode kernel in decode.hip): a
// workgroup tile of 512 rows x 128 tokens, or 256 rows when 512-row tiles would leave CUs idle;
// eight waves, two per SIMD, each owning 16 NI rows and all 128 tokens with its accumulators in
// the matrix-core accumulator registers, so every S fragment is used by one wave and goes global
// -> registers (raw buffer loads); X is shared through a five-slot LDS ring; workgroups are
// remapped so the tiles that one XCD (own L2) runs share X and S. Its DENSE form expands S to
// dense bfloat16 in registers and runs dense MFMAs instead (the measured alternative).
#include "common.hpp"
#include "kernels.hpp"
#include "tile_common.hpp"

namespace splr {
namespace {
// ----------------------------------------------------------------------------------- prefill

// EPI: how Y is stored -- bit 0: through LDS as whole token rows (else in fragment order), bit 1:
// non-temporal stores
constexpr int kEpiDirect = 0, kEpiRows = 1, kEpiDirectNT = 2, kEpiRowsNT = 3;

// Stores a wave's accumulators acc[i][j] (rows nrow0 + 16 i + 4 (lane / 16) + 0..3, tokens
// m0 + 16 j + lane % 16) through `buf`, a private LDS region of the wave (32 tokens x (16 NI + 4)
// floats), 32 tokens at a time: each global store instruction then writes whole token rows of the
// wave's 16 NI outputs (64 NI contiguous bytes per token), i.e. whole cache lines, where the fragment
// order writes 16-byte pieces of 16 token rows. float32, or (y_bf16) rounded to bfloat16 (to
// nearest even); NT: non-temporal stores. The wave reads only what it wrote, in order, so no barrier
// is needed between the phases.
template <int NI, int NJ, bool NT>
__device__ __forceinline__ void store_tile_rows_lds(const f32x4_t (&acc)[NI][NJ], float* buf, void* __restrict__ Yv,
                                                    int y_bf16, int M, int n_out, int nrow0, int m0, int lane) {
  constexpr int R = 16 * NI, kPitch = R + 4, kTok = 32;
  constexpr int kLanesPerTok = R / 4, kTokPerRead = 64 / kLanesPerTok;
  static_assert(NJ % 2 == 0 && kTok % kTokPerRead == 0, "32 tokens a round");
  const int q = lane >> 4, sb = lane & 15;
  const int rl = lane % kLanesPerTok, tl = lane / kLanesPerTok;
  const int n = nrow0 + 4 * rl;
  const bool vec_ok = (n_out & 3) == 0 && n + 3 < n_out;
#pragma unroll
  for (int c = 0; c < NJ / 2; ++c) {
#pragma unroll
    for (int jj = 0; jj < 2; ++jj)
#pragma unroll
      for (int i = 0; i < NI; ++i) *(f32x4_t*)(buf + (16 * jj + sb) * kPitch + 16 * i + 4 * q) = acc[i][2 * c + jj];
#pragma unroll
    for (int k = 0; k < kTok / kTokPerRead; ++k) {
      const int t = k * kTokPerRead + tl;
      const f32x4_t v = *(const f32x4_t*)(buf + t * kPitch + 4 * rl);
      const int m = m0 + 32 * c + t;
      if (m >= M) continue;
      if (y_bf16) {
        uint16_t* yrow = (uint16_t*)Yv + (size_t)m * n_out;
        uint32_t h[4];
#pragma unroll
        for (int e = 0; e < 4; ++e) h[e] = float_to_bf16_bits(v[e]);
        if (vec_ok) {
          const u32x2_t w = u32x2_t{h[0] | (h[1] << 16), h[2] | (h[3] << 16)};
          if constexpr (NT) __builtin_nontemporal_store(w, (u32x2_t*)(yrow + n));
          else *(u32x2_t*)(yrow + n) = w;
        } else {
#pragma unroll
          for (int e = 0; e < 4; ++e)
            if (n + e < n_out) yrow[n + e] = (uint16_t)h[e];
        }
      } else {
        float* yrow = (float*)Yv + (size_t)m * n_out;
        if (vec_ok) {
          if constexpr (NT) __builtin_nontemporal_store(v, (f32x4_t*)(yrow + n));
          else *(f32x4_t*)(yrow + n) = v;
        } else {
#pragma unroll
          for (int e = 0; e < 4; ++e)
            if (n + e < n_out) yrow[n + e] = v[e];
        }
      }
    }
  }
}

// Word 3 of a raw buffer descriptor on gfx9-family GPUs: 32-bit data format, no swizzle, no index
// stride (plain byte-addressed loads).
constexpr int kBufferFlags = 0x00020000;

// The structured-sparse MFMA with its accumulator pinned to the matrix-core accumulator registers
// (the compiler would otherwise spread the accumulators over both register files and copy them
// every step). ABID selects the half of the 32-bit index register the instruction reads (a
// metadata word holds the indices of two tile columns). Hazard rules this relies on, kept by the
// kernel below: the A, B and index operands come straight from loads (the waits for loads precede
// the instruction; a vector-ALU write of an operand is followed by operand_fence), an accumulator
// is written by these instructions only (accumulating into the same registers with the same
// instruction needs no wait states, as the compiler's own back-to-back chains show) and anything
// else touches the accumulators only across accumulator_fence().
template <int ABID>
__device__ __forceinline__ void smfmac_acc(f32x4_t& acc, bf16x8_t a, bf16x16_t b, uint32_t idx) {
  if constexpr (ABID == 0)
    asm volatile("v_smfmac_f32_16x16x64_bf16 %0, %1, %2, %3" : "+a"(acc) : "v"(a), "v"(b), "v"(idx));
  else
    asm volatile("v_smfmac_f32_16x16x64_bf16 %0, %1, %2, %3 abid:1" : "+a"(acc) : "v"(a), "v"(b), "v"(idx));
}
// Y[16 x 16] += A[16 x 32] . B[32 x 16], dense bfloat16 MFMA on an accumulator-register fragment
// (the decompress-then-dense variant of the sparse product). Same output layout as smfmac_acc.
__device__ __forceinline__ void mfma_dense_acc(f32x4_t& acc, bf16x8_t a, bf16x8_t b) {
  asm volatile("v_mfma_f32_16x16x32_bf16 %0, %1, %2, %0" : "+a"(acc) : "v"(a), "v"(b));
}

// Decompression of a lane's packed operand: the dense bfloat16 values of two consecutive groups of
// four columns, from their kept pairs k0, k1 (the first kept value in the low half) and their
// nibbles in bits 0-3 and 4-7 of nib (a | b << 2 with a < b the kept positions; nibble 0 only in
// padding, whose kept values are zero). Returns the eight columns as four words of two bfloat16.
__device__ __forceinline__ u32x4_t expand_groups(uint32_t k0, uint32_t k1, uint32_t nib) {
  auto group = [](uint32_t k, uint32_t n) -> uint64_t {
    const uint32_t a = (n & 3u) * 16u, b = ((n >> 2) & 3u) * 16u;
    return ((uint64_t)(k & 0xFFFFu) << a) | ((uint64_t)(k >> 16) << b);
  };
  const uint64_t g0 = group(k0, nib & 15u), g1 = group(k1, (nib >> 4) & 15u);
  return u32x4_t{(uint32_t)g0, (uint32_t)(g0 >> 32), (uint32_t)g1, (uint32_t)(g1 >> 32)};
}

// Wait states between accumulator writes by ordinary instructions and smfmac_acc (or the reverse),
// followed by an empty asm per accumulator that every later use depends on, so the compiler cannot
// move an accumulator read or write across the wait states (64 > the pass count of the 16x16x64
// structured-sparse MFMA and every write-to-read distance the matrix core needs).
template <int NI, int NJ>
__device__ __forceinline__ void accumulator_fence(f32x4_t (&acc)[NI][NJ]) {
  asm volatile("s_nop 15\n\ts_nop 15\n\ts_nop 15\n\ts_nop 15" ::: "memory");
#pragma unroll
  for (int i = 0; i < NI; ++i)
#pragma unroll
    for (int j = 0; j < NJ; ++j) asm volatile("" : "+a"(acc[i][j]));
}

// Operand fences: the registers passed through one were last written before it (vector-ALU
// instructions included), and 8 wait states pass before any later instruction touches them. Placed
// between a vector-ALU write and the first matrix-core read of a register, and after the last
// matrix-core read of an index register before anything may overwrite it.
template <typename A, typename B>
__device__ __forceinline__ void operand_fence(A& a, B& b) {
  asm volatile("s_nop 7" : "+v"(a), "+v"(b));
}
template <typename A, typename B, typename C, typename D>
__device__ __forceinline__ void operand_fence(A& a, B& b, C& c, D& d) {
  asm volatile("s_nop 7" : "+v"(a), "+v"(b), "+v"(c), "+v"(d));
}

// U's fragment rows for one 64-rank block of the rank-r term: row nrow0 + 16 i + lane % 16, ranks
// j0 + 16 (lane / 16) .. +15 (zeros past n_out or r), as loaded; split() gives the (0,1) and (2,3)
// halves of every group of four ranks, the A operands of the two structured-sparse MFMAs that
// together make one dense product.
template <int NI>
struct UFragments {
  u32x4_t d[NI][2];
  __device__ __forceinline__ void load(const uint16_t* __restrict__ U, int n_out, int r, int j0, int nrow0, int lane) {
    const int ju = j0 + 16 * (lane >> 4);
    const u32x4_t zero = {0, 0, 0, 0};
#pragma unroll
    for (int i = 0; i < NI; ++i) {
      const int n = nrow0 + 16 * i + (lane & 15);
      const bool ok = n < n_out && ju < r;
      const uint16_t* p = U + (size_t)(ok ? n : 0) * r + (ok ? ju : 0);
      d[i][0] = ok ? *(const u32x4_t*)p : zero;
      d[i][1] = ok ? *(const u32x4_t*)(p + 8) : zero;
    }
  }
  __device__ __forceinline__ bf16x8_t pair01(int i) const {
    return as_bf16x8(u32x4_t{d[i][0][0], d[i][0][2], d[i][1][0], d[i][1][2]});
  }
  __device__ __forceinline__ bf16x8_t pair23(int i) const {
    return as_bf16x8(u32x4_t{d[i][0][1], d[i][0][3], d[i][1][1], d[i][1][3]});
  }
};

// acc[i][j] (rows nrow0 + 16 i + ..., tokens 16 j + ...) += U[n][j0 .. j0+63] . T[token][j0 .. j0+63]
// with the accumulators in the accumulator registers (smfmac_acc): the rank-r term of
// lowrank_block, for the kernels that keep their accumulators there. U comes as loaded fragments,
// T's bfloat16 pair from the LDS planes hi / lo one token fragment at a time, the next fragment's
// read in flight during the current one's MFMAs. The MFMAs of a token fragment run over the row
// fragments innermost, so consecutive MFMAs write different accumulators.
template <int NI, int NJ>
__device__ __forceinline__ void lowrank_block_acc(f32x4_t (&acc)[NI][NJ], const UFragments<NI>& uf,
                                                  const u32x4_t* hi, const u32x4_t* lo) {
  static_assert(NI % 2 == 0, "U fragments fenced two rows at a time");
  // the lane index recomputed here (two instructions) rather than kept from the kernel's start: a
  // kept value may be spilled, and its reload would wait for every load in flight
  const int lane = (int)__builtin_amdgcn_mbcnt_hi(~0u, __builtin_amdgcn_mbcnt_lo(~0u, 0u));
  const int sub = lane & 15, quad = lane >> 4;
  bf16x8_t u01[NI], u23[NI];
#pragma unroll
  for (int i = 0; i < NI; ++i) {
    u01[i] = uf.pair01(i);
    u23[i] = uf.pair23(i);
  }
#pragma unroll
  for (int i = 0; i < NI; i += 2) operand_fence(u01[i], u23[i], u01[i + 1], u23[i + 1]);
  uint32_t i01 = 0x4444u, i23 = 0xEEEEu;
  operand_fence(i01, i23);
  // T's pair of token fragment j + 1 is read from LDS while the MFMAs of fragment j run
  bf16x16_t th[2], tl[2];
  auto read_t = [&](int j, int b) {
    const int row = (16 * j + sub) * kXPitchU4;
    th[b] = cat16(as_bf16x8(hi[row + quad]), as_bf16x8(hi[row + 4 + quad]));
    tl[b] = cat16(as_bf16x8(lo[row + quad]), as_bf16x8(lo[row + 4 + quad]));
  };
  read_t(0, 0);
#pragma unroll
  for (int j = 0; j < NJ; ++j) {
    if (j + 1 < NJ) read_t(j + 1, (j + 1) & 1);
    operand_fence(th[j & 1], tl[j & 1]);
#pragma unroll
    for (int i = 0; i < NI; ++i) smfmac_acc<0>(acc[i][j], u01[i], th[j & 1], i01);
#pragma unroll
    for (int i = 0; i < NI; ++i) smfmac_acc<0>(acc[i][j], u23[i], th[j & 1], i23);
#pragma unroll
    for (int i = 0; i < NI; ++i) smfmac_acc<0>(acc[i][j], u01[i], tl[j & 1], i01);
#pragma unroll
    for (int i = 0; i < NI; ++i) smfmac_acc<0>(acc[i][j], u23[i], tl[j & 1], i23);
  }
  operand_fence(i01, i23);  // the index registers outlive the last MFMA that reads them
}

// Operands of up to kMaxGroup layers of one shape whose tiles share one grid (passed by value;
// a single-layer launch is a group of one). A workgroup's layer follows from its tile index, so it
// is uniform across the workgroup and is selected with scalar compares (no dynamic indexing, which
// could move the table to private memory).
struct LayerGroup {
  const uint16_t* X[kMaxGroup];
  const u32x4_t* values[kMaxGroup];
  const uint32_t* meta[kMaxGroup];
  const uint16_t* U[kMaxGroup];
  const float* Tpart[kMaxGroup];
  void* Y[kMaxGroup];
};
template <typename T>
__device__ __forceinline__ T pick_layer(const T (&a)[kMaxGroup], int layer) {
  static_assert(kMaxGroup == 4, "one compare per layer");
  return layer == 0 ? a[0] : layer == 1 ? a[1] : layer == 2 ? a[2] : a[3];
}

// Prefill kernel with the accumulators in the matrix-core accumulator registers: workgroup tile
// 16*NI*WAVES rows x 128 tokens, each wave owning 16*NI rows (NI S fragments) x all 128 tokens, so
// NI*8 accumulator fragments = 32*NI accumulator registers per lane. As launched, WAVES = 8 (two
// waves per SIMD, so one wave's loads, LDS traffic and barrier waits overlap the other's MFMAs) with
// NI = 4 (512 rows; 128 accumulator + 128 arch registers per wave) or NI = 2 (256 rows); WAVES = 4
// is one wave per SIMD. Per 64-column K step a CU loads 1 KiB of S values per 16 rows and 16 KiB of
// X, and each lane loads its metadata once per 8 steps: one 16-byte word group per fragment holds
// its indices for a whole metadata block. Each 16-token group's B fragment is read from LDS LA
// groups ahead of its NI MFMAs; X goes through a five-slot LDS ring with a barrier every second
// step. The first two 64-rank blocks of the rank-r term run before the main loop (their T pairs in
// four of the ring's slots); further blocks after it.
template <int NI, int LA, int P, int EPI, int WAVES = 8, bool DENSE = false>
__global__ __launch_bounds__(64 * WAVES) __attribute__((amdgpu_waves_per_eu(WAVES / 4, WAVES / 4))) void
linear_prefill_wide_kernel(const LayerGroup lg, int layers, int slices, int y_bf16, int M, int K, int n_out, int r,
                           int tiles_n, int tiles_m, int tiles_per_xcd, int group_m) {
  constexpr int NJ = 8, PX = 2;
  static_assert(WAVES == 4 || WAVES == 8, "one or two waves per SIMD");
  constexpr int BN = 16 * NI * WAVES;  // 512 or 256 rows
  constexpr int BM = 16 * NJ;          // 128 tokens
  static_assert(NI % 2 == 0 && LA >= 1 && LA < NJ, "S loads in groups of up to four fragments");
  constexpr int kXLoads = BM / (8 * WAVES);
  static_assert(P >= 2 && 16 % P == 0, "S prefetch distance dividing the unroll");
  constexpr int kUnroll = 16;  // two metadata blocks: every S, X-register and metadata ring index is constant
  constexpr int kSlot = BM * kXPitchU4;  // one LDS slot, 16-byte units
  constexpr int kPreBlocks = 2;          // 64-rank blocks of the rank-r term run before the main loop
  // X ring: kSlots slots, X of step kc written during step kc - kLead, one barrier every kBarEvery
  // steps. A slot is rewritten kSlots - kLead steps after its last step, and data is first read
  // (by the B-fragment lookahead) kLead - 1 steps after it was written: both gaps hold a barrier
  // when they span kBarEvery steps.
  constexpr int kSlots = 5, kLead = 3, kBarEvery = 2;
  static_assert(kSlots - kLead >= kBarEvery && kLead - 1 >= kBarEvery && 16 % kBarEvery == 0, "ring");
  static_assert(2 * kPreBlocks <= kSlots, "T planes alias the ring");
  __shared__ u32x4_t xs[kSlots * kSlot];
  u32x4_t* const tp = xs;  // T's bfloat16 pair (hi, lo) of those blocks, before the ring is used

  // XCD-aware tile order: each XCD (own L2) runs a contiguous range of the tiles, layer after layer
  const int b = blockIdx.x;
  const int logical_all = (b & 7) * tiles_per_xcd + (b >> 3);
  const int per_layer = tiles_n * tiles_m;
  if (logical_all >= per_layer * layers) return;
  const int layer = logical_all / per_layer;
  const int logical = logical_all - layer * per_layer;
  const uint16_t* __restrict__ X = pick_layer(lg.X, layer);
  const u32x4_t* __restrict__ values = pick_layer(lg.values, layer);
  const uint32_t* __restrict__ meta = pick_layer(lg.meta, layer);
  const uint16_t* __restrict__ U = pick_layer(lg.U, layer);
  const float* __restrict__ Tpart = pick_layer(lg.Tpart, layer);
  void* __restrict__ Y = pick_layer(lg.Y, layer);
  const int per_group = group_m * tiles_n;
  const int g = logical / per_group;
  const int first_m = g * group_m;
  const int gsize = min(group_m, tiles_m - first_m);
  const int in_group = logical - g * per_group;
  const int m0 = (first_m + in_group % gsize) * BM;
  const int n0 = (in_group / gsize) * BN;

  const int lane = threadIdx.x & 63, wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int sub = lane & 15, quad = lane >> 4;
  const int TK = (K + 63) / 64, TR = (n_out + 15) / 16, TKB = meta_blocks(TK);
  const int nk_pad = (TK + kUnroll - 1) / kUnroll * kUnroll;

  // Loads are raw buffer loads: a wave-uniform base (buffer descriptor) plus a wave-uniform byte
  // offset (scalar register) plus one 32-bit per-lane offset, so no per-load address arithmetic
  // runs on the vector ALUs and the per-lane state is a few registers. Each descriptor covers only
  // the bytes this wave may touch; loads past it return zero (padding steps and fragments past the
  // last tile row use that).
  // S fragment i of step kk: tile row tr0 + i, 1 KiB per tile, the lane's 16 bytes; metadata block
  // kb of tile row tr0 + i: 1 KiB, the lane's 16 bytes (its slot is its lane).
  const int tr0 = __builtin_amdgcn_readfirstlane(min(n0 / 16 + wave * NI, TR - 1));
  const int rows_here = min(NI, TR - tr0);
  const __amdgpu_buffer_rsrc_t vrs = __builtin_amdgcn_make_buffer_rsrc(
      (void*)(values + (size_t)tr0 * TK * 64), (short)0, rows_here * TK * 1024, kBufferFlags);
  const __amdgpu_buffer_rsrc_t mrs = __builtin_amdgcn_make_buffer_rsrc(
      (void*)((const char*)meta + (size_t)tr0 * TKB * 1024), (short)0, rows_here * TKB * 1024, kBufferFlags);
  const int s_off = lane * 16;
  const int s_stride = TK * 1024, m_stride = TKB * 1024;  // bytes per tile row
  // X: rows m0 + wave*32 + 8t + lane/8 (clamped to M-1), 16-byte chunk lane%8 of a step; offsets
  // from the tile's first row stay below 2^31 (at most 128 rows of at most 2^20 columns)
  const int xchunk = lane & 7;
  const int x_rows = min(BM, M - m0);
  const __amdgpu_buffer_rsrc_t xrs =
      __builtin_amdgcn_make_buffer_rsrc((void*)(X + (size_t)m0 * K), (short)0, x_rows * K * 2, kBufferFlags);
  int x_off[kXLoads];
  int xdst[kXLoads];
#pragma unroll
  for (int t = 0; t < kXLoads; ++t) {
    const int tloc = wave * (BM / WAVES) + 8 * t + (lane >> 3);
    x_off[t] = min(tloc, x_rows - 1) * K * 2 + 16 * xchunk;
    xdst[t] = tloc * kXPitchU4 + xchunk;
  }

  u32x4_t xr[PX][kXLoads];
  u32x4_t sa[P][NI];
  u32x4_t mb[2][NI];  // metadata of the current and the next block of 8 steps
  bf16x16_t bx[LA + 1];
  bf16x8_t bh[LA + 1];  // DENSE: B half fragments (32 columns), LA groups ahead
  const int x_end = x_rows * K * 2, v_end = rows_here * s_stride, m_end = rows_here * m_stride;
  auto load_x = [&](int kc, u32x4_t (&v)[kXLoads]) {
    // half tail step: re-read valid columns (S is zero there); per lane, as the chunk decides
    const int back = (kc < TK && kc * 64 + 8 * xchunk >= K) ? 64 : 0;
    const int so = kc < TK ? kc * 128 : x_end;
#pragma unroll
    for (int t = 0; t < kXLoads; ++t) v[t] = __builtin_amdgcn_raw_buffer_load_b128(xrs, x_off[t] - back, so, 0);
  };
  auto load_s_frag = [&](int kc, int i, u32x4_t& va) {
    va = __builtin_amdgcn_raw_buffer_load_b128(vrs, s_off, kc < TK ? i * s_stride + kc * 1024 : v_end, 0);
  };
  auto load_m = [&](int kb, u32x4_t (&m)[NI]) {
#pragma unroll
    for (int i = 0; i < NI; ++i)
      m[i] = __builtin_amdgcn_raw_buffer_load_b128(mrs, s_off, kb < TKB ? i * m_stride + kb * 1024 : m_end, 0);
  };
  auto store_x = [&](int slot, const u32x4_t (&v)[kXLoads]) {
#pragma unroll
    for (int t = 0; t < kXLoads; ++t) xs[slot * kSlot + xdst[t]] = v[t];
  };
  auto read_b = [&](int slot, int j) {
    const int row = slot * kSlot + (16 * j + sub) * kXPitchU4;
    return cat16(as_bf16x8(xs[row + quad]), as_bf16x8(xs[row + 4 + quad]));
  };
  // DENSE: columns 16 quad + 8 h .. +7 of the step for token fragment j, the B operand of the
  // half-h dense MFMA (the lane's A half holds the same columns of its row)
  auto read_bh = [&](int slot, int j, int h) {
    return as_bf16x8(xs[slot * kSlot + (16 * j + sub) * kXPitchU4 + 2 * quad + h]);
  };
  f32x4_t acc[NI][NJ];
#pragma unroll
  for (int i = 0; i < NI; ++i)
#pragma unroll
    for (int j = 0; j < NJ; ++j) acc[i][j] = f32x4_t{0, 0, 0, 0};

  // Step kc (u = kc mod 16, LDS slots rotating with kc mod kSlots): X of step kc is in slot
  // kc % kSlots and its first LA B fragments are in registers; X of step kc+1 is in the next slot.
  // Issue order, in 8 groups fenced from each other: each group first issues the B fragment read LA
  // groups ahead (past the step's last group: the first fragments of step kc+1) and its share of the
  // step's memory work (group 0: the LDS writes of X of step kc+kLead, whose slot's last reads
  // finished before an earlier barrier; groups 1 .. NI/4: four S loads of step kc+P-1 each; the
  // next group: the X loads of step kc+kLead+PX and, at a block's first step, the next block's
  // metadata), then its NI MFMAs. A barrier after every kBarEvery-th step.
  constexpr int kXGroup = (NI + 3) / 4 + 1;
  static_assert(kXGroup < NJ, "every load has a group");
  auto step = [&](int kc, int s0, auto uu) {
    constexpr int u = decltype(uu)::value;
    constexpr int d = u % P, dprev = (u + P - 1) % P, xq = (u + kLead) % PX, mq = (u / 8) % 2;
    const int cur = (s0 + u) % kSlots, nxt = (s0 + u + 1) % kSlots, wr = (s0 + u + kLead) % kSlots;
    static_for<NJ>([&](auto jj) {
      constexpr int j = decltype(jj)::value;
      if constexpr (j == 0) store_x(wr, xr[xq]);
      bx[(j + LA) % (LA + 1)] = j + LA < NJ ? read_b(cur, j + LA) : read_b(nxt, j + LA - NJ);
      if constexpr (j >= 1 && j < kXGroup) {
#pragma unroll
        for (int i = 4 * (j - 1); i < (4 * j < NI ? 4 * j : NI); ++i) load_s_frag(kc + P - 1, i, sa[dprev][i]);
      }
      if constexpr (j == kXGroup) {
        load_x(kc + kLead + PX, xr[xq]);
        if constexpr (u % 8 == 0) load_m(kc / 8 + 1, mb[mq ^ 1]);
      }
#pragma unroll
      for (int i = 0; i < NI; ++i)
        smfmac_acc<u % 2>(acc[i][j], as_bf16x8(sa[d][i]), bx[j % (LA + 1)], mb[mq][i][(u % 8) / 2]);
      __builtin_amdgcn_sched_barrier(0);
    });
    if constexpr (u % kBarEvery == kBarEvery - 1) lds_barrier();
  };
  // DENSE step: the same memory work, but the product of a step runs as two halves of 32 columns.
  // At the start of each half every fragment's kept pairs are expanded to dense bfloat16 with the
  // step's nibbles (vector ALU, registers only); then 8 groups, one per token fragment, each read
  // the B half fragment LA groups ahead and run NI dense MFMAs: 16 groups and 2*NI*NJ MFMAs a step.
  auto step_dense = [&](int kc, int s0, auto uu) {
    constexpr int u = decltype(uu)::value;
    constexpr int d = u % P, dprev = (u + P - 1) % P, xq = (u + kLead) % PX, mq = (u / 8) % 2;
    const int cur = (s0 + u) % kSlots, nxt = (s0 + u + 1) % kSlots, wr = (s0 + u + kLead) % kSlots;
    u32x4_t ea[NI];
    static_for<2 * NJ>([&](auto gg) {
      constexpr int g = decltype(gg)::value, h = g / NJ, j = g % NJ, gn = g + LA;
      if constexpr (j == 0) {
#pragma unroll
        for (int i = 0; i < NI; ++i) {
          const uint32_t nib = (mb[mq][i][(u % 8) / 2] >> (16 * (u % 2) + 8 * h)) & 0xFFu;
          ea[i] = expand_groups(sa[d][i][2 * h], sa[d][i][2 * h + 1], nib);
        }
#pragma unroll
        for (int i = 0; i < NI; i += 2) operand_fence(ea[i], ea[i + 1]);  // vector-ALU writes, then MFMA reads
      }
      if constexpr (g == 0) store_x(wr, xr[xq]);
      bh[gn % (LA + 1)] = gn < 2 * NJ ? read_bh(cur, gn % NJ, gn / NJ) : read_bh(nxt, gn - 2 * NJ, 0);
      if constexpr (g >= 1 && g < kXGroup) {
#pragma unroll
        for (int i = 4 * (g - 1); i < (4 * g < NI ? 4 * g : NI); ++i) load_s_frag(kc + P - 1, i, sa[dprev][i]);
      }
      if constexpr (g == kXGroup) {
        load_x(kc + kLead + PX, xr[xq]);
        if constexpr (u % 8 == 0) load_m(kc / 8 + 1, mb[mq ^ 1]);
      }
#pragma unroll
      for (int i = 0; i < NI; ++i) mfma_dense_acc(acc[i][j], as_bf16x8(ea[i]), bh[g % (LA + 1)]);
      if constexpr (j == NJ - 1) {
#pragma unroll
        for (int i = 0; i < NI; i += 2) operand_fence(ea[i], ea[i + 1]);  // last MFMA reads, then rewrites
      }
      __builtin_amdgcn_sched_barrier(0);
    });
    if constexpr (u % kBarEvery == kBarEvery - 1) lds_barrier();
  };

  // The first two 64-rank blocks of the rank-r term run first (the accumulators start from U T^T),
  // with every load they need issued together: T's float32 partials of both blocks (all slices
  // when there are at most two), then U's fragments of block 0 once block 0's T pair is in LDS.
  const int nrow0 = n0 + wave * 16 * NI;
  const int r_pre = min(r, 64 * kPreBlocks);
  accumulator_fence(acc);  // the zeros written above, before the first smfmac_acc reads them
  if (r_pre > 0) {
    const bool two = r_pre > 64;  // wave-uniform: the second block's T pair is built only when used
    TPairBuilder<BM, 64 * WAVES, 2> tb0, tb1;
    tb0.init(Tpart, slices, M, r, m0, 0, threadIdx.x);
    tb1.init(Tpart, slices, M, r, m0, 64, threadIdx.x);  // ranks >= r read as zeros
    tb0.issue(0);
    if (two) tb1.issue(0);
    __builtin_amdgcn_sched_barrier(0);
    tb0.finish(tp, tp + kSlot);
    UFragments<NI> uf0, uf1;
    uf0.load(U, n_out, r, 0, nrow0, lane);
    __builtin_amdgcn_sched_barrier(0);
    if (two) tb1.finish(tp + 2 * kSlot, tp + 3 * kSlot);
    lds_barrier();
    if (r_pre > 64) uf1.load(U, n_out, r, 64, nrow0, lane);
    lowrank_block_acc<NI, NJ>(acc, uf0, tp, tp + kSlot);
    if (r_pre > 64) lowrank_block_acc<NI, NJ>(acc, uf1, tp + 2 * kSlot, tp + 3 * kSlot);
    lds_barrier();  // every wave's reads of the T planes are done before the ring overwrites them
  }

  // Prologue: virtual steps v = -VS .. -1 issue what a step would (X of step v+2 into LDS, S of
  // step v+P-1, X of step v+2+PX), so the loop starts with the steady state's loads in flight; the
  // first metadata block goes first.
  load_m(0, mb[0]);
  constexpr int VS = (P - 1 > PX + kLead) ? P - 1 : PX + kLead;
  static_for<VS>([&](auto ii) {
    constexpr int v = decltype(ii)::value - VS;
    if constexpr (v >= -kLead) store_x(v + kLead, xr[(v + kLead + PX) % PX]);
    if constexpr (v + P - 1 >= 0) {
#pragma unroll
      for (int i = 0; i < NI; ++i) load_s_frag(v + P - 1, i, sa[(v + P - 1) % P][i]);
    }
    if constexpr (v + kLead + PX >= 0) load_x(v + kLead + PX, xr[(v + kLead + PX) % PX]);
  });
  lds_barrier();
  static_for<LA>([&](auto jj) {
    constexpr int g = decltype(jj)::value;
    if constexpr (DENSE)
      bh[g] = read_bh(0, g % NJ, g / NJ);
    else
      bx[g] = read_b(0, g);
  });
  __builtin_amdgcn_sched_barrier(0);
  for (int kc0 = 0; kc0 < nk_pad; kc0 += kUnroll) {
    const int s0 = kc0 % kSlots;
    static_for<kUnroll>([&](auto u) {
      if constexpr (DENSE)
        step_dense(kc0 + decltype(u)::value, s0, u);
      else
        step(kc0 + decltype(u)::value, s0, u);
    });
  }
  // ranks past the first kPreBlocks blocks, 64 at a time: T's pair in slots 0 and 1 (the last
  // step's barrier retired every LDS access of the loop), U fragments from memory
  for (int j0 = r_pre; j0 < r; j0 += 64) {
    UFragments<NI> uf;
    uf.load(U, n_out, r, j0, nrow0, lane);
    build_t_pair<BM, 64 * WAVES>(Tpart, slices, M, r, m0, j0, xs, xs + kSlot, threadIdx.x);
    lds_barrier();
    lowrank_block_acc<NI, NJ>(acc, uf, xs, xs + kSlot);
    lds_barrier();
  }
  accumulator_fence(acc);  // the last smfmac_acc results, before the stores
  if constexpr ((EPI & kEpiRows) != 0) {
    static_assert(WAVES * 32 * (16 * NI + 4) * 4 <= (int)sizeof(xs), "a private buffer per wave");
    lds_barrier();  // every wave's reads of the ring are done before it is reused
    store_tile_rows_lds<NI, NJ, (EPI & kEpiDirectNT) != 0>(acc, (float*)xs + wave * 32 * (16 * NI + 4), Y, y_bf16, M,
                                                          n_out, nrow0, m0, lane);
  } else {
    store_tile<NI, NJ, (EPI & kEpiDirectNT) != 0>(acc, Y, y_bf16, M, n_out, nrow0, m0, lane);
  }
}

// The 512-row tile when the launch's layers together still give every CU of the chip at least one
// tile, else 256 rows.
constexpr int64_t kWideMinTiles = 256;
int64_t prefill_rows(int64_t M, int64_t n_out, int layers) {
  return layers * ceil_div(n_out, 512) * ceil_div(M, 128) >= kWideMinTiles ? 512 : 256;
}

// prefill: one workgroup per tile (512 or 256 rows x 128 tokens) of each layer, tiles dealt to the
// 8 XCDs in equal ranges
dim3 prefill_grid(int64_t M, int64_t n_out, int layers) {
  const int64_t n_tiles = layers * ceil_div(n_out, prefill_rows(M, n_out, layers)) * ceil_div(M, 128);
  return dim3((unsigned)(8 * ceil_div(n_tiles, 8)));
}

LayerGroup make_group(int layers, const void* const* X, const void* const* values, const uint32_t* const* meta,
                      const void* const* U, const float* const* Tpart, void* const* Y) {
  LayerGroup g{};
  for (int i = 0; i < kMaxGroup; ++i) {
    const int l = i < layers ? i : layers - 1;  // unused entries repeat the last layer
    g.X[i] = (const uint16_t*)X[l];
    g.values[i] = (const u32x4_t*)values[l];
    g.meta[i] = meta[l];
    g.U[i] = (const uint16_t*)U[l];
    g.Tpart[i] = Tpart[l];
    g.Y[i] = Y[l];
  }
  return g;
}

}  // namespace

bool linear_grids_fit(int64_t M, int64_t n_in, int64_t n_out, int64_t r, bool bf16) {
  if (!lowrank_grids_fit(M, n_in, r, bf16)) return false;
  if (!bf16) return grid_fits(linear_f32_grid(M, n_out), 256);
  if (M <= kDecodeMaxTokens) return decode_grids_fit(M, n_out);
  return grid_fits(prefill_grid(M, n_out, 1), 256);
}

bool linear_group_grid_fits(int64_t M, int64_t n_out, int layers) {
  return grid_fits(prefill_grid(M, n_out, layers), 256);
}

hipError_t launch_linear_bf16_group(int layers, const void* const* X, int64_t M, int64_t n_in,
                                    const void* const* values, const uint32_t* const* meta, int64_t n_out,
                                    const void* const* U, int64_t r, const float* const* Tpart, int slices,
                                    void* const* Y, bool y_bf16, hipStream_t stream) {
  const int yb = y_bf16 ? 1 : 0;
  constexpr int BM = 128;
  const int BN = (int)prefill_rows(M, n_out, layers);
  const int tiles_n = (int)ceil_div(n_out, BN), tiles_m = (int)ceil_div(M, BM);
  const dim3 grid = prefill_grid(M, n_out, layers);
  const int per_xcd = (int)grid.x / 8;
  const int group_m = 4;
  const LayerGroup lg = make_group(layers, X, values, meta, U, Tpart, Y);
  // A Y above 96 MiB is stored non-temporally (kept in the 256 MB Infinity Cache it evicts the S and
  // X rows that later tile groups re-read, and leaves dirty lines for the next kernels to write
  // back), and as whole token rows through LDS: non-temporal 16-byte fragment pieces would leave
  // partial cache lines (a 470 MB Y counted as 727 MB of writes). Measured against fragment stores:
  // -5.5 % at 4096/8192 tokens x 14336 outputs; for the 128 MiB Y of an 8192-token 4096-output layer
  // the layer alone is 1-5 % slower but the block's step 0.8 % faster (the following pack and first
  // stage gain). Smaller Y: row stores for the 256-row tiles, whose one or two rounds leave the final
  // stores exposed (-1 to -3 %); fragment stores for the 512-row tiles (the row transpose measured
  // +1-2 %).
  const bool y_nt = (double)M * n_out * (y_bf16 ? 2 : 4) > kNonTemporalYBytes;
  // eight waves, two per SIMD, each owning 16 NI rows x 128 tokens: NI = 4 for the 512-row tile, 2 for
  // the 256-row one (measured against one wave per SIMD with twice the rows: 3-6 % faster on the
  // 512-row tiles, 8 % on the 256-row tiles)
  const auto launch = [&](auto kernel) {
    kernel<<<grid, dim3(512), 0, stream>>>(lg, layers, slices, yb, (int)M, (int)n_in, (int)n_out, (int)r, tiles_n,
                                           tiles_m, per_xcd, group_m);
  };
  if (BN == 512) {
    if (y_nt)
      launch(linear_prefill_wide_kernel<4, 1, 2, kEpiRowsNT, 8>);
    else
      launch(linear_prefill_wide_kernel<4, 1, 2, kEpiDirect, 8>);
  } else {  // fewer than 256 tiles of 512 rows: Y is below 17 M elements, never non-temporal
    launch(linear_prefill_wide_kernel<2, 1, 2, kEpiRows, 8>);
  }
  return hipGetLastError();
}

hipError_t launch_linear_bf16(const void* X, int64_t M, int64_t n_in, const void* values, const uint32_t* meta,
                              int64_t n_out, const void* U, int64_t r, const float* Tpart, int slices, void* Y,
                              bool y_bf16, hipStream_t stream) {
  return launch_linear_bf16_group(1, &X, M, n_in, &values, &meta, n_out, &U, r, &Tpart, slices, &Y, y_bf16, stream);
}

bool linear_dense_grids_fit(int64_t M, int64_t n_out) { return grid_fits(prefill_grid(M, n_out, 1), 256); }

hipError_t launch_linear_bf16_dense(const void* X, int64_t M, int64_t n_in, const void* values, const uint32_t* meta,
                                    int64_t n_out, const void* U, int64_t r, const float* Tpart, int slices, void* Y,
                                    hipStream_t stream) {
  constexpr int BM = 128;
  const int BN = (int)prefill_rows(M, n_out, 1);
  const int tiles_n = (int)ceil_div(n_out, BN), tiles_m = (int)ceil_div(M, BM);
  const dim3 grid = prefill_grid(M, n_out, 1);
  const int per_xcd = (int)grid.x / 8;
  const int group_m = 4;
  const bool y_nt = (double)M * n_out * 4 > kNonTemporalYBytes;
  const LayerGroup lg = make_group(1, &X, &values, &meta, &U, &Tpart, &Y);
  const auto args = [&](auto kernel, int waves) {
    kernel<<<grid, dim3(64 * waves), 0, stream>>>(lg, 1, slices, 0, (int)M, (int)n_in, (int)n_out, (int)r, tiles_n,
                                                  tiles_m, per_xcd, group_m);
  };
  if (BN == 512) {
    if (y_nt)
      args(linear_prefill_wide_kernel<4, 1, 2, kEpiRowsNT, 8, true>, 8);
    else
      args(linear_prefill_wide_kernel<4, 1, 2, kEpiDirect, 8, true>, 8);
  } else {
    args(linear_prefill_wide_kernel<2, 1, 2, kEpiRows, 8, true>, 8);
  }
  return hipGetLastError();
}

}  // namespace splr
