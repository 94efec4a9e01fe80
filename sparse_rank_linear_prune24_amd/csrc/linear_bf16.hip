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
// The rank-r term is folded into the same accumulators with the same instruction (before the main
// loop when r <= 64, so that it overlaps the loop's first loads; block by block after it otherwise):
// dense U is the sum of two 2:4 matrices with fixed patterns (positions 0,1 and 2,3 of every group
// of four ranks), so acc += U_tile T_tile^T is two structured-sparse MFMAs per 64 ranks with
// constant index operands. T (float32) enters as a bfloat16 high part plus a bfloat16 correction.
// Y is stored once.
//
// Kernels (M > 64 tokens; fewer tokens take the decode kernel in decode.hip):
//   prefill      -- workgroup tile 256 rows x 128 tokens, 4 waves, each owning 64 rows and all
//                   tokens, so every S fragment is used by one wave and goes global -> registers;
//                   X is shared through a two-slot LDS ring; P K steps of loads in flight; one
//                   barrier per K step; workgroups remapped so the tiles that one XCD (own L2)
//                   runs share X and S.
//   prefill wide -- 512 rows x 128 tokens with the accumulators in the matrix-core accumulator
//                   registers, raw buffer loads, a five-slot X ring; taken when the grid still
//                   has a tile for every CU.
#include "common.hpp"
#include "kernels.hpp"
#include "tile_common.hpp"

namespace splr {
namespace {
// ----------------------------------------------------------------------------------- prefill

// EPI: how Y is stored -- kEpiDirect (fragment order), kEpiRows (row-contiguous through LDS),
// kEpiDirectNT (fragment order, non-temporal)
constexpr int kEpiDirect = 0, kEpiRows = 1, kEpiDirectNT = 2;
template <int NI, int NJ, int P, int PX, int EPI>
__global__ __launch_bounds__(256) void linear_prefill_kernel(
    const uint16_t* __restrict__ X, const u32x4_t* __restrict__ values, const uint32_t* __restrict__ meta,
    const uint16_t* __restrict__ U, const float* __restrict__ Tpart, int slices, void* __restrict__ Y, int y_bf16,
    int M, int K, int n_out, int r, int tiles_n, int tiles_m, int tiles_per_xcd, int group_m) {
  constexpr int WAVES = 4;
  constexpr int BN = 16 * NI * WAVES;
  constexpr int BM = 16 * NJ;
  constexpr int kXLoads = BM / (8 * WAVES);  // X load instructions per wave per step (8 tokens each)
  static_assert(BM % (8 * WAVES) == 0, "X stage must split evenly over the waves");
  static_assert(P >= 2 && PX >= 2 && P % 2 == 0 && PX % 2 == 0, "prefetch distances must be even");
  constexpr int kUnroll = lcm_int(P, PX);  // unroll factor: every register slot index is a constant
  // the two LDS slots are separate objects, so the compiler may move reads of one past writes of
  // the other
  __shared__ u32x4_t xs0[BM * kXPitchU4];
  __shared__ u32x4_t xs1[BM * kXPitchU4];
  // T's bfloat16 pair for this tile's tokens (hi, lo planes per 64 ranks), built before the main
  // loop when r <= 64 * kPreRankBlocks (registers are free then and the loads overlap the start),
  // and this tile's U rows when r <= 64
  __shared__ u32x4_t tpair[2 * kPreRankBlocks][BM * kXPitchU4];
  __shared__ u32x4_t ulds[BN * kXPitchU4];

  // XCD-aware tile order: workgroup b runs on XCD b % 8; each XCD gets a contiguous range of
  // logical tiles, walked in groups of `group_m` token tiles, so its tiles share X and S rows.
  const int b = blockIdx.x;
  const int logical = (b & 7) * tiles_per_xcd + (b >> 3);
  if (logical >= tiles_n * tiles_m) return;
  const int per_group = group_m * tiles_n;
  const int g = logical / per_group;
  const int first_m = g * group_m;
  const int gsize = min(group_m, tiles_m - first_m);
  const int in_group = logical - g * per_group;
  const int m0 = (first_m + in_group % gsize) * BM;
  const int n0 = (in_group / gsize) * BN;

  // the wave index is uniform across the wave; readfirstlane lets the compiler see that (scalar
  // loop control instead of exec-mask loops)
  const int lane = threadIdx.x & 63, wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int sub = lane & 15, quad = lane >> 4;
  const int TK = (K + 63) / 64, TR = (n_out + 15) / 16;
  const int nk_pad = (TK + kUnroll - 1) / kUnroll * kUnroll;

  // S fragments of this wave: tile rows (clamped; rows past n_out are zero padding or unused)
  const u32x4_t* vsrc[NI];
  const uint16_t* msrc[NI];  // this lane's 16 index bits of tile column 0: unit 0 of its slot (= lane)
  const int TKB = meta_blocks(TK);
#pragma unroll
  for (int i = 0; i < NI; ++i) {
    const int tr = min(n0 / 16 + wave * NI + i, TR - 1);
    vsrc[i] = values + (size_t)tr * TK * 64 + lane;
    msrc[i] = (const uint16_t*)meta + ((size_t)tr * TKB * 64 + lane) * 8;
  }
  // X rows this lane loads: token m0 + wave*BM/4 + 8 t + lane/8, 16-byte chunk lane%8 of a step
  const int xchunk = lane & 7;
  const uint16_t* xsrc[kXLoads];
  int xdst[kXLoads];
#pragma unroll
  for (int t = 0; t < kXLoads; ++t) {
    const int tloc = wave * (BM / WAVES) + 8 * t + (lane >> 3);
    xsrc[t] = X + (size_t)min(m0 + tloc, M - 1) * K + 8 * xchunk;
    xdst[t] = tloc * kXPitchU4 + xchunk;
  }

  u32x4_t xr[PX][kXLoads];  // X register ring: X of step kc is loaded PX steps before it goes to LDS
  u32x4_t sa[P][NI];
  uint32_t sw[P][NI];  // index operands, zero-extended 16-bit loads
  bf16x16_t bx[2][NJ];
  auto load_x = [&](int kc, u32x4_t (&v)[kXLoads]) {
    int col = min(kc, TK - 1) * 64;
    if (col + 8 * xchunk >= K) col -= 32;  // half tail step: re-read valid columns (S is zero there)
#pragma unroll
    for (int t = 0; t < kXLoads; ++t) v[t] = *(const u32x4_t*)(xsrc[t] + col);
  };
  auto load_s = [&](int kc, u32x4_t (&va)[NI], uint32_t (&wa)[NI]) {
    const int kk = min(kc, TK - 1);
#pragma unroll
    for (int i = 0; i < NI; ++i) {
      va[i] = vsrc[i][(size_t)kk * 64];
      wa[i] = msrc[i][(size_t)(kk >> 3) * 512 + (kk & 7)];
    }
  };
  auto store_x = [&](u32x4_t* slot, const u32x4_t (&v)[kXLoads]) {
#pragma unroll
    for (int t = 0; t < kXLoads; ++t) slot[xdst[t]] = v[t];
  };
  auto read_b = [&](const u32x4_t* slot, bf16x16_t (&b)[NJ]) {
#pragma unroll
    for (int j = 0; j < NJ; ++j) {
      const int row = (16 * j + sub) * kXPitchU4;
      b[j] = cat16(as_bf16x8(slot[row + quad]), as_bf16x8(slot[row + 4 + quad]));
    }
  };
  f32x4_t acc[NI][NJ];
#pragma unroll
  for (int i = 0; i < NI; ++i)
#pragma unroll
    for (int j = 0; j < NJ; ++j) acc[i][j] = f32x4_t{0, 0, 0, 0};

  // Software pipeline, one barrier per K step. At step kc (S register slot kc % P, X register slot
  // (kc+2) % PX, LDS slot and B register parity b = kc % 2): the B fragments of step kc are already
  // in registers bx[b], X of step kc+1 is in LDS slot b^1, X of step kc+2 is in registers. The step
  // writes X of step kc+2 into LDS slot b (whose reads, of step kc, completed before the previous
  // barrier), reads the B fragments of step kc+1 into bx[b^1] while its MFMAs run, refills the S
  // slot of step kc-1 with step kc+P-1 and the X register slot with step kc+2+PX, and ends with the
  // barrier. The instruction order inside a step is pinned (LDS writes, then LDS reads and global
  // loads each paired with an MFMA), and no instruction crosses a step boundary. Padding steps
  // (kc >= TK) zero the S operand.
  auto step = [&](int kc, auto uu, auto masked) {
    constexpr int u = decltype(uu)::value;
    constexpr int d = u % P, b = u & 1, dprev = (u + P - 1) % P, xq = (u + 2) % PX;
    store_x(b ? xs1 : xs0, xr[xq]);
    read_b(b ? xs0 : xs1, bx[b ^ 1]);
    const uint32_t keep = (!decltype(masked)::value || kc < TK) ? ~0u : 0u;
    bf16x8_t a[NI];
    int idx[NI];
#pragma unroll
    for (int i = 0; i < NI; ++i) {
      a[i] = decltype(masked)::value ? as_bf16x8(sa[d][i] & keep) : as_bf16x8(sa[d][i]);
      idx[i] = (int)(sw[d][i] & keep);
    }
#pragma unroll
    for (int j = 0; j < NJ; ++j)
#pragma unroll
      for (int i = 0; i < NI; ++i) acc[i][j] = smfmac16x16x64(a[i], bx[b][j], acc[i][j], idx[i]);
    load_s(kc + P - 1, sa[dprev], sw[dprev]);
    load_x(kc + 2 + PX, xr[xq]);
    // pinned order: the LDS writes, LDS reads and global loads are spread evenly over the MFMAs,
    // one after each MFMA, in kXLoads rounds of (1 LDS write, 2*NJ/kXLoads LDS reads, the loads'
    // share), so that no queue fills and blocks the in-order issue of the MFMAs
    constexpr int kReads = 2 * NJ, kLoads = 2 * NI + kXLoads, kMfma = NI * NJ, kRounds = kXLoads;
    static_assert(kReads % kRounds == 0 && kLoads % kRounds == 0, "even spread");
    static_assert(kRounds * (1 + kReads / kRounds + kLoads / kRounds) <= kMfma, "one MFMA per memory op");
#pragma unroll
    for (int q = 0; q < kRounds; ++q) {
      __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
      __builtin_amdgcn_sched_group_barrier(0x200, 1, 0);
#pragma unroll
      for (int t = 0; t < kReads / kRounds; ++t) {
        __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
        __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);
      }
#pragma unroll
      for (int t = 0; t < kLoads / kRounds; ++t) {
        __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
        __builtin_amdgcn_sched_group_barrier(0x020, 1, 0);
      }
    }
    __builtin_amdgcn_sched_group_barrier(0x008, kMfma - kRounds * (1 + (kReads + kLoads) / kRounds), 0);
    lds_barrier();
    __builtin_amdgcn_sched_barrier(0);
  };

  // rank-r operands staged before the main loop: loads issued here, finished after the loop's
  // prologue has issued its own loads (published by the prologue's barriers)
  const bool t_pre = r <= 64 * kPreRankBlocks, u_pre = r <= 64;
  TPairBuilder<BM, 64 * WAVES, 2> tb[kPreRankBlocks];
  UStager<BN, 64 * WAVES> us;
  if (t_pre) {
#pragma unroll
    for (int b = 0; b < kPreRankBlocks; ++b)
      if (64 * b < r) {
        tb[b].init(Tpart, slices, M, r, m0, 64 * b, threadIdx.x);
        tb[b].issue(0);
      }
  }
  if (u_pre && r > 0) us.issue(U, n_out, r, n0, 0, threadIdx.x);

  // Prologue: virtual steps v = -VS .. -1 issue exactly what a step would (X of step v+2 into LDS,
  // S of step v+P-1, X of step v+2+PX), so the loop is entered with the loads in flight in the same
  // order as in the steady state and the wait counts the compiler derives need no extra waits.
  constexpr int VS = (P - 1 > PX + 2) ? P - 1 : PX + 2;
  static_for<VS>([&](auto ii) {
    constexpr int v = decltype(ii)::value - VS;
    if constexpr (v >= -2) store_x(((v + 2) & 1) ? xs1 : xs0, xr[(v + 2 + PX) % PX]);
    if constexpr (v + P - 1 >= 0) load_s(v + P - 1, sa[(v + P - 1) % P], sw[(v + P - 1) % P]);
    if constexpr (v + 2 + PX >= 0) load_x(v + 2 + PX, xr[(v + 2 + PX) % PX]);
  });
  if (t_pre) {
#pragma unroll
    for (int b = 0; b < kPreRankBlocks; ++b)
      if (64 * b < r) tb[b].finish(tpair[2 * b], tpair[2 * b + 1]);
  }
  if (u_pre && r > 0) us.finish(ulds);
  lds_barrier();
  const int nrow0 = n0 + wave * 16 * NI;
  // rank-r term first when T's pair is already in LDS: its MFMAs run while the main loop's first
  // loads are in flight (the accumulators start from U T^T instead of zero)
  if (t_pre) {
#pragma unroll
    for (int b = 0; b < kPreRankBlocks; ++b)
      if (64 * b < r)
        lowrank_block<NI, NJ>(acc, U, tpair[2 * b], tpair[2 * b + 1], n_out, r, 64 * b, nrow0, lane,
                              u_pre ? ulds : nullptr, wave * 16 * NI);
  }
  __builtin_amdgcn_sched_barrier(0);
  read_b(xs0, bx[0]);
  lds_barrier();  // every wave's reads of slot 0 are done before step 0 overwrites it
  __builtin_amdgcn_sched_barrier(0);
  const int nk_full = TK / kUnroll * kUnroll;  // steps that need no masking
  for (int kc0 = 0; kc0 < nk_full; kc0 += kUnroll)
    static_for<kUnroll>([&](auto u) { step(kc0 + decltype(u)::value, u, std::false_type{}); });
  for (int kc0 = nk_full; kc0 < nk_pad; kc0 += kUnroll)
    static_for<kUnroll>([&](auto u) { step(kc0 + decltype(u)::value, u, std::true_type{}); });

  // larger r: the rank-r term, 64 ranks at a time, after the loop; the workgroup builds T's pair
  // block by block in the now free X slots (the last step's barrier has retired every read of them)
  // and stages the block's U rows in the U slot (unused before the loop when r > 64), the loads of
  // both in flight together
  if (!t_pre) {
    for (int j0 = 0; j0 < r; j0 += 64) {
      TPairBuilder<BM, 64 * WAVES, 2> tbp;
      UStager<BN, 64 * WAVES> usp;
      tbp.init(Tpart, slices, M, r, m0, j0, threadIdx.x);
      tbp.issue(0);
      usp.issue(U, n_out, r, n0, j0, threadIdx.x);
      __builtin_amdgcn_sched_barrier(0);
      tbp.finish(xs0, xs1);
      usp.finish(ulds);
      lds_barrier();
      lowrank_block<NI, NJ>(acc, U, xs0, xs1, n_out, r, j0, nrow0, lane, ulds, wave * 16 * NI);
      lds_barrier();
    }
  }
  if constexpr (EPI == kEpiRows) {
    // Y leaves through LDS (every slot is free now: the last barrier above retired all reads of
    // them); waves 0, 1 use the T pair slot, waves 2, 3 the U slot
    static_assert(2 * 64 * kYPitch * 4 <= (int)sizeof(tpair) && 2 * 64 * kYPitch * 4 <= (int)sizeof(ulds),
                  "epilogue buffers fit");
    float* ybuf = (wave < 2 ? (float*)&tpair[0][0] : (float*)&ulds[0]) + (wave & 1) * 64 * kYPitch;
    store_tile_rows<NI, NJ>(acc, ybuf, Y, y_bf16, M, n_out, nrow0, m0);
  } else {
    store_tile<NI, NJ, EPI == kEpiDirectNT>(acc, Y, y_bf16, M, n_out, nrow0, m0, lane);
  }
}

// ----------------------------------------------------------------------------------- prefill, wide tile

// Word 3 of a raw buffer descriptor on gfx9-family GPUs: 32-bit data format, no swizzle, no index
// stride (plain byte-addressed loads).
constexpr int kBufferFlags = 0x00020000;

// The structured-sparse MFMA with its accumulator pinned to the matrix-core accumulator registers
// (the compiler would otherwise spread 256 accumulators over both register files and copy them
// every step). ABID selects the half of the 32-bit index register the instruction reads (a
// metadata word holds the indices of two tile columns). Hazard rules this relies on, kept by the
// kernel below: the A, B and index operands come straight from loads (the waits for loads precede
// the instruction; no vector-ALU instruction writes an operand), an accumulator is written by these
// instructions only and 64 instructions apart, and anything else touches the accumulators only
// across accumulator_fence().
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
// T's bfloat16 pair from the LDS planes hi / lo one token fragment at a time. The MFMAs of a token
// fragment run over the row fragments innermost, so consecutive MFMAs write different accumulators.
template <int NI, int NJ>
__device__ __forceinline__ void lowrank_block_acc(f32x4_t (&acc)[NI][NJ], const UFragments<NI>& uf,
                                                  const u32x4_t* hi, const u32x4_t* lo, int lane) {
  static_assert(NI % 2 == 0, "U fragments fenced two rows at a time");
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
#pragma unroll
  for (int j = 0; j < NJ; ++j) {
    const int row = (16 * j + sub) * kXPitchU4;
    bf16x16_t th = cat16(as_bf16x8(hi[row + quad]), as_bf16x8(hi[row + 4 + quad]));
    bf16x16_t tl = cat16(as_bf16x8(lo[row + quad]), as_bf16x8(lo[row + 4 + quad]));
    operand_fence(th, tl);
#pragma unroll
    for (int i = 0; i < NI; ++i) smfmac_acc<0>(acc[i][j], u01[i], th, i01);
#pragma unroll
    for (int i = 0; i < NI; ++i) smfmac_acc<0>(acc[i][j], u23[i], th, i23);
#pragma unroll
    for (int i = 0; i < NI; ++i) smfmac_acc<0>(acc[i][j], u01[i], tl, i01);
#pragma unroll
    for (int i = 0; i < NI; ++i) smfmac_acc<0>(acc[i][j], u23[i], tl, i23);
  }
  operand_fence(i01, i23);  // the index registers outlive the last MFMA that reads them
}

// Prefill kernel with the accumulators in the matrix-core accumulator registers: workgroup tile
// 16*NI*WAVES rows x 128 tokens, each wave owning 16*NI rows (NI S fragments) x all 128 tokens, so
// NI*8 accumulator fragments = 32*NI accumulator registers per lane. With WAVES = 8 (two waves per
// SIMD, NI = 4: 512 rows) each wave has 128 accumulator and 128 arch registers, and one wave's
// loads, LDS traffic and barrier waits overlap the other's MFMAs; WAVES = 4 (NI = 8) is the same
// tile with one wave per SIMD and 256 + 256 registers. Per 64-column K step a CU loads 4 KiB of S
// values per 16 rows and 16 KiB of X, and each lane loads its metadata once per 8 steps: one
// 16-byte word group per fragment holds its indices for a whole metadata block. Each 16-token
// group's B fragment is read from LDS LA groups ahead of its NI MFMAs; X goes through a five-slot
// LDS ring with a barrier every second step. The first two 64-rank blocks of the rank-r term run
// before the main loop (their T pairs in four of the ring's slots); further blocks after it.
template <int NI, int LA, int P, int EPI, int WAVES = 4, bool DENSE = false>
__global__ __launch_bounds__(64 * WAVES) __attribute__((amdgpu_waves_per_eu(WAVES / 4, WAVES / 4))) void
linear_prefill_wide_kernel(
    const uint16_t* __restrict__ X, const u32x4_t* __restrict__ values, const uint32_t* __restrict__ meta,
    const uint16_t* __restrict__ U, const float* __restrict__ Tpart, int slices, void* __restrict__ Y, int y_bf16,
    int M, int K, int n_out, int r, int tiles_n, int tiles_m, int tiles_per_xcd, int group_m) {
  constexpr int NJ = 8, PX = 2;
  static_assert(WAVES == 4 || WAVES == 8, "one or two waves per SIMD");
  constexpr int BN = 16 * NI * WAVES;  // 512 or 256 rows
  constexpr int BM = 16 * NJ;          // 128 tokens
  static_assert(NI % 4 == 0 && LA >= 1 && LA < NJ, "S loads in groups of four fragments");
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

  // XCD-aware tile order (as in the 256 x 128 kernel)
  const int b = blockIdx.x;
  const int logical = (b & 7) * tiles_per_xcd + (b >> 3);
  if (logical >= tiles_n * tiles_m) return;
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
  constexpr int kXGroup = NI / 4 + 1;
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
        for (int i = 4 * (j - 1); i < 4 * j; ++i) load_s_frag(kc + P - 1, i, sa[dprev][i]);
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
        for (int i = 4 * (g - 1); i < 4 * g; ++i) load_s_frag(kc + P - 1, i, sa[dprev][i]);
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
    TPairBuilder<BM, 64 * WAVES, 2> tb0, tb1;
    tb0.init(Tpart, slices, M, r, m0, 0, threadIdx.x);
    tb1.init(Tpart, slices, M, r, m0, 64, threadIdx.x);  // ranks >= r read as zeros
    tb0.issue(0);
    tb1.issue(0);
    __builtin_amdgcn_sched_barrier(0);
    tb0.finish(tp, tp + kSlot);
    UFragments<NI> uf0, uf1;
    uf0.load(U, n_out, r, 0, nrow0, lane);
    __builtin_amdgcn_sched_barrier(0);
    tb1.finish(tp + 2 * kSlot, tp + 3 * kSlot);
    lds_barrier();
    if (r_pre > 64) uf1.load(U, n_out, r, 64, nrow0, lane);
    lowrank_block_acc<NI, NJ>(acc, uf0, tp, tp + kSlot, lane);
    if (r_pre > 64) lowrank_block_acc<NI, NJ>(acc, uf1, tp + 2 * kSlot, tp + 3 * kSlot, lane);
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
    lowrank_block_acc<NI, NJ>(acc, uf, xs, xs + kSlot, lane);
    lds_barrier();
  }
  accumulator_fence(acc);  // the last smfmac_acc results, before the stores
  store_tile<NI, NJ, EPI == kEpiDirectNT>(acc, Y, y_bf16, M, n_out, nrow0, m0, lane);
}

// The 512-row tile when it still gives every CU of the chip at least one tile, else 256 rows.
constexpr int64_t kWideMinTiles = 256;
int64_t prefill_rows(int64_t M, int64_t n_out) {
  return ceil_div(n_out, 512) * ceil_div(M, 128) >= kWideMinTiles ? 512 : 256;
}

// prefill: one workgroup per tile (512 or 256 rows x 128 tokens), tiles dealt to the 8 XCDs in
// equal ranges
dim3 prefill_grid(int64_t M, int64_t n_out) {
  const int64_t n_tiles = ceil_div(n_out, prefill_rows(M, n_out)) * ceil_div(M, 128);
  return dim3((unsigned)(8 * ceil_div(n_tiles, 8)));
}

}  // namespace

bool linear_grids_fit(int64_t M, int64_t n_in, int64_t n_out, int64_t r, bool bf16) {
  if (!lowrank_grids_fit(M, n_in, r, bf16)) return false;
  if (!bf16) return grid_fits(linear_f32_grid(M, n_out), 256);
  if (M <= kDecodeMaxTokens) return decode_grids_fit(M, n_out);
  return grid_fits(prefill_grid(M, n_out), 256);
}

hipError_t launch_linear_bf16(const void* X, int64_t M, int64_t n_in, const void* values, const uint32_t* meta,
                              int64_t n_out, const void* U, int64_t r, const float* Tpart, int slices, void* Y,
                              bool y_bf16, hipStream_t stream) {
  const int yb = y_bf16 ? 1 : 0;

  constexpr int NI = 4, NJ = 8, P = 4, PX = 2;
  constexpr int BM = 16 * NJ;
  const int BN = (int)prefill_rows(M, n_out);
  const int tiles_n = (int)ceil_div(n_out, BN), tiles_m = (int)ceil_div(M, BM);
  const int n_tiles = tiles_n * tiles_m;
  const dim3 grid = prefill_grid(M, n_out);
  const int per_xcd = (int)grid.x / 8;
  const int group_m = 4;
  // When every tile runs at once (one workgroup per CU), the Y stores of all tiles come at the end
  // together and are exposed: the row-contiguous epilogue stores them faster. With several tiles per
  // CU the stores overlap the next tile's loop, and with r > 64 the extra registers of that
  // epilogue cost spills in the rank-r blocks after the loop: there the direct epilogue is faster.
  // A Y larger than three quarters of the 256 MB Infinity Cache is stored non-temporally: kept in the
  // cache it evicts the S and X rows that later tile groups re-read (measured: -6 to -11 % on
  // 4096/8192 tokens x 14336 outputs; +5 % slower on 8192 x 4096, 134 MB, so the threshold sits
  // between).
  const bool y_nt = (double)M * n_out * (y_bf16 ? 2 : 4) > kNonTemporalYBytes;
  const dim3 block(256);
  if (BN == 512) {
    // eight waves, two per SIMD, 64 rows each (measured against four waves of 128 rows: 3-6 % faster
    // on the 8192-token layers; Y bit-identical)
    constexpr int kWideWaves = 8, kWideNI = 512 / (16 * kWideWaves);
    if (y_nt)
      linear_prefill_wide_kernel<kWideNI, 1, 2, kEpiDirectNT, kWideWaves><<<grid, dim3(64 * kWideWaves), 0, stream>>>(
          (const uint16_t*)X, (const u32x4_t*)values, meta, (const uint16_t*)U, Tpart, slices, Y, yb, (int)M,
          (int)n_in, (int)n_out, (int)r, tiles_n, tiles_m, per_xcd, group_m);
    else
      linear_prefill_wide_kernel<kWideNI, 1, 2, kEpiDirect, kWideWaves><<<grid, dim3(64 * kWideWaves), 0, stream>>>(
          (const uint16_t*)X, (const u32x4_t*)values, meta, (const uint16_t*)U, Tpart, slices, Y, yb, (int)M,
          (int)n_in, (int)n_out, (int)r, tiles_n, tiles_m, per_xcd, group_m);
    return hipGetLastError();
  }
  if (n_tiles <= kRowsEpilogueMaxTiles && r <= 64)
    linear_prefill_kernel<NI, NJ, P, PX, kEpiRows><<<grid, block, 0, stream>>>(
        (const uint16_t*)X, (const u32x4_t*)values, meta, (const uint16_t*)U, Tpart, slices, Y, yb, (int)M,
        (int)n_in, (int)n_out, (int)r, tiles_n, tiles_m, per_xcd, group_m);
  else if (y_nt)
    linear_prefill_kernel<NI, NJ, P, PX, kEpiDirectNT><<<grid, block, 0, stream>>>(
        (const uint16_t*)X, (const u32x4_t*)values, meta, (const uint16_t*)U, Tpart, slices, Y, yb, (int)M,
        (int)n_in, (int)n_out, (int)r, tiles_n, tiles_m, per_xcd, group_m);
  else
    linear_prefill_kernel<NI, NJ, P, PX, kEpiDirect><<<grid, block, 0, stream>>>(
        (const uint16_t*)X, (const u32x4_t*)values, meta, (const uint16_t*)U, Tpart, slices, Y, yb, (int)M,
        (int)n_in, (int)n_out, (int)r, tiles_n, tiles_m, per_xcd, group_m);
  return hipGetLastError();
}

bool linear_dense_grids_fit(int64_t M, int64_t n_out) { return grid_fits(prefill_grid(M, n_out), 256); }

hipError_t launch_linear_bf16_dense(const void* X, int64_t M, int64_t n_in, const void* values, const uint32_t* meta,
                                    int64_t n_out, const void* U, int64_t r, const float* Tpart, int slices, void* Y,
                                    hipStream_t stream) {
  constexpr int BM = 128;
  const int BN = (int)prefill_rows(M, n_out);
  const int tiles_n = (int)ceil_div(n_out, BN), tiles_m = (int)ceil_div(M, BM);
  const dim3 grid = prefill_grid(M, n_out);
  const int per_xcd = (int)grid.x / 8;
  const int group_m = 4;
  const bool y_nt = (double)M * n_out * 4 > kNonTemporalYBytes;
  const auto args = [&](auto kernel, int waves) {
    kernel<<<grid, dim3(64 * waves), 0, stream>>>((const uint16_t*)X, (const u32x4_t*)values, meta,
                                                  (const uint16_t*)U, Tpart, slices, Y, 0, (int)M, (int)n_in,
                                                  (int)n_out, (int)r, tiles_n, tiles_m, per_xcd, group_m);
  };
  if (BN == 512) {
    if (y_nt)
      args(linear_prefill_wide_kernel<4, 1, 2, kEpiDirectNT, 8, true>, 8);
    else
      args(linear_prefill_wide_kernel<4, 1, 2, kEpiDirect, 8, true>, 8);
  } else {
    if (y_nt)
      args(linear_prefill_wide_kernel<4, 1, 2, kEpiDirectNT, 4, true>, 4);
    else
      args(linear_prefill_wide_kernel<4, 1, 2, kEpiDirect, 4, true>, 4);
  }
  return hipGetLastError();
}

}  // namespace splr
