// Fused RMSNorm + projection (+ SwiGLU) for many rows (prefill): the
// compute-bound regime, one launch.
//
// A workgroup computes a BM x BN output tile (BM = 16*FM*WM rows, BN =
// 16*FN*WN columns per weight matrix) with WM x WN waves, each owning a
// 16*FM x 16*FN sub-tile whose fp32 accumulators stay in registers for the
// whole k loop.  The instances use 256x256 tiles (256x128 per matrix for
// SwiGLU) with eight waves, two per SIMD: of 64x128 where W' streams through
// an LDS ring, of 128x64 where each wave loads its W' fragments straight
// into registers (the large grids of plain and SwiGLU projections).
// Measured on MI355X four waves of 128x128 (one per SIMD) ran 1.8x slower,
// nothing covering one wave's barrier and memory latency.
//
// Schedule: ping-pong.  Waves 0-3 (one per SIMD) and waves
// 4-7 alternate between a compute slot -- the k-block's MFMAs, operands
// already in registers -- and a memory slot -- LDS reads of the wave's next
// k-block into registers, its share of the global-to-LDS loads, the waits --
// with a barrier between slots, so each SIMD's matrix pipe is fed by one
// wave while the other wave's memory work runs beside it (measured 2-3%
// faster than interleaving loads and MFMAs in every wave; without the
// global loads the same loop runs at the MFMA-only time, so the L2-to-CU
// delivery of the operands, about 32 KiB per k-block per CU, is what bounds
// it).
//
// Operands stream through LDS rings filled by direct global-to-LDS buffer
// loads (no register staging): W' one 32-wide k-block per slot (4 slots),
// x a pair of k-blocks per slot (2 slots).  W' lands in MFMA fragment order
// because the packed layout is fragment-major.  x arrives as whole 128-byte
// lines -- each load brings 8 rows x 64 k values -- because a direct-to-LDS
// load whose lanes fetch 16 rows x 64 bytes (half lines) measured 37.5 GB/s
// per CU from L2-resident data against 74-90 GB/s for whole lines; row r's
// 16-byte chunks are stored permuted by r/2 so the quarter-wave operand
// reads (ds_read_b128) hit distinct bank groups.  Loads past the matrix
// edges (rows >= M, columns past the packed width, k >= K) use out-of-range
// buffer offsets, which read as zero.
//
// The per-row sum of squares comes from the x fragments already in
// registers: each of the WN waves that share a row block takes a 1/WN share
// of its row fragments as the diagonal of an x x^T MFMA (measured faster
// than convert-and-FMA on the VALU).  The shares meet in LDS before the
// epilogue applies 1/RMS (and SiLU * up) to the accumulators and stores
// ([FlashNorm digest] proposals 1-2; [FlashInfer #5521] "Design" items 1-2,
// tiles kept resident across the k loop and the SwiGLU applied to the
// accumulators in registers).
#include <type_traits>

#include "fn_device.h"
#include "fn_launch.h"

namespace fn {

struct PrefillArgs {
  const void* x;
  const void* wg;    // packed W' (gate for SwiGLU)
  const void* wu;    // packed W'_up, SwiGLU only
  void* y;
  int M, K, N;
  int kblocks;       // ceil(K / 32)
  int nblocks;       // ceil(N / 16)
  float eps;
  uint8_t* q;        // fp8 output: E4M3 codes [M, N] (y unused)
  float* qs;         // fp8 output: scales [M, nblocks], one per 16-column row block
  const int* idx;    // EX: AdaLN table row of each x row [M]
  const float* bg;   // EX: AdaLN bias rows [T, N] (gate for SwiGLU)
  const float* bu;   // EX: AdaLN bias rows of W_up
  int T;             // EX: AdaLN table rows
  const float* rs;   // EX: 1/RMS of each row [M], from the AdaLN pre-pass
  const float* sg;   // F8: column scales of wg [N]
  const float* su;   // F8: column scales of wu [N]
};

typedef __attribute__((address_space(3))) void* lds_ptr;

// Raw buffer descriptor over [base, base + bytes); reads past the end return 0.
__device__ inline __amdgpu_buffer_rsrc_t make_rsrc(const void* base, int64_t bytes) {
  const int n = bytes > 0x7fffffff ? 0x7fffffff : (bytes < 0 ? 0 : (int)bytes);
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), 0, n, 0x00020000);
}

// s_waitcnt with only the vector-memory counter constrained (gfx9 encoding).
template <int N>
__device__ inline void wait_vmcnt() {
  static_assert(N >= 0 && N < 64, "vmcnt range");
  __builtin_amdgcn_s_waitcnt((N & 15) | (7 << 4) | (15 << 8) | ((N >> 4) << 14));
}

constexpr uint32_t kOutOfRange = 0x80000000u;

// EX: the projection half of the two-launch AdaLN form.  x is the operand
// the pre-pass already modulated, 1/RMS of each raw row comes from a.rs (no
// Gram blocks), and the epilogue adds the row's bias rows (zero for an
// index outside the table, whose operand row the pre-pass zeroed).
//
// PAIR (with EX, bf16 output): the operand arrives split in two bf16 parts,
// row 2m the rounded operand of x row m and row 2m+1 its remainder, and the
// kernel runs over the 2M operand rows (a.M = 2M).  A lane's accumulator
// holds 4 consecutive rows, so each pair meets in registers and the
// epilogue adds the two products before the scale, the bias and the
// SwiGLU: the product of the unrounded operand at twice the matrix work.
//
// F8: fp8 (E4M3) weights with one scale per output column, packed in 1 KiB
// fragments of 16 columns x 64 k (a pair of k-blocks, the lane's 16 bytes
// holding its 8 codes of each).  W' then travels with x: both rings hold
// pairs, filled together, and each B operand is the lane's 8 codes of the
// k-block (ds_read_b64) decoded to bf16 in the memory slot
// (v_cvt_scalef32_pk_bf16_fp8 with scale 1 is exact).  Per k-block a CU
// moves 24 KiB of operands instead of 32 and its waves read 64 KiB of LDS
// instead of 96; the column scale joins 1/RMS in the epilogue.
template <int FM, int FN, int WM, int WN, bool SW, bool Q8, bool EX = false, bool F8 = false, bool PAIR = false,
          bool WD = false>
__global__ __launch_bounds__(kWave * WM * WN) void prefill_kernel(PrefillArgs a) {
  constexpr int NW = WM * WN;
  constexpr int NMAT = SW ? 2 : 1;
  constexpr int BMF = FM * WM;                   // 16-row fragments per tile
  constexpr int BNF = FN * WN;                   // 16-column fragments per tile and matrix
  constexpr int WFR = NMAT * BNF;                // W' fragments per k-block
  constexpr int WPW = WFR / NW;                  // W' loads per wave per k-block
  constexpr int XFR = 2 * BMF;                   // x loads per pair of k-blocks (8 rows x 128 B each)
  constexpr int XPW = XFR / NW;                  // x loads per wave per pair
  constexpr int SSF = FM / WN;                   // row fragments whose squares this wave sums
  static_assert(WFR % NW == 0 && XFR % NW == 0 && FM % WN == 0, "tile shape");
  constexpr int WSLOT = WD ? 16 : WFR * kFragBytes;   // WD: no W' ring
  constexpr int XSLOT = XFR * kFragBytes;
  static_assert(4 * WSLOT + 2 * XSLOT + BMF * 64 <= 160 * 1024, "LDS budget");
  static_assert(NW == 8, "ping-pong: two groups of one wave per SIMD");
  static_assert(!PAIR || (EX && !Q8), "split operand: the two-launch AdaLN form, bf16 output");
  static_assert(!WD || !F8, "W' fragments straight to registers: bf16 weights");
  constexpr bool BIAS = EX;

  __shared__ __attribute__((aligned(1024))) uint8_t wring0[WSLOT];
  __shared__ __attribute__((aligned(1024))) uint8_t wring1[WSLOT];
  __shared__ __attribute__((aligned(1024))) uint8_t wring2[WSLOT];
  __shared__ __attribute__((aligned(1024))) uint8_t wring3[WSLOT];
  __shared__ __attribute__((aligned(1024))) uint8_t xring0[XSLOT];
  __shared__ __attribute__((aligned(1024))) uint8_t xring1[XSLOT];
  __shared__ __attribute__((aligned(16))) float ssbuf[BMF * 16];   // sums of squares, then 1/RMS
  auto wslot = [&](int s) __attribute__((always_inline)) -> uint8_t* {
    return s == 0 ? wring0 : (s == 1 ? wring1 : (s == 2 ? wring2 : wring3));
  };
  auto xslot = [&](int s) __attribute__((always_inline)) -> uint8_t* { return s == 0 ? xring0 : xring1; };

  const int lane = threadIdx.x & (kWave - 1);
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x / kWave);
  const int wm = wave / WN, wn = wave % WN;
  const int lrow = lane & 15, lgrp = lane >> 4;
  // Row fragment of the tile held in the wave's i-th A operand.  WD: rotated
  // by the wave's column group so that the fragments whose squares it sums
  // (the SSF fragments from wn * SSF) sit first, at compile-time positions.
  static_assert(!WD || (FM & (FM - 1)) == 0, "rotated fragment order");
  auto rfrag = [&](int i) __attribute__((always_inline)) -> int {
    return WD ? wm * FM + ((i + wn * SSF) & (FM - 1)) : wm * FM + i;
  };
  // Tile order for the 8 XCDs: workgroup L = y * gridDim.x + x is placed on
  // XCD L % 8, and each XCD's L2 serves only its own workgroups.  When the
  // tile count divides by 8, XCD j takes the j-th eighth of a grouped order
  // (6 row tiles per group, rows fastest), so the 32 workgroups it runs at
  // once cover about 6 x 6 tiles and share their operand tiles in its L2
  // (a row of tiles that does not divide by 8 otherwise scatters them over
  // ~32 column tiles: measured 5% on the FFN gate/up prefill shape, same
  // bits).  Any other count keeps the launch order.
  int tile_x = blockIdx.x, tile_y = blockIdx.y;
  {
    const int NTX = gridDim.x, NTY = gridDim.y, T = NTX * NTY;
    if ((T & 7) == 0) {
      const int L = blockIdx.y * NTX + blockIdx.x;
      const int t = (L & 7) * (T >> 3) + (L >> 3);
      constexpr int GM = 6;
      const int group = t / (GM * NTX);
      const int first = group * GM;
      const int gm = min(NTY - first, GM);
      const int r = t - group * GM * NTX;
      tile_y = first + r % gm;
      tile_x = r / gm;
    }
  }
  const int m0 = tile_y * BMF * 16;
  const int nb0 = tile_x * BNF;
  // bytes of one packed column block: a fragment per k-block (bf16) or per
  // pair of k-blocks (fp8)
  const int kpairs = (a.kblocks + 1) / 2;
  const int64_t kfrag = (int64_t)(F8 ? kpairs : a.kblocks) * kFragBytes;

  const __amdgpu_buffer_rsrc_t xr =
      make_rsrc(static_cast<const __bf16*>(a.x) + (size_t)m0 * a.K, (int64_t)min(BMF * 16, a.M - m0) * a.K * 2);
  const int64_t wbytes = (int64_t)min(BNF, a.nblocks - nb0) * kfrag;
  const __amdgpu_buffer_rsrc_t wr0 = make_rsrc(static_cast<const uint8_t*>(a.wg) + nb0 * kfrag, wbytes);
  const __amdgpu_buffer_rsrc_t wr1 = make_rsrc(static_cast<const uint8_t*>(SW ? a.wu : a.wg) + nb0 * kfrag, wbytes);

  // x load q = wave + NW*j of a pair: rows 8*(q%2) .. +7 of row block q/2,
  // both k-blocks; lane l brings row lr = 8*(q%2) + l/8 of the block, chunk
  // (l%8) ^ (lr/2) of its eight 16-byte chunks (k within the pair).  NW is
  // even, so q%2 (hence lr and the chunk) is the same for every j and load j
  // sits 8*NW*j rows below load 0: one lane offset plus a uniform stride.
  static_assert(NW % 2 == 0, "x load rows");
  const int x_lr = 8 * (wave & 1) + (lane >> 3);
  const int x_c = (lane & 7) ^ (x_lr >> 1);
  const int xk = (x_c >> 2) * 32 + (x_c & 3) * 8;
  const uint32_t xoff0 = (uint32_t)((16 * (wave >> 1) + x_lr) * a.K + xk) * 2u;
  const uint32_t xstride = (uint32_t)(16 * NW) * (uint32_t)a.K;   // bytes between loads j and j+1
  auto issue_x = [&](uint8_t* base, int p) __attribute__((always_inline)) {
    const int k0 = p * 64;
    const uint32_t in = (uint32_t)((k0 + xk - a.K) >> 31);   // all ones while k < K
    // opaque to the optimiser: otherwise the XPW loop-invariant sums
    // xoff0 + j * xstride are hoisted out of the k loop into registers (a
    // spilled offset's reload would wait for every DMA load in flight)
    uint32_t xb = xoff0 + (uint32_t)k0 * 2u;
    asm volatile("" : "+v"(xb));
#pragma unroll
    for (int j = 0; j < XPW; ++j) {
      const uint32_t off = ((xb + xstride * (uint32_t)j) & in) | (kOutOfRange & ~in);
      __builtin_amdgcn_raw_ptr_buffer_load_lds(xr, (lds_ptr)(base + (wave + NW * j) * kFragBytes), 16, off, 0, 0,
                                               0);
    }
  };
  auto issue_w = [&](uint8_t* base, int kb) __attribute__((always_inline)) {
    const uint32_t win = (uint32_t)((kb - a.kblocks) >> 31);
#pragma unroll
    for (int i = 0; i < WPW; ++i) {
      const int f = wave + NW * i;
      const int m = f / BNF, ni = f % BNF;
      const uint32_t off = ((uint32_t)((ni * a.kblocks + kb) * kFragBytes + lane * 16) & win) | (kOutOfRange & ~win);
      __builtin_amdgcn_raw_ptr_buffer_load_lds(m == 0 ? wr0 : wr1, (lds_ptr)(base + f * kFragBytes), 16, off, 0, 0,
                                               0);
    }
  };
  // F8: the W' fragments of pair p (16 columns x 64 k each) into a pair slot
  constexpr int WP8 = WPW;   // fragments per wave per pair (the bf16 count per k-block)
  auto issue_w8 = [&](uint8_t* base, int p) __attribute__((always_inline)) {
    const uint32_t win = (uint32_t)((p - kpairs) >> 31);
#pragma unroll
    for (int i = 0; i < WP8; ++i) {
      const int f = wave + NW * i;
      const int m = f / BNF, ni = f % BNF;
      const uint32_t off = ((uint32_t)((ni * kpairs + p) * kFragBytes + lane * 16) & win) | (kOutOfRange & ~win);
      __builtin_amdgcn_raw_ptr_buffer_load_lds(m == 0 ? wr0 : wr1, (lds_ptr)(base + f * kFragBytes), 16, off, 0, 0,
                                               0);
    }
  };
  // LDS offset of this lane's x operand (row lrow, k-group lgrp) for k-block
  // u of the pair and row block rb
  auto x_at = [&](int u, int rb) __attribute__((always_inline)) -> int {
    const int c = (u * 4 + lgrp) ^ (lrow >> 1);
    return (2 * rb + (lrow >> 3)) * kFragBytes + (lrow & 7) * 128 + c * 16;
  };

  f32x4 acc[NMAT][FM][FN];
#pragma unroll
  for (int m = 0; m < NMAT; ++m)
#pragma unroll
    for (int i = 0; i < FM; ++i)
#pragma unroll
      for (int j = 0; j < FN; ++j) acc[m][i][j] = f32x4{0.f, 0.f, 0.f, 0.f};
  f32x4 gram[SSF];
#pragma unroll
  for (int i = 0; i < SSF; ++i) gram[i] = f32x4{0.f, 0.f, 0.f, 0.f};

  constexpr int NB = NMAT * FN;            // W' fragments per wave and k-block
  u32x4 av[FM], bv[NB];                    // one k-block's operands
  auto read_a = [&](const uint8_t* base, int u) __attribute__((always_inline)) {
#pragma unroll
    for (int i = 0; i < FM; ++i) av[i] = *reinterpret_cast<const u32x4*>(base + x_at(u, rfrag(i)));
  };
  auto read_b = [&](int j0, int j1, const uint8_t* base) __attribute__((always_inline)) {
#pragma unroll
    for (int j = j0; j < j1; ++j) {
      const int m = j / FN, jj = j % FN;
      bv[j] = *reinterpret_cast<const u32x4*>(base + (m * BNF + wn * FN + jj) * kFragBytes + lane * 16);
    }
  };
  // F8: this lane's 8 codes of k-block u of the pair for each B fragment,
  // then (after lgkmcnt(0)) decoded exactly to the bf16 operands
  uint32_t braw[F8 ? NB : 1][2];
  auto read_b8 = [&](const uint8_t* base, int u) __attribute__((always_inline)) {
#pragma unroll
    for (int j = 0; j < NB; ++j) {
      const int m = j / FN, jj = j % FN;
      const uint2 w = *reinterpret_cast<const uint2*>(base + (m * BNF + wn * FN + jj) * kFragBytes + lane * 16 + u * 8);
      braw[F8 ? j : 0][0] = w.x;
      braw[F8 ? j : 0][1] = w.y;
    }
  };
  auto decode_b8 = [&]() __attribute__((always_inline)) {
#pragma unroll
    for (int j = 0; j < NB; ++j) {
#pragma unroll
      for (int h = 0; h < 2; ++h) {
        bv[j][2 * h] = __builtin_bit_cast(uint32_t,
                                          __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(braw[F8 ? j : 0][h], 1.0f, false));
        bv[j][2 * h + 1] = __builtin_bit_cast(uint32_t,
                                              __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(braw[F8 ? j : 0][h], 1.0f, true));
      }
    }
  };
  auto mfma_cols = [&](int j0, int j1) __attribute__((always_inline)) {
#pragma unroll
    for (int j = j0; j < j1; ++j)
#pragma unroll
      for (int i = 0; i < FM; ++i) acc[j / FN][i][j % FN] = mfma_chunk<__bf16>(av[i], bv[j], acc[j / FN][i][j % FN]);
  };
  auto squares = [&]() __attribute__((always_inline)) {
#pragma unroll
    for (int i = 0; i < FM; ++i)
      if (i / SSF == wn) gram[i % SSF] = mfma_chunk<__bf16>(av[i], av[i], gram[i % SSF]);
  };
  auto lgkm0 = [&]() __attribute__((always_inline)) {
    __builtin_amdgcn_s_waitcnt((15) | (7 << 4) | (0 << 8) | (3 << 14));   // lgkmcnt(0)
  };

  if constexpr (F8) {
    // Ping-pong with pairs: the same slots as below, but W' rides with x --
    // pair p (k-blocks 2p, 2p+1) of both is loaded in slots 4p-5 (group A)
    // and 4p-4 (group B) into pair slot p % 2, after group B's last read of
    // pair p-2.  When the next k-block q opens a pair, that pair's loads are
    // the newest this wave has issued, so all must have landed (vmcnt 0);
    // when q is the second half, its pair landed before the previous slot.
    auto compute = [&]() __attribute__((always_inline)) {
      __builtin_amdgcn_sched_barrier(0);
      mfma_cols(0, NB);
      if constexpr (!EX) squares();
      __builtin_amdgcn_sched_barrier(0);
    };
    auto ready = [&](auto T4c) __attribute__((always_inline)) {
      constexpr int T4 = decltype(T4c)::value;
      if constexpr (T4 % 2 == 1) wait_vmcnt<0>();
      else wait_vmcnt<XPW + WP8>();
    };
    auto issue_pair = [&](int slot, int p) __attribute__((always_inline)) {
      issue_x(xslot(slot), p);
      issue_w8(wslot(slot), p);
    };
    auto stepA = [&](auto T4c, int s) __attribute__((always_inline)) {
      constexpr int T4 = decltype(T4c)::value;
      compute();
      ready(T4c);
      __builtin_amdgcn_s_barrier();
      __builtin_amdgcn_sched_barrier(0);
      read_a(xslot(((T4 + 1) % 4) / 2), (T4 + 1) % 2);
      read_b8(wslot(((T4 + 1) % 4) / 2), (T4 + 1) % 2);
      if constexpr (T4 % 2 == 1) issue_pair(((T4 + 3) / 2) % 2, (s + 3) / 2);
      lgkm0();
      decode_b8();
      __builtin_amdgcn_sched_barrier(0);
      __builtin_amdgcn_s_barrier();
    };
    auto stepB = [&](auto T4c, int s) __attribute__((always_inline)) {
      constexpr int T4 = decltype(T4c)::value;
      __builtin_amdgcn_sched_barrier(0);
      read_a(xslot(T4 / 2), T4 % 2);
      read_b8(wslot(T4 / 2), T4 % 2);
      if constexpr (T4 % 2 == 0) issue_pair(((T4 + 2) / 2) % 2, (s + 2) / 2);
      lgkm0();
      decode_b8();
      ready(T4c);
      __builtin_amdgcn_sched_barrier(0);
      __builtin_amdgcn_s_barrier();
      compute();
      __builtin_amdgcn_s_barrier();
    };
    if (wave & 4) {
      issue_pair(0, 0);
      __builtin_amdgcn_sched_barrier(0);
      wait_vmcnt<0>();
      __builtin_amdgcn_s_barrier();
      for (int s = 0; s < a.kblocks; s += 4) {
        stepB(std::integral_constant<int, 0>{}, s);
        stepB(std::integral_constant<int, 1>{}, s + 1);
        stepB(std::integral_constant<int, 2>{}, s + 2);
        stepB(std::integral_constant<int, 3>{}, s + 3);
      }
    } else {
      issue_pair(0, 0);
      issue_pair(1, 1);
      __builtin_amdgcn_sched_barrier(0);
      wait_vmcnt<XPW + WP8>();
      __builtin_amdgcn_s_barrier();
      read_a(xring0, 0);
      read_b8(wring0, 0);
      lgkm0();
      decode_b8();
      for (int s = 0; s < a.kblocks; s += 4) {
        stepA(std::integral_constant<int, 0>{}, s);
        stepA(std::integral_constant<int, 1>{}, s + 1);
        stepA(std::integral_constant<int, 2>{}, s + 2);
        stepA(std::integral_constant<int, 3>{}, s + 3);
      }
    }
  } else if constexpr (WD) {
    // W' straight to registers.  A packed fragment (16 columns x 32 k) is
    // 1 KiB of contiguous memory, the lane's 16 bytes its B operand, so each
    // wave loads its own fragments with whole-line buffer loads instead of
    // sharing them through an LDS ring; only x goes through LDS.  With waves
    // of 128 x 64 (WM = 2, WN = 4) a k-block of a 256 x 256 tile then moves
    // 16 KiB of DMA writes and 64 KiB of operand reads through the LDS
    // instead of 32 + 96 KiB, while each W' fragment is fetched twice, by
    // the waves of the two groups one slot apart.  (The same loads without
    // the ping-pong -- every wave alike, one barrier per pair of k-blocks,
    // a four-pair x ring -- gave the same bits 10-17% slower on every shape
    // measured: the two groups' alternation is worth more than its barriers.)
    //
    // The slots are the ping-pong's above; x keeps its ring and issue
    // order.  A wave's B operands of k-block s are loaded 3 slots before its
    // compute slot: group A issues B(s+2) in the memory slot after
    // computing s, group B issues B(s+1) in the memory slot before computing
    // s.  The compiler's own counter waits cover the register loads; the
    // explicit ones below cover x: when k-block q = s+1 opens a pair, the
    // pair's loads have been followed by exactly two k-blocks of this
    // wave's B loads in both groups' issue orders.
    u32x4 bq[NB];   // the next k-block's B operands in flight
    auto issue_wd = [&](int kb) __attribute__((always_inline)) {
      const uint32_t win = (uint32_t)((kb - a.kblocks) >> 31);
#pragma unroll
      for (int j = 0; j < NB; ++j) {
        const int m = j / FN, ni = wn * FN + j % FN;
        const uint32_t off = ((uint32_t)((ni * a.kblocks + kb) * kFragBytes + lane * 16) & win) | (kOutOfRange & ~win);
        bq[j] = __builtin_bit_cast(u32x4, __builtin_amdgcn_raw_buffer_load_b128(m == 0 ? wr0 : wr1, off, 0, 0));
      }
    };
    // with the rotated fragment order (rfrag) this wave's share of the
    // squares is its first SSF fragments
    auto squares_wd = [&]() __attribute__((always_inline)) {
#pragma unroll
      for (int t = 0; t < SSF; ++t) gram[t] = mfma_chunk<__bf16>(av[t], av[t], gram[t]);
    };
    auto compute = [&]() __attribute__((always_inline)) {
      __builtin_amdgcn_sched_barrier(0);
      mfma_cols(0, NB);
      if constexpr (!EX) squares_wd();
      __builtin_amdgcn_sched_barrier(0);
    };
    auto ready = [&](auto T4c) __attribute__((always_inline)) {
      constexpr int T4 = decltype(T4c)::value;
      if constexpr (T4 % 2 == 1) wait_vmcnt<2 * NB>();
    };
    auto stepA = [&](auto T4c, int s) __attribute__((always_inline)) {
      constexpr int T4 = decltype(T4c)::value;
      compute();
#pragma unroll
      for (int j = 0; j < NB; ++j) bv[j] = bq[j];
      ready(T4c);
      __builtin_amdgcn_s_barrier();
      __builtin_amdgcn_sched_barrier(0);
      read_a(xslot(((T4 + 1) % 4) / 2), (T4 + 1) % 2);
      if constexpr (T4 % 2 == 1) issue_x(xslot(((T4 + 3) / 2) % 2), (s + 3) / 2);
      issue_wd(s + 2);
      lgkm0();
      __builtin_amdgcn_sched_barrier(0);
      __builtin_amdgcn_s_barrier();
    };
    auto stepB = [&](auto T4c, int s) __attribute__((always_inline)) {
      constexpr int T4 = decltype(T4c)::value;
      __builtin_amdgcn_sched_barrier(0);
      read_a(xslot(T4 / 2), T4 % 2);
#pragma unroll
      for (int j = 0; j < NB; ++j) bv[j] = bq[j];
      if constexpr (T4 % 2 == 0) issue_x(xslot(((T4 + 2) / 2) % 2), (s + 2) / 2);
      issue_wd(s + 1);
      lgkm0();
      ready(T4c);
      __builtin_amdgcn_sched_barrier(0);
      __builtin_amdgcn_s_barrier();
      compute();
      __builtin_amdgcn_s_barrier();
    };
    if (wave & 4) {
      issue_x(xring0, 0);
      issue_wd(0);
      __builtin_amdgcn_sched_barrier(0);
      wait_vmcnt<NB>();
      __builtin_amdgcn_s_barrier();
      for (int s = 0; s < a.kblocks; s += 4) {
        stepB(std::integral_constant<int, 0>{}, s);
        stepB(std::integral_constant<int, 1>{}, s + 1);
        stepB(std::integral_constant<int, 2>{}, s + 2);
        stepB(std::integral_constant<int, 3>{}, s + 3);
      }
    } else {
      issue_x(xring0, 0);
      issue_x(xring1, 1);
      issue_wd(0);
#pragma unroll
      for (int j = 0; j < NB; ++j) bv[j] = bq[j];
      issue_wd(1);
      __builtin_amdgcn_sched_barrier(0);
      wait_vmcnt<XPW + 2 * NB>();
      __builtin_amdgcn_s_barrier();
      read_a(xring0, 0);
      for (int s = 0; s < a.kblocks; s += 4) {
        stepA(std::integral_constant<int, 0>{}, s);
        stepA(std::integral_constant<int, 1>{}, s + 1);
        stepA(std::integral_constant<int, 2>{}, s + 2);
        stepA(std::integral_constant<int, 3>{}, s + 3);
      }
    }
  } else {
    // Ping-pong.  k-block s: group A (waves 0-3) reads it in slot 2s-1 and
    // computes it in slot 2s; group B (waves 4-7) reads it in slot 2s and
    // computes it in slot 2s+1.  A memory slot also issues the wave's share
    // of the loads of a later k-block: group A W'(s+4) in slot 2s+1, group
    // B W'(s+3) in slot 2s -- each into the ring slot whose last reader
    // (group B) passed a barrier before -- and the x pair of k-blocks 2p,
    // 2p+1 in slots 4p-5 (A) and 4p-4 (B), after group B's last read of
    // pair p-2.  Unrolled by four k-blocks (W' slot s % 4, x slot s/2 % 2).
    auto compute = [&]() __attribute__((always_inline)) {
      __builtin_amdgcn_sched_barrier(0);
      mfma_cols(0, NB);
      if constexpr (!EX) squares();
      __builtin_amdgcn_sched_barrier(0);
    };
    // k-block q = s+1 is first read in slot 2s+1: every wave's loads of it
    // (W'(q), and x pair q/2 when q is even) must have landed by the barrier
    // that ends slot 2s.  In both groups' issue orders at most 2 WPW loads
    // follow them when q is even, 2 WPW + XPW when q is odd.
    auto ready = [&](auto T4c) __attribute__((always_inline)) {
      constexpr int T4 = decltype(T4c)::value;
      if constexpr (T4 % 2 == 1) wait_vmcnt<2 * WPW>();
      else wait_vmcnt<2 * WPW + XPW>();
    };
    auto stepA = [&](auto T4c, int s) __attribute__((always_inline)) {
      constexpr int T4 = decltype(T4c)::value;
      compute();
      ready(T4c);
      __builtin_amdgcn_s_barrier();
      __builtin_amdgcn_sched_barrier(0);
      read_a(xslot(((T4 + 1) % 4) / 2), (T4 + 1) % 2);
      read_b(0, NB, wslot((T4 + 1) % 4));
      if constexpr (T4 % 2 == 1) issue_x(xslot(((T4 + 3) / 2) % 2), (s + 3) / 2);
      issue_w(wslot(T4), s + 4);
      lgkm0();
      __builtin_amdgcn_sched_barrier(0);
      __builtin_amdgcn_s_barrier();
    };
    auto stepB = [&](auto T4c, int s) __attribute__((always_inline)) {
      constexpr int T4 = decltype(T4c)::value;
      __builtin_amdgcn_sched_barrier(0);
      read_a(xslot(T4 / 2), T4 % 2);
      read_b(0, NB, wslot(T4));
      if constexpr (T4 % 2 == 0) issue_x(xslot(((T4 + 2) / 2) % 2), (s + 2) / 2);
      issue_w(wslot((T4 + 3) % 4), s + 3);
      lgkm0();
      ready(T4c);
      __builtin_amdgcn_sched_barrier(0);
      __builtin_amdgcn_s_barrier();
      compute();
      __builtin_amdgcn_s_barrier();
    };
    // prologues: each group's loads of the slots before 0 in its own issue
    // order; then k-block 0 and x pair 0 have landed everywhere
    if (wave & 4) {
      issue_w(wring0, 0);
      issue_x(xring0, 0);
      issue_w(wring1, 1);
      issue_w(wring2, 2);
      __builtin_amdgcn_sched_barrier(0);
      wait_vmcnt<2 * WPW>();
      __builtin_amdgcn_s_barrier();
      for (int s = 0; s < a.kblocks; s += 4) {
        stepB(std::integral_constant<int, 0>{}, s);
        stepB(std::integral_constant<int, 1>{}, s + 1);
        stepB(std::integral_constant<int, 2>{}, s + 2);
        stepB(std::integral_constant<int, 3>{}, s + 3);
      }
    } else {
      issue_w(wring0, 0);
      issue_x(xring0, 0);
      issue_w(wring1, 1);
      issue_w(wring2, 2);
      issue_x(xring1, 1);
      issue_w(wring3, 3);
      __builtin_amdgcn_sched_barrier(0);
      wait_vmcnt<3 * WPW + XPW>();
      __builtin_amdgcn_s_barrier();
      read_a(xring0, 0);
      read_b(0, NB, wring0);
      for (int s = 0; s < a.kblocks; s += 4) {
        stepA(std::integral_constant<int, 0>{}, s);
        stepA(std::integral_constant<int, 1>{}, s + 1);
        stepA(std::integral_constant<int, 2>{}, s + 2);
        stepA(std::integral_constant<int, 3>{}, s + 3);
      }
    }
  }
  wait_vmcnt<0>();   // retire the zero-filled loads issued past the last k-block

#pragma unroll
  for (int i = 0; i < (EX ? 0 : SSF); ++i) {
    if ((lrow >> 2) == lgrp) {
      const int e = lrow & 3;
      const f32x4 gv = gram[i];
      ssbuf[(wm * FM + wn * SSF + i) * 16 + lrow] = e == 0 ? gv[0] : (e == 1 ? gv[1] : (e == 2 ? gv[2] : gv[3]));
    }
  }
  __syncthreads();
  // 1/RMS once per row of the tile, in place (EX: the pre-pass's)
  if (threadIdx.x < BMF * 16) {
    if constexpr (EX) {
      const int row = m0 + (int)threadIdx.x;
      ssbuf[threadIdx.x] = row < a.M ? a.rs[PAIR ? row >> 1 : row] : 0.f;
    } else {
      ssbuf[threadIdx.x] = inv_rms(ssbuf[threadIdx.x], (float)a.K, a.eps);
    }
  }
  __syncthreads();

  // F8: this lane's column scales (its columns, both matrices)
  float csc[NMAT][FN];
#pragma unroll
  for (int m = 0; m < NMAT; ++m)
#pragma unroll
    for (int j = 0; j < FN; ++j) {
      const int col = min((nb0 + wn * FN + j) * 16 + lrow, a.N - 1);
      csc[m][j] = F8 ? (m == 0 ? a.sg : a.su)[col] : 1.f;
    }
#pragma unroll
  for (int i = 0; i < FM; ++i) {
    const f32x4 inv4 = *reinterpret_cast<const f32x4*>(&ssbuf[rfrag(i) * 16 + 4 * lgrp]);
    // EX: the AdaLN bias values of this row fragment's outputs, all fetched
    // before its first store (the loads then overlap instead of each waiting
    // behind the previous store); where the index is outside the table or
    // the output outside the matrix a valid element is read and dropped, so
    // an index outside the table adds nothing
    float bias[NMAT][4][FN];
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      const int row = m0 + rfrag(i) * 16 + 4 * lgrp + r;
      const int trow = BIAS && row < a.M ? a.idx[PAIR ? row >> 1 : row] : -1;
      const bool tv = BIAS && (unsigned)trow < (unsigned)a.T;
      const size_t tb = (size_t)(tv ? trow : 0) * a.N;
#pragma unroll
      for (int j = 0; j < FN; ++j) {
        const int col = min((nb0 + wn * FN + j) * 16 + lrow, a.N - 1);
#pragma unroll
        for (int m = 0; m < NMAT; ++m) {
          float b = 0.f;
          if constexpr (BIAS) b = (m == 0 ? a.bg : a.bu)[tb + col];
          bias[m][r][j] = tv ? b : 0.f;
        }
      }
    }
#pragma unroll
    for (int r = 0; r < 4; r += (PAIR ? 2 : 1)) {
      const int rl = rfrag(i) * 16 + 4 * lgrp + r;   // row within the tile
      const int row = m0 + rl;
      const float inv = inv4[r];
      // PAIR: operand rows r and r+1 are one output row's two parts
      auto prod = [&](int m, int j) __attribute__((always_inline)) -> float {
        if constexpr (PAIR) return acc[m][i][j][r] + acc[m][i][j][r + 1];
        else return acc[m][i][j][r];
      };
      if constexpr (Q8) {
#pragma unroll
        for (int j = 0; j < FN; ++j) {
          const int nb = nb0 + wn * FN + j;
          const int col = nb * 16 + lrow;
          const float i0 = F8 ? inv * csc[0][j] : inv, i1 = F8 ? inv * csc[NMAT - 1][j] : inv;
          const float ga = BIAS ? fmaf(acc[0][i][j][r], i0, bias[0][r][j]) : acc[0][i][j][r] * i0;
          const float ua = BIAS ? fmaf(acc[NMAT - 1][i][j][r], i1, bias[NMAT - 1][r][j]) : acc[NMAT - 1][i][j][r] * i1;
          const float v = SW ? silu_times(ga, ua) : ga;
          store_q8(v, col < a.N, row < a.M, nb < a.nblocks, a.q + (size_t)row * a.N + col,
                   a.qs + (size_t)row * a.nblocks + nb);
        }
      } else if (row < a.M) {
        __bf16* yrow = static_cast<__bf16*>(a.y) + (size_t)(PAIR ? row >> 1 : row) * a.N;
#pragma unroll
        for (int j = 0; j < FN; ++j) {
          const int col = (nb0 + wn * FN + j) * 16 + lrow;
          if (col < a.N) {
            const float i0 = F8 ? inv * csc[0][j] : inv, i1 = F8 ? inv * csc[NMAT - 1][j] : inv;
            const float ga = prod(0, j) * i0 + bias[0][r][j];
            const float ua = prod(NMAT - 1, j) * i1 + bias[NMAT - 1][r][j];
            const float v = SW ? silu_times(ga, ua) : ga;
            Store<__bf16>::one(yrow + col, v);
          }
        }
      }
    }
  }
}

struct PrefillInstance {
  const void* fn;
  int fm, fn_, wm, wn, ns;
  bool sw, q8, ex, f8, pair;
  const char* name;
  bool wd;   // W' fragments straight to registers
};

#define FN_PREFILL(FM, FN_, WM, WN, SW, Q8, EX, F8, NAME)                                                   \
  PrefillInstance {                                                                                          \
    reinterpret_cast<const void*>(&prefill_kernel<FM, FN_, WM, WN, SW, Q8, EX, F8>), FM, FN_, WM, WN, 4, SW, Q8, \
        EX, F8, false, NAME                                                                                  \
  }
// the two-launch AdaLN SwiGLU on the split operand (bf16 output)
#define FN_PREFILL_PAIR(F8, NAME)                                                                            \
  PrefillInstance {                                                                                          \
    reinterpret_cast<const void*>(&prefill_kernel<4, 4, 4, 2, true, false, true, F8, true>), 4, 4, 4, 2, 4, true, \
        false, true, F8, true, NAME                                                                          \
  }

// W' fragments straight to registers, waves of 128 x 64: listed first, so
// plain projections on 256-row tiles take it when the grid has at least 256
// tiles (one per CU or more) and K is at least 4096.  Measured against the LDS-ring instance on
// the same inputs (the same bits), hot (one weight copy, cache-resident)
// and cold (copies rotated over 1.2 GiB): 4096 x 4096 -> 12288 hot 291-303
// against 296-308 us, cold 304-309 against 302-309 us; 8192 x 4096 -> 4096
// hot 196-200 against 201-209 us, cold 198-201 against 202 us.  Each wave's
// own W' loads are issued three slots ahead where the ring runs four
// k-blocks ahead, so HBM latency shows more: on shorter k loops and grids
// that leave CUs with a single tile it lost (2000 x 4104 -> 4100, 136
// tiles: cold 104 against 91 us, hot 90 against 83 us; 2000 x 1064 ->
// 4100: 34.4 against 33.2 us; 1000 x 4000 -> 1000: 81 against 76 us), on the SwiGLU pair 4096 x 4096 ->
// 2 x 11008 it won hot (547-564 against 551-569 us) and lost cold (565-567
// against 559-560 us), and on the AdaLN operand (no Gram blocks) it lost at
// every size (QKV 309 against 295 us); those keep the ring.
#define FN_PREFILL_WD(FN_, SW, Q8, EX, NAME)                                                                \
  PrefillInstance {                                                                                          \
    reinterpret_cast<const void*>(&prefill_kernel<8, FN_, 2, 4, SW, Q8, EX, false, false, true>), 8, FN_, 2, 4, 4, \
        SW, Q8, EX, false, false, NAME, true                                                                 \
  }

static const PrefillInstance kPrefill[] = {
    FN_PREFILL_WD(4, false, false, false, "prefill_bf16_256x256_w2x4_wd"),
    FN_PREFILL(4, 8, 4, 2, false, false, false, false, "prefill_bf16_256x256_w4x2_xl"),
    // narrow projections (one GPU's column share under tensor parallelism):
    // fewer than 128 tiles of 256 x 256 leave most CUs idle; 256 x 128 tiles
    // double the count (1536 columns x 4096 rows: 81.3 -> 57.9 us, same bits)
    FN_PREFILL(4, 4, 4, 2, false, false, false, false, "prefill_bf16_256x128_w4x2_xl"),
    FN_PREFILL(4, 4, 4, 2, true, false, false, false, "prefill_swiglu_bf16_256x128_w4x2_xl"),
    FN_PREFILL(4, 4, 4, 2, true, true, false, false, "prefill_swiglu_bf16_q8_256x128_w4x2_xl"),
    FN_PREFILL(4, 8, 4, 2, false, false, true, false, "prefill_premod_bf16_256x256_w4x2_xl"),
    FN_PREFILL_PAIR(false, "prefill_swiglu_premod_split_bf16_256x128_w4x2_xl"),
    FN_PREFILL(4, 4, 4, 2, true, true, true, false, "prefill_swiglu_bf16_q8_premod_256x128_w4x2_xl"),
    // fp8 (E4M3) weights with column scales
    FN_PREFILL(4, 8, 4, 2, false, false, false, true, "prefill_fp8_256x256_w4x2_xl"),
    FN_PREFILL(4, 4, 4, 2, false, false, false, true, "prefill_fp8_256x128_w4x2_xl"),   // narrow
    FN_PREFILL(4, 4, 4, 2, true, false, false, true, "prefill_swiglu_fp8_256x128_w4x2_xl"),
    FN_PREFILL(4, 4, 4, 2, true, true, false, true, "prefill_swiglu_fp8_q8_256x128_w4x2_xl"),
    FN_PREFILL(4, 8, 4, 2, false, false, true, true, "prefill_fp8_premod_256x256_w4x2_xl"),
    FN_PREFILL_PAIR(true, "prefill_swiglu_fp8_premod_split_256x128_w4x2_xl"),
    FN_PREFILL(4, 4, 4, 2, true, true, true, true, "prefill_swiglu_fp8_q8_premod_256x128_w4x2_xl"),
    // 129..256 rows of wide projections (at least 512 column blocks) with
    // bf16 weights: 128-row tiles, twice the workgroups of 256-row tiles with
    // half as many empty rows -- measured at K = 4096: QKV 64-66 -> 54-56 us,
    // gate/up pairs 83 -> 72-74 us (fp8 output 92-100 -> 75-79 us), AdaLN
    // QKV on the modulated operand 78-86 -> 59-60 us (fp8 output 94-105 ->
    // 81-86 us), the same bits; slower from 384 rows on
    FN_PREFILL(2, 4, 4, 2, false, false, false, false, "prefill_bf16_128x128_w4x2"),
    FN_PREFILL(2, 4, 4, 2, true, false, false, false, "prefill_swiglu_bf16_128x128_w4x2"),
    FN_PREFILL(2, 4, 4, 2, true, true, false, false, "prefill_swiglu_bf16_q8_128x128_w4x2"),
    FN_PREFILL(2, 4, 4, 2, false, false, true, false, "prefill_premod_bf16_128x128_w4x2"),
    FN_PREFILL(2, 4, 4, 2, true, true, true, false, "prefill_swiglu_bf16_q8_premod_128x128_w4x2"),
};

// The first instance with exactly these flags (q8 implies SwiGLU), mf
// 16-row fragments per tile and, when nf is given, nf 16-column fragments;
// the plain projection when none matches.
static const PrefillInstance& pick(bool sw, bool q8 = false, bool ex = false, bool f8 = false, int nf = 0,
                                   int mf = 16, bool wd_ok = false) {
  for (const PrefillInstance& d : kPrefill)
    if (d.sw == (sw || q8) && d.q8 == q8 && d.ex == ex && d.f8 == f8 && d.fm * d.wm == mf &&
        (nf == 0 || d.fn_ * d.wn == nf) && (wd_ok || !d.wd))
      return d;
  return kPrefill[1];
}

// The instance a plan names (plans carry the table's own name pointers).
static const PrefillInstance* by_name(const char* name) {
  for (const PrefillInstance& d : kPrefill)
    if (d.name == name) return &d;
  return nullptr;
}

FusedPlan plan_prefill(DType dt, int64_t M, int64_t K, int64_t N, bool swiglu, bool q8, bool ex, bool f8) {
  (void)dt;
  const bool plain = !swiglu && !q8 && !ex;
  const bool narrow = plain && ceil_div(N, 256) * ceil_div(M, 256) < 128;
  // 128-row tiles: bf16 weights, not the split AdaLN operand (its tiles
  // already hold 128 output rows)
  const bool split = ex && swiglu && !q8;
  const bool rows128 = !f8 && !split && M <= 256 && ceil_div(N, 16) >= 512;
  // W' straight to registers pays on long k loops over grids that fill the
  // chip at least once
  const int64_t tiles = ceil_div(M, 256) * ceil_div(N, swiglu ? 128 : 256);
  const PrefillInstance& d = rows128 ? pick(swiglu, q8, ex, false, 8, 8)
                                     : pick(swiglu, q8, ex, f8, narrow ? 8 : 0, 16, tiles >= 256 && K >= 4096);
  FusedPlan p{};
  p.kind = f8 ? 11 : (ex ? (q8 ? 10 : 8) : (q8 ? 5 : 1));
  p.mf = d.fm * d.wm;
  p.nf = d.fn_ * d.wn;
  p.waves = d.wm * d.wn;
  // a split operand has two rows per output row
  p.grid = dim3((unsigned)ceil_div(ceil_div(N, 16), p.nf), (unsigned)ceil_div(d.pair ? 2 * M : M, 16 * p.mf), 1);
  p.block = dim3(kWave * p.waves, 1, 1);
  p.name = d.name;
  return p;
}

hipError_t launch_prefill(DType dt, const FusedPlan& p, const void* x, const void* wg, const void* wu, void* y,
                          int M, int K, int N, float eps, hipStream_t stream, uint8_t* q, float* qs) {
  if (dt != DType::BF16 || (q != nullptr && wu == nullptr)) return hipErrorInvalidValue;
  const PrefillInstance* dp = by_name(p.name);
  if (dp == nullptr || dp->ex || dp->f8 || dp->sw != (wu != nullptr) || dp->q8 != (q != nullptr))
    return hipErrorInvalidValue;
  const PrefillInstance& d = *dp;
  PrefillArgs a{};
  a.q = q;
  a.qs = qs;
  a.sg = nullptr;
  a.su = nullptr;
  a.x = x;
  a.wg = wg;
  a.wu = wu;
  a.y = y;
  a.M = M;
  a.K = K;
  a.N = N;
  a.kblocks = (int)ceil_div(K, 32);
  a.nblocks = (int)ceil_div(N, 16);
  a.eps = eps;
  void* args[] = {&a};
  (void)p;
  return hipLaunchKernel(d.fn, p.grid, p.block, args, 0, stream);
}

hipError_t launch_prefill_fp8(const FusedPlan& p, const void* x, const void* wg, const float* sg, const void* wu,
                              const float* su, void* y, int M, int K, int N, float eps, hipStream_t stream, uint8_t* q,
                              float* qs) {
  if ((q != nullptr && wu == nullptr) || sg == nullptr || (wu != nullptr && su == nullptr)) return hipErrorInvalidValue;
  const PrefillInstance& d = pick(wu != nullptr, q != nullptr, false, true, p.nf, p.mf);
  PrefillArgs a{};
  a.x = x;
  a.wg = wg;
  a.wu = wu;
  a.y = y;
  a.M = M;
  a.K = K;
  a.N = N;
  a.kblocks = (int)ceil_div(K, 32);
  a.nblocks = (int)ceil_div(N, 16);
  a.eps = eps;
  a.q = q;
  a.qs = qs;
  a.sg = sg;
  a.su = su;
  void* args[] = {&a};
  return hipLaunchKernel(d.fn, p.grid, p.block, args, 0, stream);
}

hipError_t launch_prefill_premod(const FusedPlan& p, const void* u, const float* rs, const void* wg, const void* wu,
                                 void* y, int M, int K, int N, const AdalnArgs& ad, hipStream_t stream, uint8_t* q,
                                 float* qs, const float* sg, const float* su) {
  if (q != nullptr && wu == nullptr) return hipErrorInvalidValue;
  const bool f8 = sg != nullptr;
  if (f8 && wu != nullptr && su == nullptr) return hipErrorInvalidValue;
  const PrefillInstance* dp = by_name(p.name);
  if (dp == nullptr || !dp->ex || dp->f8 != f8 || dp->sw != (wu != nullptr) || dp->q8 != (q != nullptr))
    return hipErrorInvalidValue;
  const PrefillInstance& d = *dp;
  PrefillArgs a{};
  a.sg = sg;
  a.su = su;
  a.q = q;
  a.qs = qs;
  a.x = u;
  a.wg = wg;
  a.wu = wu;
  a.y = y;
  a.M = d.pair ? 2 * M : M;   // operand rows
  a.K = K;
  a.N = N;
  a.kblocks = (int)ceil_div(K, 32);
  a.nblocks = (int)ceil_div(N, 16);
  a.idx = ad.idx;
  a.bg = ad.bias_g;
  a.bu = ad.bias_u;
  a.T = ad.T;
  a.rs = rs;
  void* args[] = {&a};
  return hipLaunchKernel(d.fn, p.grid, p.block, args, 0, stream);
}

}  // namespace fn
