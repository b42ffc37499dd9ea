// Fused RMSNorm + projection (+ SwiGLU) with x shared through LDS: the bf16
// path for 17..64 rows, and every row count with fp8 (E4M3) weights.
//
// Past 16 rows x stops being small next to W': at 64 rows it is 128 KiB per
// 1024 k values, and a kernel that loads x into every wave's registers
// (decode.hip) pushes about as many x bytes through each CU's vector memory
// path as W' bytes, which is what bounds a skinny kernel on this chip (the
// per-CU request rate, not HBM).  With fp8 weights the weight stream halves
// and the same holds from a few rows on.  Here a workgroup owns NWV weight
// column blocks -- one (or NC) per wave, for SwiGLU with both the gate and
// the up stream -- and 16*MF rows (more rows tile over grid.y), and its waves
// walk the k range in lock step.  Per stage of U k-blocks the x rows are
// fetched once for the workgroup, split across its waves, straight into an
// LDS ring slot with direct global-to-LDS buffer loads; every wave then reads
// its MFMA operands with ds_read_b128.  Each wave streams its own weight
// fragments from HBM into registers with non-temporal buffer loads, NS-1
// stages ahead.
//
// x layout in a slot: each 1 KiB load carries 8 rows x 128 bytes (two
// k-blocks), so every request is a whole cache line; the 16-byte chunks of
// row r are stored permuted by r/2 so that the 16 lanes of each quarter
// wave read 16 distinct bank groups.
//
// fp8 weights: one 16-byte lane load carries the lane's 8 codes of two
// consecutive k-blocks, decoded in registers right before the MFMAs
// ([Fused-kernel memory hierarchy] "Fused 커널은 왜 3~4배 빠른가", section
// "트릭 2"); v_cvt_scalef32_pk_bf16_fp8 with scale 1 is exact (every E4M3
// value is a bf16 value), and the column scale s[n] joins 1/RMS in the
// epilogue ([FlashNorm digest] proposal 2, the deferred scale).
//
// Per k-block a wave runs MF projection MFMAs per weight stream, and per
// stage a few Gram MFMAs (x x^T of the fragments it loaded) whose diagonals
// are partial sums of squares ([FlashNorm digest] proposal 2: the sum of
// squares comes from the operands of the product, not from a second pass).
// The Gram diagonals meet in LDS for the epilogue: 1/RMS, SiLU(gate) * up
// for SwiGLU ([FlashInfer #5521] "Design" item 2), one RNE store.
//
// Edges: rows past M and k past K read as zero (buffer offsets out of
// range), and so do the stages past the last that fill the final round of
// the ring; column blocks past N read as zero and are not stored.
#include "fn_device.h"
#include "fn_launch.h"

namespace fn {

struct DecodeXArgs {
  const void* x;
  const void* wg;    // packed W' (gate for SwiGLU)
  const void* wu;    // packed W'_up, SwiGLU only
  void* y;
  int M, K, N;
  int kblocks;       // ceil(K / 32)
  int nblocks;       // ceil(N / 16)
  int stages;        // ceil(kblocks / U)
  float eps;
  const float* sg;   // fp8 weights: column scales of wg (else unused)
  const float* su;   // fp8 weights: column scales of wu
  uint8_t* q;        // fp8 output: E4M3 codes [M, N] (y unused)
  float* qs;         // fp8 output: scales [M, nblocks], one per 16-column row block
  const float* mod;  // AdaLN: modulation table g * (1 + scale) [T, K] (fp32)
  const int* idx;    // AdaLN: table row of each x row [M]
  const float* bg;   // AdaLN: bias rows shift @ W [T, N] (gate for SwiGLU)
  const float* bu;   // AdaLN: bias rows of W_up
  int T;             // AdaLN: table rows
  const float* rs;   // EX: 1/RMS of each row [M], from the AdaLN pre-pass
};


typedef __attribute__((address_space(3))) void* lds_ptr_x;

__device__ inline __amdgpu_buffer_rsrc_t make_rsrc_x(const void* base, int64_t bytes) {
  const int n = bytes > 0x7fffffff ? 0x7fffffff : (bytes < 0 ? 0 : (int)bytes);
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), 0, n, 0x00020000);
}

template <int N>
__device__ inline void wait_vmcnt_x() {
  static_assert(N >= 0 && N < 64, "vmcnt range");
  __builtin_amdgcn_s_waitcnt((N & 15) | (7 << 4) | (15 << 8) | ((N >> 4) << 14));
}

constexpr uint32_t kOutOfRangeX = 0x80000000u;

// MF: 16-row blocks of x.  NC: 16-column blocks per wave (for SwiGLU each
// with its gate and up stream).  NWV: waves, sharing the x fragments.  U:
// k-blocks per stage.  F8: E4M3 weights.  Q8: E4M3 output with row-block
// scales instead of a y in x's dtype.  AD: AdaLN, one row block -- the
// MFMA operand is x * mod[idx] (the modulation table row of each x row,
// loaded beside x in x's layout, two 16-byte loads per x chunk since the
// table is fp32) rounded to bf16 in registers, while the sum of squares
// stays on x; the epilogue adds the row's bias row.  EX: the projection
// half of the two-launch AdaLN form -- x is the operand the pre-pass already
// modulated, 1/RMS of each raw row comes from a.rs (no Gram blocks) and the
// epilogue adds the row's bias row.  LO: the operand in two bf16 parts,
// each multiplied with the same weight fragment, so the product is that of
// the unrounded operand (AD: split in registers, modulate8_split; EX: the
// pre-pass's [2M, K] operand, row 2m the rounded part of x row m and row
// 2m+1 the remainder, the remainder staged in LDS beside x).
// One workgroup's tile: column-block group bx, row-block group by (the
// kernel below takes them from the grid; the grouped launch from its call
// table).
template <int MF, int NC, int NWV, bool SW, int U, bool F8, bool Q8, bool AD = false, int NS = 4, bool EX = false,
          bool LO = false>
__device__ __forceinline__ void decode_x_tile(const DecodeXArgs& a, int bx, int by) {
  static_assert(NS >= 3 && NS <= 6, "LDS ring slots");
  constexpr int D = NS - 1;                // stages in flight
  constexpr int NMAT = SW ? 2 : 1;
  constexpr int NST = NMAT * NC;           // weight streams per wave
  constexpr int XF = U * MF;               // x loads (1 KiB each) per stage
  constexpr int XPW = (XF + NWV - 1) / NWV;   // x loads each wave issues per stage
  constexpr int WLD = F8 ? U / 2 : U;      // weight loads per stream per stage (fp8: one per k-block pair)
  // vector-memory ops per wave per stage (AdaLN: two loads of modulation
  // values per x load; a split operand: one load of its remainder)
  constexpr int LPW = WLD * NST + XPW + (AD ? 2 * XPW : 0) + (EX && LO ? XPW : 0);
  static_assert(!LO || (AD && MF == 1) || (EX && !Q8), "split operand: AdaLN, bf16 output");
  // Loads q >= XF (when NWV does not divide XF) fetch nothing and write
  // zeros into the slot's padding, so every wave issues the same count
  // (measured: skipping them instead is no faster).
  constexpr int XSL = XPW * NWV * kFragBytes;   // x part of a slot
  // AdaLN: per ring slot also the modulation values of its x chunks, the
  // first and the second four of each chunk in LDS arrays of their own: the
  // compiler then sees that the operand reads of a slot cannot alias the
  // global-to-LDS loads still landing in other slots (one shared array made
  // it drain every load in flight before them)
  constexpr int SLOT = XSL;
  constexpr int MSLOT = AD || LO ? XSL : 16;   // EX && LO: the remainder part of x
  static_assert(!AD || (MF == 1 && NC == 1 && !F8 && !Q8),
                "AdaLN: one row block, bf16 weights and output, one column block per wave");
  // Epilogue through LDS (one lane per row, 16-byte stores): fp8 output
  // always, bf16 output when each wave owns one column block.
  constexpr bool STAGE = Q8 || (NC == 1 && NWV <= NS && MF <= 4);   // one lane per row
  static_assert(!STAGE || (NC == 1 && NWV <= NS && 16 * MF * 16 * 4 <= SLOT), "staging fits a ring slot");
  static_assert(!EX || (!AD && NC == 1), "pre-modulated operand: one column block per wave");
  constexpr bool BIAS = AD || EX;
  static_assert(!BIAS || STAGE, "the AdaLN bias is added in the staged epilogue");
  static_assert(U % 2 == 0, "each x load moves two k-blocks of 8 rows");
  static_assert(D * LPW < 64, "vmcnt range");
  static_assert(NS * (SLOT + (AD ? 2 * MSLOT : (LO ? MSLOT : 0))) + NWV * XPW * 16 * 4 <= 160 * 1024, "LDS budget");

  __shared__ __attribute__((aligned(1024))) uint8_t ring0[SLOT];
  __shared__ __attribute__((aligned(1024))) uint8_t ring1[SLOT];
  __shared__ __attribute__((aligned(1024))) uint8_t ring2[SLOT];
  __shared__ __attribute__((aligned(1024))) uint8_t ring3[NS > 3 ? SLOT : 16];
  __shared__ __attribute__((aligned(1024))) uint8_t ring4[NS > 4 ? SLOT : 16];
  __shared__ __attribute__((aligned(1024))) uint8_t ring5[NS > 5 ? SLOT : 16];
  __shared__ __attribute__((aligned(1024))) uint8_t mring0[MSLOT];
  __shared__ __attribute__((aligned(1024))) uint8_t mring1[MSLOT];
  __shared__ __attribute__((aligned(1024))) uint8_t mring2[MSLOT];
  __shared__ __attribute__((aligned(1024))) uint8_t mring3[NS > 3 ? MSLOT : 16];
  __shared__ __attribute__((aligned(1024))) uint8_t mring4[NS > 4 ? MSLOT : 16];
  __shared__ __attribute__((aligned(1024))) uint8_t mring5[NS > 5 ? MSLOT : 16];
  __shared__ __attribute__((aligned(1024))) uint8_t hring0[MSLOT];
  __shared__ __attribute__((aligned(1024))) uint8_t hring1[MSLOT];
  __shared__ __attribute__((aligned(1024))) uint8_t hring2[MSLOT];
  __shared__ __attribute__((aligned(1024))) uint8_t hring3[NS > 3 ? MSLOT : 16];
  __shared__ __attribute__((aligned(1024))) uint8_t hring4[NS > 4 ? MSLOT : 16];
  __shared__ __attribute__((aligned(1024))) uint8_t hring5[NS > 5 ? MSLOT : 16];
  __shared__ float ssp[NWV][XPW][16];      // Gram diagonals
  __shared__ __attribute__((aligned(16))) float inv_s[MF * 16];   // 1/RMS per row
  auto slot_ptr = [&](int s) __attribute__((always_inline)) -> uint8_t* {
    return s == 0 ? ring0 : (s == 1 ? ring1 : (s == 2 ? ring2 : (s == 3 ? ring3 : (s == 4 ? ring4 : ring5))));
  };
  auto mod_ptr = [&](int s) __attribute__((always_inline)) -> uint8_t* {
    return s == 0 ? mring0 : (s == 1 ? mring1 : (s == 2 ? mring2 : (s == 3 ? mring3 : (s == 4 ? mring4 : mring5))));
  };
  auto modh_ptr = [&](int s) __attribute__((always_inline)) -> uint8_t* {
    return s == 0 ? hring0 : (s == 1 ? hring1 : (s == 2 ? hring2 : (s == 3 ? hring3 : (s == 4 ? hring4 : hring5))));
  };

  const int lane = threadIdx.x & (kWave - 1);
  const int w = __builtin_amdgcn_readfirstlane(threadIdx.x / kWave);
  const int lrow = lane & 15, lgrp = lane >> 4;
  const int nb0 = (bx * NWV + w) * NC;   // first column block of this wave
  const int m0 = by * MF * 16;           // first row of this workgroup
  // bytes of one packed column block: a fragment per k-block (bf16) or per
  // pair of k-blocks (fp8)
  const int64_t kfrag = (int64_t)(F8 ? (a.kblocks + 1) / 2 : a.kblocks) * kFragBytes;

  // fp8 weights: this lane's column scales, fetched now so the epilogue does
  // not wait for them
  float scol[NST];
#pragma unroll
  for (int c = 0; c < NST; ++c) {
    const int col = (nb0 + c % NC) * 16 + lrow;
    scol[c] = F8 && col < a.N ? (c < NC ? a.sg : a.su)[col] : 1.f;
  }

  // x rows of this workgroup; a split operand (EX && LO) has two rows per x
  // row, the rounded part at even rows and the remainder at odd ones: rows
  // past M then lie past both ranges
  constexpr int XRS = EX && LO ? 2 : 1;   // operand rows per x row
  const int nrows = min(MF * 16, a.M - m0);
  const __amdgpu_buffer_rsrc_t xr = make_rsrc_x(static_cast<const __bf16*>(a.x) + (size_t)XRS * m0 * a.K,
                                                (int64_t)(XRS * nrows - (XRS - 1)) * a.K * 2);
  __amdgpu_buffer_rsrc_t xlr = xr;
  if constexpr (EX && LO)
    xlr = make_rsrc_x(static_cast<const __bf16*>(a.x) + ((size_t)2 * m0 + 1) * a.K, (int64_t)(2 * nrows - 1) * a.K * 2);
  // AdaLN: this lane's bias values (its rows, its column), fetched now
  float bias[MF][4][NMAT];
#pragma unroll
  for (int i = 0; i < MF; ++i)
#pragma unroll
    for (int e = 0; e < 4; ++e)
#pragma unroll
      for (int m = 0; m < NMAT; ++m) bias[i][e][m] = 0.f;
  if constexpr (BIAS) {
    const int col = nb0 * 16 + lrow;
#pragma unroll
    for (int i = 0; i < MF; ++i)
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        const int row = m0 + 16 * i + 4 * lgrp + e;
        const int t = row < a.M ? a.idx[row] : -1;
        if ((unsigned)t < (unsigned)a.T && col < a.N) {
#pragma unroll
          for (int m = 0; m < NMAT; ++m) bias[i][e][m] = (m ? a.bu : a.bg)[(size_t)t * a.N + col];
        }
      }
  }
  // weight stream c = m * NC + j: matrix m, column block nb0 + j (reads zero past N)
  __amdgpu_buffer_rsrc_t wr[NST];
#pragma unroll
  for (int m = 0; m < NMAT; ++m)
#pragma unroll
    for (int j = 0; j < NC; ++j) {
      const int nb = nb0 + j;
      wr[m * NC + j] = make_rsrc_x(
          static_cast<const uint8_t*>(m ? a.wu : a.wg) + (int64_t)min(nb, a.nblocks - 1) * kfrag,
          nb < a.nblocks ? kfrag : 0);
    }

  // x loads: the stage's U*MF KiB of x arrive as XF one-KiB DMA loads, load
  // q = w + NWV*i issued by wave w.  Load q covers rows 8*(q%2) .. +7 of row
  // block (q/2) % MF and k-blocks 2*(q / (2*MF)) .. +1 of the stage; lane l
  // brings row l/8 of those, chunk (l%8) ^ (row/2) of its 8 16-byte chunks.
  // The same numbering, q = u*MF + i, names the MFMA fragment (k-block u,
  // row block i) whose Gram block wave q % NWV accumulates.
  uint32_t xoff[XPW];
  int xk[XPW];
  uint32_t soff[XPW], sok[XPW];   // AdaLN: the same chunk of the row's modulation-table row (fp32)
#pragma unroll
  for (int i = 0; i < XPW; ++i) {
    const int q = w + NWV * i;
    const int lr = 8 * (q & 1) + (lane >> 3);
    const int c = (lane & 7) ^ (lr >> 1);
    const int row = 16 * ((q >> 1) % MF) + lr;
    xk[i] = q < XF ? (2 * (q / (2 * MF)) + (c >> 2)) * 32 + (c & 3) * 8 : 1 << 30;   // past XF: never in range
    xoff[i] = (uint32_t)(row * XRS * a.K + (q < XF ? xk[i] : 0)) * 2u;
    if constexpr (AD) {
      const int t = (q < XF && m0 + row < a.M) ? a.idx[m0 + row] : -1;
      sok[i] = (unsigned)t < (unsigned)a.T ? 0xffffffffu : 0u;   // out-of-range index: modulation 0
      soff[i] = sok[i] ? (uint32_t)(t * a.K + xk[i]) * 4u : 0u;
    }
  }
  __amdgpu_buffer_rsrc_t sr = xr;
  if constexpr (AD) sr = make_rsrc_x(a.mod, (int64_t)a.T * a.K * 4);
  // LDS offset of this lane's MFMA operand (row lrow, chunk lgrp) for
  // k-block u, row block i of a stage
  auto x_at = [&](int u, int i) __attribute__((always_inline)) -> int {
    const int c = ((u & 1) * 4 + lgrp) ^ (lrow >> 1);
    return ((u >> 1) * 2 * MF + 2 * i + (lrow >> 3)) * kFragBytes + (lrow & 7) * 128 + c * 16;
  };
  // LDS offset of fragment q of a stage (for the Gram blocks); past XF, the
  // zero-filled padding
  auto frag_at = [&](int q) __attribute__((always_inline)) -> int {
    return q < XF ? x_at(q / MF, q % MF) : XF * kFragBytes + lane * 16;
  };
  // Issue stage st into slot base; stages past the last, and k past K, read
  // as zero without touching memory.
  auto issue_x = [&](int slot, int st) __attribute__((always_inline)) {
    uint8_t* base = slot_ptr(slot);
    const uint32_t live = (uint32_t)((st - a.stages) >> 31);
    const int k0 = st * U * 32;
#pragma unroll
    for (int i = 0; i < XPW; ++i) {
      const uint32_t in = live & (uint32_t)((k0 + xk[i] - a.K) >> 31);
      const uint32_t off = ((xoff[i] + (uint32_t)k0 * 2u) & in) | (kOutOfRangeX & ~in);
      __builtin_amdgcn_raw_ptr_buffer_load_lds(xr, (lds_ptr_x)(base + (w + NWV * i) * kFragBytes), 16, off, 0, 0,
                                               0);
    }
    if constexpr (AD) {
      // the chunk's 8 modulation values, 32 bytes: the first 16 into the
      // slot's first array, the second 16 into its second
#pragma unroll
      for (int i = 0; i < XPW; ++i) {
        const uint32_t in = sok[i] & live & (uint32_t)((k0 + xk[i] - a.K) >> 31);
        const uint32_t off = ((soff[i] + (uint32_t)k0 * 4u) & in) | (kOutOfRangeX & ~in);
        const uint32_t offh = ((soff[i] + (uint32_t)k0 * 4u + 16u) & in) | (kOutOfRangeX & ~in);
        __builtin_amdgcn_raw_ptr_buffer_load_lds(sr, (lds_ptr_x)(mod_ptr(slot) + (w + NWV * i) * kFragBytes), 16,
                                                 off, 0, 0, 0);
        __builtin_amdgcn_raw_ptr_buffer_load_lds(sr, (lds_ptr_x)(modh_ptr(slot) + (w + NWV * i) * kFragBytes), 16,
                                                 offh, 0, 0, 0);
      }
    }
    if constexpr (EX && LO) {
      // the remainder rows, at the same offsets from their own base
#pragma unroll
      for (int i = 0; i < XPW; ++i) {
        const uint32_t in = live & (uint32_t)((k0 + xk[i] - a.K) >> 31);
        const uint32_t off = ((xoff[i] + (uint32_t)k0 * 2u) & in) | (kOutOfRangeX & ~in);
        __builtin_amdgcn_raw_ptr_buffer_load_lds(xlr, (lds_ptr_x)(mod_ptr(slot) + (w + NWV * i) * kFragBytes), 16, off,
                                                 0, 0, 0);
      }
    }
  };
  u32x4 wv[NS][WLD][NST];
  auto issue_w = [&](int b, int st) __attribute__((always_inline)) {
    const uint32_t live = (uint32_t)((st - a.stages) >> 31);
#pragma unroll
    for (int u = 0; u < WLD; ++u) {
      const uint32_t off = (uint32_t)((st * WLD + u) * kFragBytes + lane * 16);
#pragma unroll
      for (int c = 0; c < NST; ++c)
        wv[b][u][c] = __builtin_bit_cast(
            u32x4, __builtin_amdgcn_raw_buffer_load_b128(wr[c], (off & live) | (kOutOfRangeX & ~live), 0, 2));
    }
  };

  f32x4 acc[NST][MF];
  f32x4 gram[XPW];
#pragma unroll
  for (int c = 0; c < NST; ++c)
#pragma unroll
    for (int i = 0; i < MF; ++i) acc[c][i] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
  for (int j = 0; j < XPW; ++j) gram[j] = f32x4{0.f, 0.f, 0.f, 0.f};

  // Stage st lives in ring slot s and W' buffer s.
  auto step = [&](int s, int st) __attribute__((always_inline)) {
    // Own loads of stage st are done once at most the D-1 younger stages
    // are in flight; the barrier extends that to the x loads of every wave
    // and retires every wave's reads of the slot refilled below.
    __builtin_amdgcn_sched_barrier(0);
    wait_vmcnt_x<(D - 1) * LPW>();
    uint8_t* base = slot_ptr(s);
    __builtin_amdgcn_s_barrier();
    __builtin_amdgcn_sched_barrier(0);
    u32x4 xv[U][MF];
    u32x4 xg[XPW];
#pragma unroll
    for (int u = 0; u < U; ++u)
#pragma unroll
      for (int i = 0; i < MF; ++i) xv[u][i] = *reinterpret_cast<const u32x4*>(base + x_at(u, i));
    if constexpr (!EX) {
#pragma unroll
      for (int j = 0; j < XPW; ++j) xg[j] = *reinterpret_cast<const u32x4*>(base + frag_at(w + NWV * j));
    }
    // AdaLN: the few operand chunks are modulated in registers, after the
    // next stage's loads are issued
    u32x4 svl[AD ? U : 1], svh[AD ? U : 1];
    if constexpr (AD) {
#pragma unroll
      for (int u = 0; u < U; ++u) {
        svl[u] = *reinterpret_cast<const u32x4*>(mod_ptr(s) + x_at(u, 0));
        svh[u] = *reinterpret_cast<const u32x4*>(modh_ptr(s) + x_at(u, 0));
      }
    }
    u32x4 xl[EX && LO ? U : 1][EX && LO ? MF : 1];   // the operand's remainder part
    if constexpr (EX && LO) {
#pragma unroll
      for (int u = 0; u < U; ++u)
#pragma unroll
        for (int i = 0; i < MF; ++i) xl[u][i] = *reinterpret_cast<const u32x4*>(mod_ptr(s) + x_at(u, i));
    }
    __builtin_amdgcn_sched_barrier(0);
    issue_w((s + D) % NS, st + D);
    issue_x((s + D) % NS, st + D);
    __builtin_amdgcn_sched_barrier(0);
    // B operands: the bf16 fragments as loaded, or the two halves of each
    // fp8 fragment decoded exactly to bf16 (every E4M3 value is a bf16 value)
    u32x4 bw[U][NST];
#pragma unroll
    for (int c = 0; c < NST; ++c) {
      if constexpr (F8) {
#pragma unroll
        for (int p = 0; p < U / 2; ++p) e4m3x16_to_bf16(wv[s][p][c], bw[2 * p][c], bw[2 * p + 1][c]);
      } else {
#pragma unroll
        for (int u = 0; u < U; ++u) bw[u][c] = wv[s][u][c];
      }
    }
#pragma unroll
    for (int u = 0; u < U; ++u)
#pragma unroll
      for (int i = 0; i < MF; ++i) {
        u32x4 xa = xv[u][i], xb = {0u, 0u, 0u, 0u};
        if constexpr (AD && LO) modulate8_split(xa, svl[AD ? u : 0], svh[AD ? u : 0], xa, xb);
        else if constexpr (AD) xa = modulate8(xa, svl[AD ? u : 0], svh[AD ? u : 0]);
        if constexpr (EX && LO) xb = xl[EX && LO ? u : 0][EX && LO ? i : 0];
#pragma unroll
        for (int c = 0; c < NST; ++c) {
          acc[c][i] = mfma_chunk<__bf16>(xa, bw[u][c], acc[c][i]);
          if constexpr (LO) acc[c][i] = mfma_chunk<__bf16>(xb, bw[u][c], acc[c][i]);
        }
      }
    if constexpr (!EX) {
#pragma unroll
      for (int j = 0; j < XPW; ++j) gram[j] = mfma_chunk<__bf16>(xg[j], xg[j], gram[j]);
    }
  };

  // the loop's load order: W', then x (and its modulation values)
#pragma unroll
  for (int p = 0; p < D; ++p) {
    issue_w(p, p);
    issue_x(p, p);
    __builtin_amdgcn_sched_barrier(0);
  }
  // whole rounds of the ring; stages past the last read as zero
  for (int st = 0; st < a.stages; st += NS) {
#pragma unroll
    for (int r = 0; r < NS; ++r) step(r, st + r);
  }
  wait_vmcnt_x<0>();

  // Accumulator element e of lane l is row 4*(l/16) + e, column l%16 of its
  // 16x16 tile, so the Gram diagonal sits in lanes with (l%16)/4 == l/16.
  if (!EX && (lrow >> 2) == lgrp) {
    const int e = lrow & 3;
#pragma unroll
    for (int j = 0; j < XPW; ++j)
      ssp[w][j][lrow] = e == 0 ? gram[j][0] : (e == 1 ? gram[j][1] : (e == 2 ? gram[j][2] : gram[j][3]));
  }
  __syncthreads();
  // 1/RMS once per row: thread t sums row t's Gram diagonals (accumulator j
  // of wave v holds fragment q = v + NWV*j, row block q % MF)
  if (threadIdx.x < MF * 16) {
    if constexpr (EX) {
      const int row = m0 + (int)threadIdx.x;
      inv_s[threadIdx.x] = row < a.M ? a.rs[row] : 0.f;
    } else {
      const int i = threadIdx.x / 16, rr = threadIdx.x % 16;
      float ss = 0.f;
#pragma unroll
      for (int v = 0; v < NWV; ++v)
#pragma unroll
        for (int j = 0; j < XPW; ++j)
          if (v + NWV * j < XF && (v + NWV * j) % MF == i) ss += ssp[v][j][rr];
      inv_s[threadIdx.x] = inv_rms(ss, (float)a.K, a.eps);
    }
  }
  __syncthreads();

#pragma unroll
  for (int i = 0; i < MF; ++i) {
    const f32x4 inv4 = *reinterpret_cast<const f32x4*>(&inv_s[16 * i + 4 * lgrp]);
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      const int rr = 4 * lgrp + e;
      const int row = m0 + 16 * i + rr;
      const float inv = inv4[e];
#pragma unroll
      for (int j = 0; j < NC; ++j) {
        const int col = (nb0 + j) * 16 + lrow;
        const bool col_ok = col < a.N;
        // fp8 weights: the column scale joins 1/RMS
        const float ig = F8 ? scol[j] * inv : inv;
        const float iu = F8 && SW ? scol[NC + j] * inv : inv;
        if constexpr (STAGE) {
          // staged in this wave's (now idle) ring slot as [row][16 columns]
          const float ga = BIAS ? fmaf(acc[j][i][e], ig, bias[i][e][0]) : acc[j][i][e] * ig;
          const float val = SW ? silu_times(ga, BIAS ? fmaf(acc[NC + j][i][e], iu, bias[i][e][NMAT - 1])
                                                   : acc[NC + j][i][e] * iu)
                               : ga;
          reinterpret_cast<float*>(slot_ptr(w))[(16 * i + rr) * 16 + lrow] = val;
        } else if (row < a.M && col_ok) {
          const float val = SW ? silu_times(acc[j][i][e] * ig, acc[NC + j][i][e] * iu) : acc[j][i][e] * ig;
          Store<__bf16>::one(static_cast<__bf16*>(a.y) + (size_t)row * a.N + col, val);
        }
      }
    }
  }
  if constexpr (STAGE) {
    // One lane per row: the lane reads its row's 16 values of the wave's
    // column block back and stores them with 16-byte stores when the block
    // is whole and aligned.  fp8 output: the block's largest magnitude (NaN
    // propagates), r = 448/amax and s = amax/448 (correctly rounded; 1 for
    // an all-zero block), codes RNE_E4M3(v * r).
    // the values cross lanes through LDS: order this wave's writes before its reads
    __builtin_amdgcn_fence(__ATOMIC_SEQ_CST, "wavefront");
    __builtin_amdgcn_wave_barrier();
    const float* tile = reinterpret_cast<const float*>(slot_ptr(w));
    const int nb = nb0;
    const int row = m0 + lane;
    if (lane < 16 * MF && row < a.M && nb < a.nblocks) {
      const int ncols = min(16, a.N - 16 * nb);
      float v[16];
#pragma unroll
      for (int k = 0; k < 4; ++k) {
        const f32x4 t4 = *reinterpret_cast<const f32x4*>(tile + lane * 16 + 4 * k);
#pragma unroll
        for (int c = 0; c < 4; ++c) v[4 * k + c] = t4[c];
      }
      if constexpr (Q8) {
        float m = 0.f;
#pragma unroll
        for (int c = 0; c < 16; ++c) m = nan_max(m, c < ncols ? fabsf(v[c]) : 0.f);
        const bool zero = m == 0.f;
        const float r = zero ? 1.f : __fdiv_rn(448.f, m);
        u32x4 packed = {0u, 0u, 0u, 0u};
#pragma unroll
        for (int c = 0; c < 16; ++c) packed[c / 4] |= e4m3_rne(v[c] * r) << (8 * (c % 4));
        uint8_t* dst = a.q + (size_t)row * a.N + 16 * nb;
        if (ncols == 16 && ((reinterpret_cast<uintptr_t>(dst) & 15) == 0)) {
          *reinterpret_cast<u32x4*>(dst) = packed;
        } else {
          for (int c = 0; c < ncols; ++c) dst[c] = (uint8_t)(packed[c / 4] >> (8 * (c % 4)));
        }
        a.qs[(size_t)row * a.nblocks + nb] = zero ? 1.f : __fdiv_rn(m, 448.f);
      } else {
        u32x4 p0, p1;
#pragma unroll
        for (int c = 0; c < 4; ++c) {
          p0[c] = pack_bf16x2(v[2 * c], v[2 * c + 1]);
          p1[c] = pack_bf16x2(v[8 + 2 * c], v[8 + 2 * c + 1]);
        }
        __bf16* dst = static_cast<__bf16*>(a.y) + (size_t)row * a.N + 16 * nb;
        if (ncols == 16 && ((reinterpret_cast<uintptr_t>(dst) & 15) == 0)) {
          reinterpret_cast<u32x4*>(dst)[0] = p0;
          reinterpret_cast<u32x4*>(dst)[1] = p1;
        } else {
          for (int c = 0; c < ncols; ++c) Store<__bf16>::one(dst + c, v[c]);
        }
      }
    }
  }
}

template <int MF, int NC, int NWV, bool SW, int U, bool F8, bool Q8, bool AD = false, int NS = 4, bool EX = false,
          bool LO = false>
__global__ __launch_bounds__(kWave * NWV) void decode_x_kernel(DecodeXArgs a) {
  decode_x_tile<MF, NC, NWV, SW, U, F8, Q8, AD, NS, EX, LO>(a, blockIdx.x, blockIdx.y);
}

struct DecodeXInstance {
  const void* fn;
  int mf, nc, nwv, u;
  bool sw, f8, q8;
  const char* name;
};

#define FN_DECODE_XI(MF, NC, NWV, SW, U, F8, Q8, NAME)                                                     \
  DecodeXInstance {                                                                                     \
    reinterpret_cast<const void*>(&decode_x_kernel<MF, NC, NWV, SW, U, F8, Q8>), MF, NC, NWV, U, SW, F8, Q8, NAME \
  }
#define FN_DECODE_X(MF, NC, NWV, SW, U, NAME) FN_DECODE_XI(MF, NC, NWV, SW, U, false, false, NAME)
#define FN_DECODE_X8(MF, NC, NWV, SW, U, NAME) FN_DECODE_XI(MF, NC, NWV, SW, U, true, false, NAME)

// Rows tile over grid.y in blocks of 16*MF; sg and su are the fp8 column
// scales (null for bf16 weights); q and qs the fp8 output (codes, row-block
// scales) of the Q8 instances.
inline hipError_t launch_decode_x_instance(const DecodeXInstance& d, const void* x, const void* wg, const void* wu,
                                           void* y, int M, int K, int N, float eps, hipStream_t stream,
                                           const float* sg = nullptr, const float* su = nullptr,
                                           uint8_t* q = nullptr, float* qs = nullptr,
                                           const AdalnArgs* ad = nullptr, const float* rs = nullptr) {
  DecodeXArgs a;
  a.rs = rs;
  a.sg = sg;
  a.su = su;
  a.q = q;
  a.qs = qs;
  a.mod = ad ? ad->mod : nullptr;
  a.idx = ad ? ad->idx : nullptr;
  a.bg = ad ? ad->bias_g : nullptr;
  a.bu = ad ? ad->bias_u : nullptr;
  a.T = ad ? ad->T : 0;
  a.x = x;
  a.wg = wg;
  a.wu = wu;
  a.y = y;
  a.M = M;
  a.K = K;
  a.N = N;
  a.kblocks = (int)ceil_div(K, 32);
  a.nblocks = (int)ceil_div(N, 16);
  a.stages = (int)ceil_div(a.kblocks, d.u);
  a.eps = eps;
  void* args[] = {&a};
  return hipLaunchKernel(d.fn, dim3((unsigned)ceil_div(a.nblocks, d.nc * d.nwv), (unsigned)ceil_div(M, 16 * d.mf)),
                         dim3(kWave * d.nwv), args, 0, stream);
}

// Measured on MI355X (cold weights): three one-column-block waves per
// workgroup, two-k-block stages.  A skinny kernel is bounded by each CU's
// vector-memory request rate, so what counts is the bytes each CU moves and
// that every CU moves some: three column blocks per workgroup give 256
// workgroups for 12288 columns (one per CU) and 230 for 11008, with each CU
// fetching x once per three weight streams.  Four waves (192 and 172
// workgroups) measured 10-15% slower, two waves slower still; wider waves,
// deeper stages and k-splits inside the workgroup did not help.
static const DecodeXInstance kDecodeX[] = {
    // plain projections: a 5-slot ring (four stages in flight) measured 7%
    // (32 rows) and 2% (64 rows) faster; the SwiGLU rungs are fastest with 4
    DecodeXInstance{reinterpret_cast<const void*>(&decode_x_kernel<2, 1, 3, false, 2, false, false, false, 5>), 2, 1, 3,
                    2, false, false, false, "decode_bf16_m32_xlds_w3_u2_s5"},
    DecodeXInstance{reinterpret_cast<const void*>(&decode_x_kernel<4, 1, 3, false, 2, false, false, false, 5>), 4, 1, 3,
                    2, false, false, false, "decode_bf16_m64_xlds_w3_u2_s5"},
    FN_DECODE_X(2, 1, 3, true, 2, "decode_swiglu_bf16_m32_xlds_w3_u2"),
    FN_DECODE_X(4, 1, 3, true, 2, "decode_swiglu_bf16_m64_xlds_w3_u2"),
    // 65..128 rows of wide projections (the row ladder sends them here
    // instead of the prefill kernel): one workgroup holds all 128 rows, so
    // each weight column block is requested once, not once per 64-row
    // block -- measured against the 64-row rung tiled over the rows: QKV
    // 39-43 -> 39-42 us, gate/up pairs 66-70 -> 51-53 us
    FN_DECODE_X(8, 1, 3, false, 2, "decode_bf16_m128_xlds_w3_u2"),
    FN_DECODE_X(8, 1, 3, true, 2, "decode_swiglu_bf16_m128_xlds_w3_u2"),
};

// fp8 weights, measured the same way: with half the weight bytes per stage
// the sixteen-row rungs want longer stages (eight k-blocks for a plain
// projection, four with SwiGLU), the 64-row SwiGLU rung four waves.
static const DecodeXInstance kDecodeF8[] = {
    FN_DECODE_X8(1, 1, 3, false, 8, "decode_fp8_m16_xlds_w3_u8"),
    FN_DECODE_X8(2, 1, 3, false, 4, "decode_fp8_m32_xlds_w3_u4"),
    FN_DECODE_X8(4, 1, 3, false, 2, "decode_fp8_m64_xlds_w3_u2"),
    FN_DECODE_X8(1, 1, 3, true, 4, "decode_swiglu_fp8_m16_xlds_w3_u4"),
    FN_DECODE_X8(2, 1, 3, true, 4, "decode_swiglu_fp8_m32_xlds_w3_u4"),
    FN_DECODE_X8(4, 1, 4, true, 2, "decode_swiglu_fp8_m64_xlds_w4_u2"),
    // gate/up pairs of 65..256 rows: 128-row blocks (44-76 -> 42-68 us
    // against the 64-row rung tiled over the rows); plain projections stay on
    // 64-row blocks, which measured faster there (29-32 against 36-38 us)
    FN_DECODE_X8(8, 1, 4, true, 2, "decode_swiglu_fp8_m128_xlds_w4_u2"),
};

// SwiGLU with fp8 output: the instances above with the row-block epilogue.
static const DecodeXInstance kDecodeQ8[] = {
    FN_DECODE_XI(1, 1, 3, true, 2, false, true, "decode_swiglu_bf16_q8_m16_xlds_w3_u2"),
    FN_DECODE_XI(2, 1, 3, true, 2, false, true, "decode_swiglu_bf16_q8_m32_xlds_w3_u2"),
    FN_DECODE_XI(4, 1, 3, true, 2, false, true, "decode_swiglu_bf16_q8_m64_xlds_w3_u2"),
    FN_DECODE_XI(1, 1, 3, true, 4, true, true, "decode_swiglu_fp8_q8_m16_xlds_w3_u4"),
    FN_DECODE_XI(2, 1, 3, true, 4, true, true, "decode_swiglu_fp8_q8_m32_xlds_w3_u4"),
    FN_DECODE_XI(4, 1, 4, true, 2, true, true, "decode_swiglu_fp8_q8_m64_xlds_w4_u2"),
};

template <size_t L>
static const DecodeXInstance* find_instance(const DecodeXInstance (&t)[L], int mf, bool sw) {
  for (const DecodeXInstance& d : t)
    if (d.mf == mf && d.sw == sw) return &d;
  return nullptr;
}

static FusedPlan plan_of(const DecodeXInstance* d, int kind, int64_t M, int64_t N) {
  FusedPlan p{};
  p.kind = kind;
  p.mf = d->mf;
  p.nf = d->nc * d->nwv;
  p.waves = d->nwv;
  p.grid = dim3((unsigned)ceil_div(ceil_div(N, 16), p.nf), (unsigned)ceil_div(M, 16 * d->mf), 1);
  p.block = dim3(kWave * p.waves, 1, 1);
  p.name = d->name;
  return p;
}

// bf16 row ladder rungs 32, 64 and 128 (the last for the wide projections
// the row ladder sends here past 64 rows; narrow ones repeat the 64-row rung
// over grid.y, which keeps three or four times the workgroups).
FusedPlan plan_decode_x(DType dt, int64_t M, int64_t K, int64_t N, bool swiglu) {
  (void)dt;
  (void)K;
  const bool wide = ceil_div(N, 16) >= 512;
  return plan_of(find_instance(kDecodeX, M <= 32 ? 2 : (M <= 64 || !wide ? 4 : 8), swiglu), 2, M, N);
}

hipError_t launch_decode_x(DType dt, const FusedPlan& p, const void* x, const void* wg, const void* wu, void* y,
                           int M, int K, int N, float eps, hipStream_t stream) {
  const DecodeXInstance* d = find_instance(kDecodeX, p.mf, wu != nullptr);
  if (dt != DType::BF16 || d == nullptr) return hipErrorInvalidValue;   // rows past 16 * mf: tiled over grid.y
  return launch_decode_x_instance(*d, x, wg, wu, y, M, K, N, eps, stream);
}

// fp8 row ladder 16 / 32 / 64 (128 for SwiGLU pairs past 64 rows); past the
// rung the row blocks repeat over grid.y (each streams the weights again: a
// decode design, used up to 256 rows of wide projections).
FusedPlan plan_fp8(int64_t M, int64_t K, int64_t N, bool swiglu) {
  (void)K;
  return plan_of(find_instance(kDecodeF8, M <= 16 ? 1 : (M <= 32 ? 2 : (M <= 64 || !swiglu ? 4 : 8)), swiglu), 3, M, N);
}

// AdaLN prologue (bf16), one launch, up to 16 rows: one modulation-table row
// per x row, the operands modulated in registers; five ring slots measured
// fastest.  SwiGLU takes the operand split in two parts (two MFMAs per
// weight fragment, idle matrix cores in this HBM-bound kernel): the SiLU
// times up of two rounded products has no margin left against the
// tolerance at large sizes, the single-rounding projection does.
#define FN_DECODE_XA5(NWV, SW, U, NAME)                                                                         \
  DecodeXInstance {                                                                                            \
    reinterpret_cast<const void*>(&decode_x_kernel<1, 1, NWV, SW, U, false, false, true, 5, false, SW>), 1, 1, NWV, \
        U, SW, false, false, NAME                                                                              \
  }
static const DecodeXInstance kDecodeAd[] = {
    FN_DECODE_XA5(3, false, 2, "decode_adaln_bf16_m16_xlds_w3_u2_s5"),
    FN_DECODE_XA5(3, true, 2, "decode_swiglu_adaln_split_bf16_m16_xlds_w3_u2_s5"),
};

FusedPlan plan_adaln(int64_t M, int64_t N, bool swiglu) {
  return plan_of(find_instance(kDecodeAd, 1, swiglu), 6, M, N);
}

hipError_t launch_adaln(const FusedPlan& p, const void* x, const void* wg, const void* wu, void* y, int M, int K,
                        int N, float eps, const AdalnArgs& ad, hipStream_t stream) {
  const DecodeXInstance* d = find_instance(kDecodeAd, p.mf, wu != nullptr);
  if (d == nullptr || M > 16) return hipErrorInvalidValue;
  return launch_decode_x_instance(*d, x, wg, wu, y, M, K, N, eps, stream, nullptr, nullptr, nullptr, nullptr, &ad);
}

// Two-launch AdaLN, 17..64 rows (and, the 64-row tiles repeated over
// grid.y, 65..128 rows of wide projections): the plain 32- and 64-row rungs
// on the operand the pre-pass modulated, 1/RMS from the pre-pass, bias rows
// added in the epilogue (no Gram blocks).
// SwiGLU: the split operand (LO).
#define FN_DECODE_XE(MF, SW, NS, NAME)                                                                          \
  DecodeXInstance {                                                                                            \
    reinterpret_cast<const void*>(&decode_x_kernel<MF, 1, 3, SW, 2, false, false, false, NS, true, SW>), MF, 1, \
        3, 2, SW, false, false, NAME                                                                           \
  }
static const DecodeXInstance kDecodeEx[] = {
    FN_DECODE_XE(2, false, 5, "decode_premod_bf16_m32_xlds_w3_u2_s5"),
    FN_DECODE_XE(4, false, 5, "decode_premod_bf16_m64_xlds_w3_u2_s5"),
    FN_DECODE_XE(2, true, 4, "decode_swiglu_premod_split_bf16_m32_xlds_w3_u2"),
    FN_DECODE_XE(4, true, 4, "decode_swiglu_premod_split_bf16_m64_xlds_w3_u2"),
};

// fp8 weights: the fp8 rungs above on the pre-modulated operand (every M;
// past 64 rows the 64-row tiles repeat over grid.y); SwiGLU on the split
// operand.
#define FN_DECODE_X8E(MF, NWV, SW, U, NAME)                                                                      \
  DecodeXInstance {                                                                                             \
    reinterpret_cast<const void*>(&decode_x_kernel<MF, 1, NWV, SW, U, true, false, false, 4, true, SW>), MF, 1, \
        NWV, U, SW, true, false, NAME                                                                           \
  }
static const DecodeXInstance kDecodeF8Ex[] = {
    FN_DECODE_X8E(1, 3, false, 8, "decode_fp8_premod_m16_xlds_w3_u8"),
    FN_DECODE_X8E(2, 3, false, 4, "decode_fp8_premod_m32_xlds_w3_u4"),
    FN_DECODE_X8E(4, 3, false, 2, "decode_fp8_premod_m64_xlds_w3_u2"),
    FN_DECODE_X8E(1, 3, true, 4, "decode_swiglu_fp8_premod_split_m16_xlds_w3_u4"),
    FN_DECODE_X8E(2, 3, true, 4, "decode_swiglu_fp8_premod_split_m32_xlds_w3_u4"),
    FN_DECODE_X8E(4, 4, true, 2, "decode_swiglu_fp8_premod_split_m64_xlds_w4_u2"),
};

// SwiGLU with fp8 output on the pre-modulated operand: the q8 rungs above
// (every M; past 64 rows the 64-row tiles repeat over grid.y).
#define FN_DECODE_XQE(MF, NWV, U, F8, NAME)                                                                     \
  DecodeXInstance {                                                                                            \
    reinterpret_cast<const void*>(&decode_x_kernel<MF, 1, NWV, true, U, F8, true, false, 4, true>), MF, 1,     \
        NWV, U, true, F8, true, NAME                                                                           \
  }
static const DecodeXInstance kDecodeQ8Ex[] = {
    FN_DECODE_XQE(1, 3, 2, false, "decode_swiglu_bf16_q8_premod_m16_xlds_w3_u2"),
    FN_DECODE_XQE(2, 3, 2, false, "decode_swiglu_bf16_q8_premod_m32_xlds_w3_u2"),
    FN_DECODE_XQE(4, 3, 2, false, "decode_swiglu_bf16_q8_premod_m64_xlds_w3_u2"),
    FN_DECODE_XQE(1, 3, 4, true, "decode_swiglu_fp8_q8_premod_m16_xlds_w3_u4"),
    FN_DECODE_XQE(2, 3, 4, true, "decode_swiglu_fp8_q8_premod_m32_xlds_w3_u4"),
    FN_DECODE_XQE(4, 4, 2, true, "decode_swiglu_fp8_q8_premod_m64_xlds_w4_u2"),
};

static const DecodeXInstance* find_q8_premod(bool f8, int mf) {
  for (const DecodeXInstance& d : kDecodeQ8Ex)
    if (d.f8 == f8 && d.mf == mf) return &d;
  return nullptr;
}

FusedPlan plan_decode_q8_premod(bool f8_weights, int64_t M, int64_t N) {
  return plan_of(find_q8_premod(f8_weights, M <= 16 ? 1 : (M <= 32 ? 2 : 4)), 10, M, N);
}

hipError_t launch_decode_q8_premod(bool f8_weights, const FusedPlan& p, const void* u, const float* rs,
                                   const void* wg, const float* sg, const void* wu, const float* su, uint8_t* q,
                                   float* qs, int M, int K, int N, const AdalnArgs& ad, hipStream_t stream) {
  const DecodeXInstance* d = find_q8_premod(f8_weights, p.mf);
  if (d == nullptr) return hipErrorInvalidValue;
  return launch_decode_x_instance(*d, u, wg, wu, nullptr, M, K, N, 0.f, stream, sg, su, q, qs, &ad, rs);
}

FusedPlan plan_decode_premod(int64_t M, int64_t N, bool swiglu, bool f8) {
  if (f8) return plan_of(find_instance(kDecodeF8Ex, M <= 16 ? 1 : (M <= 32 ? 2 : 4), swiglu), 9, M, N);
  return plan_of(find_instance(kDecodeEx, M <= 32 ? 2 : 4, swiglu), 9, M, N);
}

hipError_t launch_decode_premod(const FusedPlan& p, const void* u, const float* rs, const void* wg, const float* sg,
                                const void* wu, const float* su, void* y, int M, int K, int N, const AdalnArgs& ad,
                                hipStream_t stream) {
  const bool f8 = sg != nullptr;
  const DecodeXInstance* d =
      f8 ? find_instance(kDecodeF8Ex, p.mf, wu != nullptr) : find_instance(kDecodeEx, p.mf, wu != nullptr);
  if (d == nullptr) return hipErrorInvalidValue;
  return launch_decode_x_instance(*d, u, wg, wu, y, M, K, N, 0.f, stream, sg, su, nullptr, nullptr, &ad, rs);
}

// SwiGLU with fp8 output, every M (past 64 rows the 64-row tiles repeat over
// grid.y; the API sends more than 128 rows with bf16 weights, 256 with fp8,
// and more than 64 rows of narrow projections to the prefill kernel).
static const DecodeXInstance* find_q8(bool f8, int mf) {
  for (const DecodeXInstance& d : kDecodeQ8)
    if (d.f8 == f8 && d.mf == mf) return &d;
  return nullptr;
}

FusedPlan plan_decode_q8(bool f8_weights, int64_t M, int64_t N) {
  return plan_of(find_q8(f8_weights, M <= 16 ? 1 : (M <= 32 ? 2 : 4)), 4, M, N);
}

hipError_t launch_decode_q8(bool f8_weights, const FusedPlan& p, const void* x, const void* wg, const float* sg,
                            const void* wu, const float* su, uint8_t* q, float* qs, int M, int K, int N, float eps,
                            hipStream_t stream) {
  const DecodeXInstance* d = find_q8(f8_weights, p.mf);
  if (d == nullptr) return hipErrorInvalidValue;
  return launch_decode_x_instance(*d, x, wg, wu, nullptr, M, K, N, eps, stream, sg, su, q, qs);
}

hipError_t launch_fp8(const FusedPlan& p, const void* x, const void* wg, const float* sg, const void* wu,
                      const float* su, void* y, int M, int K, int N, float eps, hipStream_t stream) {
  const DecodeXInstance* d = find_instance(kDecodeF8, p.mf, wu != nullptr);
  if (d == nullptr) return hipErrorInvalidValue;
  return launch_decode_x_instance(*d, x, wg, wu, y, M, K, N, eps, stream, sg, su);
}

// Grouped launch of independent calls of up to 128 rows: every call's column
// blocks in workgroups of the tile above at its 64-row capacity (one per
// 64-row block of the call), one column block per wave and kGroupedXWaves
// waves sharing x through the LDS ring.  A single call cannot take that many
// column blocks per workgroup -- a QKV projection would fill fewer
// workgroups than there are CUs -- but the thousands of workgroups of a
// whole step can, and each x byte a workgroup fetches then serves
// kGroupedXWaves weight streams instead of three or four.  Measured on the
// 65 calls of a 32-layer step (speed-up over the calls launched one by one,
// bf16 / fp8 weights): 1.06 / 1.38 at 32 rows, 1.15 / 1.76 at 64, 1.13 /
// 1.66 at 128; eight waves per workgroup 1.13 / 1.68 at 64 rows, four 1.09 /
// 1.52.
struct GroupCallX {
  DecodeXArgs a;
  int first;       // index of the call's first workgroup in the launch
  int swiglu;
  int rowblocks;   // 64-row blocks of the call
};
// Workgroup r of a call with several row blocks: eight column groups side by
// side, then the next row block of the same eight.  Workgroup L of the launch
// runs on XCD L % 8, so the row blocks of one column group (r apart by
// multiples of 8) share an XCD and its L2, and start close together: the
// weights stream from HBM once.  Groups past the call's last (the padding of
// its last eight) read nothing and store nothing.

template <bool F8>
__global__ __launch_bounds__(kWave * kGroupedXWaves) void decode_x_grouped_kernel(
    const GroupCallX* __restrict__ calls, const uint16_t* __restrict__ item_call) {
  const int item = blockIdx.x;
  const int c = __builtin_amdgcn_readfirstlane((int)item_call[item]);
  const GroupCallX& g = calls[c];
  const int r = item - g.first;
  const int oct = r / (8 * g.rowblocks), w8 = r - oct * 8 * g.rowblocks;
  const int by = w8 >> 3, bx = oct * 8 + (w8 & 7);
  if (g.swiglu)
    decode_x_tile<4, kGroupedXCols, kGroupedXWaves, true, kGroupedXStage, F8, false>(g.a, bx, by);
  else
    decode_x_tile<4, kGroupedXCols, kGroupedXWaves, false, kGroupedXStage, F8, false>(g.a, bx, by);
}

hipError_t launch_decode_x_grouped(const void* calls, const void* item_call, int items, bool fp8,
                                   hipStream_t stream) {
  const GroupCallX* c = static_cast<const GroupCallX*>(calls);
  const uint16_t* ic = static_cast<const uint16_t*>(item_call);
  void* args[] = {&c, &ic};
  const void* k = fp8 ? reinterpret_cast<const void*>(&decode_x_grouped_kernel<true>)
                      : reinterpret_cast<const void*>(&decode_x_grouped_kernel<false>);
  return hipLaunchKernel(k, dim3((unsigned)items), dim3(kWave * kGroupedXWaves), args, 0, stream);
}

size_t grouped_x_call_bytes() { return sizeof(GroupCallX); }

void grouped_x_call_fill(void* dst, const void* x, const void* wg, const void* wu, const float* sg, const float* su,
                         void* y, int M, int K, int N, float eps, int first) {
  GroupCallX g{};
  g.a.x = x;
  g.a.wg = wg;
  g.a.wu = wu;
  g.a.y = y;
  g.a.M = M;
  g.a.K = K;
  g.a.N = N;
  g.a.kblocks = (int)ceil_div(K, 32);
  g.a.nblocks = (int)ceil_div(N, 16);
  g.a.stages = (int)ceil_div(g.a.kblocks, kGroupedXStage);
  g.a.eps = eps;
  g.a.sg = sg;
  g.a.su = su;
  g.first = first;
  g.swiglu = wu != nullptr;
  g.rowblocks = (int)ceil_div(M, 64);
  *static_cast<GroupCallX*>(dst) = g;
}
}  // namespace fn
