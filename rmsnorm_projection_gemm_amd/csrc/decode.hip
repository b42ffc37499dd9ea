// Fused RMSNorm + projection (+ SwiGLU) for small row counts (decode).
//
// One launch computes, per output tile, the contraction x * W' and the
// per-row sum of squares of x from the very same x registers, then applies
// the deferred 1/RMS scale (and SiLU * up) to the fp32 accumulators and
// stores the tile once ([FlashNorm digest] proposals 1-2; [FlashInfer #5521]
// "Design" item 2, register-level SwiGLU).  Nothing intermediate is written
// to memory and there is no second stream to join, so the stale-buffer race
// the FlashNorm talk describes (a post-scale step reading a product another
// stream had not finished) cannot occur.
//
// Decomposition: a workgroup owns WN*NF 16-column blocks of W' (for SwiGLU
// the same columns of W'_gate and W'_up) and MF 16-row blocks of x.  Its
// WN*WK waves form WN column groups of NF blocks each and WK k-splits; every
// wave streams its share of W' from HBM exactly once, with non-temporal
// loads so W' does not evict x from the caches, and loads the x fragments it
// needs into its own registers.  That suits up to 16 rows, where x is a
// small fraction of the bytes each CU moves; bf16 with more rows shares x
// through LDS instead (decode_x.hip).  W' uses the packed fragment layout:
// each lane's weight operand is one 16-byte load and a wave reads 1 KiB of
// contiguous memory per fragment.
//
// In this regime the matrix cores idle while W' streams in, and every VALU
// instruction costs four cycles per wave on the critical path.  So the sum of
// squares is taken on the matrix cores too: an MFMA with the x fragment as
// both operands yields the 16x16 Gram block x x^T whose diagonal holds each
// row's partial sum of squares (fp32 products of bf16 values are exact).
// Rows past M and columns past N are clamped to the last valid one instead
// of masked: their results are never stored, and rows do not mix in the
// product (nor on the Gram diagonal), so the clamped lanes cannot disturb
// valid outputs.  Only the ragged last k-block (K % KB != 0) is masked.
#include <type_traits>

#include "fn_device.h"
#include "fn_launch.h"

namespace fn {

struct DecodeArgs {
  const void* x;
  const u32x4* wg;   // packed W' (gate for SwiGLU)
  const u32x4* wu;   // packed W'_up, SwiGLU only
  void* y;
  int M, K, N;
  int kblocks;       // ceil(K / KB)
  int nblocks;       // ceil(N / 16)
  float eps;
};

// One workgroup's tile: column-block group bx, row-block group by.
template <typename T, int MF, int NF, bool SW, int WN, int WK, int U>
__device__ __forceinline__ void decode_tile(const DecodeArgs& a, int bx, int by) {
  constexpr int V = Geo<T>::V;
  constexpr int KB = Geo<T>::KB;
  constexpr int NMAT = SW ? 2 : 1;
  const int lane = threadIdx.x & (kWave - 1);
  // wave-uniform: loop bounds and weight offsets stay in scalar registers
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x / kWave);
  const int wn = wave % WN;         // column group of this wave
  const int wk = wave / WN;         // k split of this wave
  const int lrow = lane & 15;       // operand row (x) / column (W') of this lane
  const int lgrp = lane >> 4;       // k group of this lane
  const int nb0 = (bx * WN + wn) * NF;
  const int m0 = by * 16 * MF;
  const int kb_begin = (int)((int64_t)a.kblocks * wk / WK);
  const int kb_end = (int)((int64_t)a.kblocks * (wk + 1) / WK);
  const int kb_full = a.K / KB;     // k-blocks with no ragged tail

  const T* xrow[MF];
#pragma unroll
  for (int mf = 0; mf < MF; ++mf) {
    const int row = min(m0 + 16 * mf + lrow, a.M - 1);
    xrow[mf] = static_cast<const T*>(a.x) + (size_t)row * a.K + lgrp * V;
  }
  const u32x4* wp[NMAT][NF];
#pragma unroll
  for (int nf = 0; nf < NF; ++nf) {
    const size_t base = (size_t)min(nb0 + nf, a.nblocks - 1) * a.kblocks * kWave + lane;
    wp[0][nf] = a.wg + base;
    if (SW) wp[NMAT - 1][nf] = a.wu + base;
  }

  f32x4 acc[NMAT][MF][NF];
  f32x4 gram[MF];
#pragma unroll
  for (int mf = 0; mf < MF; ++mf) {
    gram[mf] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int m = 0; m < NMAT; ++m)
#pragma unroll
      for (int nf = 0; nf < NF; ++nf) acc[m][mf][nf] = f32x4{0.f, 0.f, 0.f, 0.f};
  }
  // fp32 operands: two-level sums.  The MFMAs accumulate a run of k-blocks
  // into acc / gram, which are then added into the totals and cleared, so
  // each fp32 sum has about sqrt(K) terms per level instead of K in one
  // (the rounding error of a K-term fp32 sum grows with its length: a
  // single level misses 1e-5 relative at K = 2^20).  bf16 keeps one level:
  // its operands' own rounding dominates.
  constexpr bool TWO = std::is_same<T, float>::value;
  f32x4 tacc[TWO ? NMAT : 1][TWO ? MF : 1][TWO ? NF : 1];
  f32x4 tgram[TWO ? MF : 1];
#pragma unroll
  for (int mf = 0; mf < (TWO ? MF : 1); ++mf) {
    tgram[mf] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int m = 0; m < (TWO ? NMAT : 1); ++m)
#pragma unroll
      for (int nf = 0; nf < (TWO ? NF : 1); ++nf) tacc[m][mf][nf] = f32x4{0.f, 0.f, 0.f, 0.f};
  }
  auto fold = [&]() {
    if constexpr (TWO) {
#pragma unroll
      for (int mf = 0; mf < MF; ++mf) {
        tgram[mf] += gram[mf];
        gram[mf] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int m = 0; m < NMAT; ++m)
#pragma unroll
          for (int nf = 0; nf < NF; ++nf) {
            tacc[m][mf][nf] += acc[m][mf][nf];
            acc[m][mf][nf] = f32x4{0.f, 0.f, 0.f, 0.f};
          }
      }
    }
  };
  // k-blocks per first-level run: 64 (1024 k values of fp32)
  constexpr int FOLD_ITERS = 32 / U > 0 ? 32 / U : 1;   // main-loop iterations of 2 U k-blocks

  // One stage = U k-blocks of operands in registers.
  struct Stage {
    u32x4 x[U][MF];
    u32x4 w[U][NMAT][NF];
  };
  auto load = [&](Stage& s, int kb) {
#pragma unroll
    for (int u = 0; u < U; ++u) {
#pragma unroll
      for (int mf = 0; mf < MF; ++mf)
        s.x[u][mf] = *reinterpret_cast<const u32x4*>(xrow[mf] + (size_t)(kb + u) * KB);
#pragma unroll
      for (int m = 0; m < NMAT; ++m)
#pragma unroll
        for (int nf = 0; nf < NF; ++nf)
          s.w[u][m][nf] = __builtin_nontemporal_load(wp[m][nf] + (size_t)(kb + u) * kWave);
    }
  };
  auto load1 = [&](Stage& s, int kb) {
#pragma unroll
    for (int mf = 0; mf < MF; ++mf) s.x[0][mf] = *reinterpret_cast<const u32x4*>(xrow[mf] + (size_t)kb * KB);
#pragma unroll
    for (int m = 0; m < NMAT; ++m)
#pragma unroll
      for (int nf = 0; nf < NF; ++nf) s.w[0][m][nf] = __builtin_nontemporal_load(wp[m][nf] + (size_t)kb * kWave);
  };
  auto step = [&](const u32x4 (&xv)[MF], const u32x4 (&wv)[NMAT][NF]) {
#pragma unroll
    for (int mf = 0; mf < MF; ++mf) {
      gram[mf] = mfma_chunk<T>(xv[mf], xv[mf], gram[mf]);
#pragma unroll
      for (int m = 0; m < NMAT; ++m)
#pragma unroll
        for (int nf = 0; nf < NF; ++nf) acc[m][mf][nf] = mfma_chunk<T>(xv[mf], wv[m][nf], acc[m][mf][nf]);
    }
  };
  auto compute = [&](const Stage& s) {
#pragma unroll
    for (int u = 0; u < U; ++u) step(s.x[u], s.w[u]);
  };

  // Double-buffered stream: the loads of the next stage are in flight while
  // the current one is consumed.  The scheduling barriers keep the compiler
  // from sinking loads below the matrix instructions that do not need them.
  auto stream_range = [&](int lo, int hi) {
    int kb = lo;
    if (kb + 2 * U <= hi) {
      Stage s0, s1;
      load(s0, kb);
      int it = 0;
      for (; kb + 4 * U <= hi; kb += 2 * U) {
        load(s1, kb + U);
        __builtin_amdgcn_sched_barrier(0);
        compute(s0);
        __builtin_amdgcn_sched_barrier(0);
        load(s0, kb + 2 * U);
        __builtin_amdgcn_sched_barrier(0);
        compute(s1);
        __builtin_amdgcn_sched_barrier(0);
        if constexpr (TWO) {
          if (++it == FOLD_ITERS) {
            fold();
            it = 0;
          }
        }
      }
      load(s1, kb + U);
      __builtin_amdgcn_sched_barrier(0);
      compute(s0);
      compute(s1);
      kb += 2 * U;
    }
    for (; kb < hi; ++kb) {
      Stage s;
      load1(s, kb);
      step(s.x[0], s.w[0]);
    }
  };

  const int kb_main_end = min(kb_end, kb_full);
  stream_range(kb_begin, kb_main_end);
  // The ragged last k-block (K % KB != 0): x is masked past K.
  for (int kb = max(kb_main_end, kb_begin); kb < kb_end; ++kb) {
    u32x4 xv[MF];
    u32x4 wv[NMAT][NF];
    const bool kin = kb * KB + lgrp * V < a.K;
#pragma unroll
    for (int mf = 0; mf < MF; ++mf)
      xv[mf] = kin ? *reinterpret_cast<const u32x4*>(xrow[mf] + (size_t)kb * KB) : u32x4{0u, 0u, 0u, 0u};
#pragma unroll
    for (int m = 0; m < NMAT; ++m)
#pragma unroll
      for (int nf = 0; nf < NF; ++nf) wv[m][nf] = __builtin_nontemporal_load(wp[m][nf] + (size_t)kb * kWave);
    step(xv, wv);
  }
  if constexpr (TWO) {
    // the totals become the sums the epilogue reads
    fold();
#pragma unroll
    for (int mf = 0; mf < MF; ++mf) {
      gram[mf] = tgram[mf];
#pragma unroll
      for (int m = 0; m < NMAT; ++m)
#pragma unroll
        for (int nf = 0; nf < NF; ++nf) acc[m][mf][nf] = tacc[m][mf][nf];
    }
  }

  // Partials meet in LDS.  Accumulator element r of lane l is row
  // 4*(l/16) + r, column l%16 of its 16x16 tile; the Gram diagonal (row ==
  // column) therefore sits in lanes whose l%16 / 4 == l/16, element l%4.
  // Without a k-split (WK == 1) the accumulators stay in registers and the
  // diagonal lanes turn their sums of squares into 1/RMS right away, one
  // per row.
  constexpr bool ONE = WK == 1;
  const float kf = (float)a.K;
  __shared__ float red_acc[ONE ? 1 : WK][WN][NMAT][MF][NF][4][kWave];
  __shared__ float red_ss[WK][WN][MF][16];
  if constexpr (!ONE) {
#pragma unroll
    for (int m = 0; m < NMAT; ++m)
#pragma unroll
      for (int mf = 0; mf < MF; ++mf)
#pragma unroll
        for (int nf = 0; nf < NF; ++nf)
#pragma unroll
          for (int r = 0; r < 4; ++r) red_acc[wk][wn][m][mf][nf][r][lane] = acc[m][mf][nf][r];
  }
  if ((lrow >> 2) == lgrp) {
    const int r = lrow & 3;
#pragma unroll
    for (int mf = 0; mf < MF; ++mf) {
      const f32x4 gv = gram[mf];
      const float g = r == 0 ? gv[0] : (r == 1 ? gv[1] : (r == 2 ? gv[2] : gv[3]));
      red_ss[wk][wn][mf][lrow] = ONE ? inv_rms(g, kf, a.eps) : g;
    }
  }
  __syncthreads();

  if constexpr (ONE) {
#pragma unroll
    for (int mf = 0; mf < MF; ++mf)
#pragma unroll
      for (int nf = 0; nf < NF; ++nf) {
        const int col = (nb0 + nf) * 16 + lrow;
#pragma unroll
        for (int r = 0; r < 4; ++r) {
          const int i = 4 * lgrp + r;
          const int row = m0 + 16 * mf + i;
          if (row < a.M && col < a.N) {
            const float inv = red_ss[0][wn][mf][i];
            const float p0 = acc[0][mf][nf][r];
            const float v = SW ? silu_times(p0 * inv, acc[NMAT - 1][mf][nf][r] * inv) : p0 * inv;
            Store<T>::one(static_cast<T*>(a.y) + (size_t)row * a.N + col, v);
          }
        }
      }
    return;
  }
  // Epilogue: the WK waves of column group wn finish its tiles wk, wk + WK, ...
  for (int t = wk; t < MF * NF; t += WK) {
    const int mf = t / NF, nf = t % NF;
    const int col = (nb0 + nf) * 16 + lrow;
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      const int i = 4 * lgrp + r;
      const int row = m0 + 16 * mf + i;
      float sum_sq = 0.f, p0 = 0.f, p1 = 0.f;
#pragma unroll
      for (int w = 0; w < WK; ++w) {
        sum_sq += red_ss[w][wn][mf][i];
        p0 += red_acc[w][wn][0][mf][nf][r][lane];
        if (SW) p1 += red_acc[w][wn][NMAT - 1][mf][nf][r][lane];
      }
      if (row < a.M && col < a.N) {
        const float inv = inv_rms(sum_sq, kf, a.eps);
        const float v = SW ? silu_times(p0 * inv, p1 * inv) : p0 * inv;
        Store<T>::one(static_cast<T*>(a.y) + (size_t)row * a.N + col, v);
      }
    }
  }
}

template <typename T, int MF, int NF, bool SW, int WN, int WK, int U>
__global__ __launch_bounds__(kWave * WN * WK) void decode_kernel(DecodeArgs a) {
  decode_tile<T, MF, NF, SW, WN, WK, U>(a, blockIdx.x, blockIdx.y);
}

// Grouped launch: the column blocks of several independent calls (bf16, at
// most 16 rows each) as the workgroups of one launch, in call order.  The
// hardware starts each workgroup as a CU frees up, so the calls follow one
// another with no drain and ramp between kernels -- what a launch per call
// costs at the end and start of every call ([FlashNorm digest], summary
// bullets on the dozens of norm launches per decode step).  Each
// workgroup looks up its call (item -> call table) and runs the one-wave,
// whole-k tile of the decode kernel on kGroupedBlocks column blocks of it.
// Two blocks per wave load each x fragment once for two weight fragments:
// measured on MI355X over the 65 calls of a 32-layer step at 8 rows, 1.416
// against 1.468 ms for one block (three: 1.427, four: 1.444), the same bits
// (each column's k order does not depend on how many blocks a wave holds).
// A single call of QKV or gate/up width does not gain from it: its few
// hundred waves would no longer spread evenly over the CUs (an LM head's
// thousands do, and take the decode kernel's two-block instances).
struct GroupCall {
  DecodeArgs a;
  const float* sg;   // fp8 weights: column scales of W'_gate (else unused)
  const float* su;   // fp8 weights: column scales of W'_up
  int first;         // index of the call's first workgroup in the launch
  int swiglu;
};

__global__ __launch_bounds__(kWave) void decode_grouped_kernel(const GroupCall* __restrict__ calls,
                                                               const uint16_t* __restrict__ item_call) {
  const int item = blockIdx.x;
  const int c = __builtin_amdgcn_readfirstlane((int)item_call[item]);
  const GroupCall& g = calls[c];
  const int nb = item - g.first;
  if (g.swiglu)
    decode_tile<__bf16, 1, kGroupedBlocks, true, 1, 1, 2>(g.a, nb, 0);
  else
    decode_tile<__bf16, 1, kGroupedBlocks, false, 1, 1, 4>(g.a, nb, 0);
}

// The grouped tile for fp8 (E4M3) weights with column scales and bf16 x of
// at most 16 rows: one wave streams the whole of k for NF column blocks
// (each with its gate and up streams for SwiGLU), x in registers.  The
// packed fp8 layout has one 1 KiB fragment per pair of k-blocks, a lane's
// 16 bytes being its 8 codes of each k-block of the pair (the B operand
// layout of v_mfma_f32_16x16x32_bf16), so one 16-byte load brings two
// k-blocks of a column block.  P pairs per stage, two stages in flight.
// Per column block and matrix the products are accumulated in k order, one
// MFMA per k-block, as in the entry point's kernel; the sum of squares is
// one Gram chain over k here, where the entry point adds per-wave partials,
// so 1/RMS can differ from it in the last fp32 bit.  The column scale joins
// 1/RMS in the epilogue.
// WK > 1 (single narrow calls): WK waves split the k pairs of the same
// column blocks, each a contiguous range in k order; wave 0 adds the other
// waves' partial products and Gram blocks in wave order after its own (fixed
// order, the same bits on every run) and runs the epilogue.
template <int NF, bool SW, int P, int WK = 1>
__device__ __forceinline__ void decode_tile_fp8(const DecodeArgs& a, const float* sg, const float* su, int bx) {
  constexpr int NMAT = SW ? 2 : 1;
  const int lane = threadIdx.x & (kWave - 1);
  const int wk = WK == 1 ? 0 : __builtin_amdgcn_readfirstlane((int)threadIdx.x / kWave);
  const int lrow = lane & 15, lgrp = lane >> 4;
  const int nb0 = bx * NF;
  const int kpairs = (a.kblocks + 1) / 2;
  const int full_pairs = a.K / 64;   // pairs whose two k-blocks lie inside K
  const int p_begin = (int)((int64_t)kpairs * wk / WK), p_end = (int)((int64_t)kpairs * (wk + 1) / WK);
  const int p_main_end = min(p_end, full_pairs);
  const __bf16* xrow = static_cast<const __bf16*>(a.x) + (size_t)min(lrow, a.M - 1) * a.K + lgrp * 8;
  const u32x4* wp[NMAT][NF];
  float sc[NMAT][NF];
#pragma unroll
  for (int nf = 0; nf < NF; ++nf) {
    const size_t base = (size_t)min(nb0 + nf, a.nblocks - 1) * kpairs * kWave + lane;
    const int col = (nb0 + nf) * 16 + lrow;
    wp[0][nf] = a.wg + base;
    sc[0][nf] = col < a.N ? sg[col] : 1.f;
    if constexpr (SW) {
      wp[NMAT - 1][nf] = a.wu + base;
      sc[NMAT - 1][nf] = col < a.N ? su[col] : 1.f;
    }
  }
  f32x4 acc[NMAT][NF];
  f32x4 gram = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
  for (int m = 0; m < NMAT; ++m)
#pragma unroll
    for (int nf = 0; nf < NF; ++nf) acc[m][nf] = f32x4{0.f, 0.f, 0.f, 0.f};

  struct Stage {
    u32x4 x[2 * P];
    u32x4 w[P][NMAT][NF];
  };
  auto load = [&](Stage& s, int p0) {
#pragma unroll
    for (int q = 0; q < P; ++q) {
      s.x[2 * q] = *reinterpret_cast<const u32x4*>(xrow + (size_t)(2 * (p0 + q)) * 32);
      s.x[2 * q + 1] = *reinterpret_cast<const u32x4*>(xrow + (size_t)(2 * (p0 + q) + 1) * 32);
#pragma unroll
      for (int m = 0; m < NMAT; ++m)
#pragma unroll
        for (int nf = 0; nf < NF; ++nf)
          s.w[q][m][nf] = __builtin_nontemporal_load(wp[m][nf] + (size_t)(p0 + q) * kWave);
    }
  };
  auto pair = [&](u32x4 x0, u32x4 x1, const u32x4 (&w)[NMAT][NF]) {
    u32x4 lo[NMAT][NF], hi[NMAT][NF];
#pragma unroll
    for (int m = 0; m < NMAT; ++m)
#pragma unroll
      for (int nf = 0; nf < NF; ++nf) e4m3x16_to_bf16(w[m][nf], lo[m][nf], hi[m][nf]);
    gram = mfma_chunk<__bf16>(x0, x0, gram);
#pragma unroll
    for (int m = 0; m < NMAT; ++m)
#pragma unroll
      for (int nf = 0; nf < NF; ++nf) acc[m][nf] = mfma_chunk<__bf16>(x0, lo[m][nf], acc[m][nf]);
    gram = mfma_chunk<__bf16>(x1, x1, gram);
#pragma unroll
    for (int m = 0; m < NMAT; ++m)
#pragma unroll
      for (int nf = 0; nf < NF; ++nf) acc[m][nf] = mfma_chunk<__bf16>(x1, hi[m][nf], acc[m][nf]);
  };
  auto compute = [&](const Stage& s) {
#pragma unroll
    for (int q = 0; q < P; ++q) pair(s.x[2 * q], s.x[2 * q + 1], s.w[q]);
  };

  // whole pairs, double-buffered as in decode_tile
  int p = p_begin;
  if (p + 2 * P <= p_main_end) {
    Stage s0, s1;
    load(s0, p);
    for (; p + 4 * P <= p_main_end; p += 2 * P) {
      load(s1, p + P);
      __builtin_amdgcn_sched_barrier(0);
      compute(s0);
      __builtin_amdgcn_sched_barrier(0);
      load(s0, p + 2 * P);
      __builtin_amdgcn_sched_barrier(0);
      compute(s1);
      __builtin_amdgcn_sched_barrier(0);
    }
    load(s1, p + P);
    __builtin_amdgcn_sched_barrier(0);
    compute(s0);
    compute(s1);
    p += 2 * P;
  }
  // the remaining pairs one at a time; x past K (a ragged last k-block, the
  // missing half of an odd last pair) reads as zero, and its codes are zero
  for (; p < p_end; ++p) {
    const bool in0 = (2 * p) * 32 + lgrp * 8 < a.K, in1 = (2 * p + 1) * 32 + lgrp * 8 < a.K;
    const u32x4 x0 = in0 ? *reinterpret_cast<const u32x4*>(xrow + (size_t)(2 * p) * 32) : u32x4{0u, 0u, 0u, 0u};
    const u32x4 x1 = in1 ? *reinterpret_cast<const u32x4*>(xrow + (size_t)(2 * p + 1) * 32) : u32x4{0u, 0u, 0u, 0u};
    u32x4 w[NMAT][NF];
#pragma unroll
    for (int m = 0; m < NMAT; ++m)
#pragma unroll
      for (int nf = 0; nf < NF; ++nf) w[m][nf] = __builtin_nontemporal_load(wp[m][nf] + (size_t)p * kWave);
    pair(x0, x1, w);
  }

  if constexpr (WK > 1) {
    __shared__ f32x4 red[WK - 1][NMAT * NF + 1][kWave];
    if (wk > 0) {
#pragma unroll
      for (int m = 0; m < NMAT; ++m)
#pragma unroll
        for (int nf = 0; nf < NF; ++nf) red[wk - 1][m * NF + nf][lane] = acc[m][nf];
      red[wk - 1][NMAT * NF][lane] = gram;
    }
    __syncthreads();
    if (wk == 0) {
#pragma unroll
      for (int w = 0; w < WK - 1; ++w) {
#pragma unroll
        for (int m = 0; m < NMAT; ++m)
#pragma unroll
          for (int nf = 0; nf < NF; ++nf) acc[m][nf] += red[w][m * NF + nf][lane];
        gram += red[w][NMAT * NF][lane];
      }
    }
  }

  // 1/RMS per row from the Gram diagonal (accumulator element r of lane l is
  // row 4*(l/16) + r, column l%16), shared through LDS
  __shared__ float inv_s[16];
  if (wk == 0 && (lrow >> 2) == lgrp) {
    const int r = lrow & 3;
    inv_s[lrow] = inv_rms(r == 0 ? gram[0] : (r == 1 ? gram[1] : (r == 2 ? gram[2] : gram[3])), (float)a.K, a.eps);
  }
  __syncthreads();
#pragma unroll
  for (int nf = 0; nf < NF; ++nf) {
    const int col = (nb0 + nf) * 16 + lrow;
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      const int row = 4 * lgrp + r;
      if (wk == 0 && row < a.M && col < a.N) {
        const float inv = inv_s[row];
        const float ga = acc[0][nf][r] * (sc[0][nf] * inv);
        const float v = SW ? silu_times(ga, acc[NMAT - 1][nf][r] * (sc[NMAT - 1][nf] * inv)) : ga;
        Store<__bf16>::one(static_cast<__bf16*>(a.y) + (size_t)row * a.N + col, v);
      }
    }
  }
}

// The grouped launch of fp8-weight calls.  Measured on MI355X over the 65
// calls of a 32-layer step at 8 rows (4.63 GB of codes): 678 us against
// 908 us for the same calls launched one by one (6.83 TB/s of weights);
// column blocks per wave (projection / SwiGLU pair) and k-block pairs per
// stage: 2/2/4 678 us, 2/2/2 684, 2/2/1 690, 4/2/4 694, 3/2/2 and 2/3/2 695,
// 4/2/2 699, 8/4/1 712, 2/1/2 723, 1/2/2 728.  The single calls, each a
// kernel of 9-17 us, lose most to their own ramp and drain, which the one
// grid removes.
__global__ __launch_bounds__(kWave) void decode_grouped_fp8_kernel(const GroupCall* __restrict__ calls,
                                                                   const uint16_t* __restrict__ item_call) {
  const int item = blockIdx.x;
  const int c = __builtin_amdgcn_readfirstlane((int)item_call[item]);
  const GroupCall& g = calls[c];
  const int nb = item - g.first;
  if (g.swiglu)
    decode_tile_fp8<kGroupedBlocksFp8Swiglu, true, kGroupedPairsFp8>(g.a, g.sg, g.su, nb);
  else
    decode_tile_fp8<kGroupedBlocksFp8, false, kGroupedPairsFp8>(g.a, g.sg, g.su, nb);
}

hipError_t launch_decode_grouped(const void* calls, const void* item_call, int items, bool fp8, hipStream_t stream) {
  const GroupCall* c = static_cast<const GroupCall*>(calls);
  const uint16_t* ic = static_cast<const uint16_t*>(item_call);
  void* args[] = {&c, &ic};
  const void* k = fp8 ? reinterpret_cast<const void*>(&decode_grouped_fp8_kernel)
                      : reinterpret_cast<const void*>(&decode_grouped_kernel);
  return hipLaunchKernel(k, dim3((unsigned)items), dim3(kWave), args, 0, stream);
}

size_t grouped_call_bytes() { return sizeof(GroupCall); }

// Single fp8-weight calls of at most 16 rows on narrow projections (at most
// 256 column blocks): the LDS-shared-x kernel gives them a workgroup per
// three column blocks (32 for a 1536-column share) and each wave's chain
// over k waits on memory at every stage; here one workgroup per column
// block splits k over four waves.  Measured on MI355X, K = 4096, 1-16 rows:
// 1536 columns 8.1-9.0 -> 6.2-7.3 us, 2 x 1376 11.8-12.8 -> 6.6-8.5 us,
// 4000 columns 8.6-9.2 -> 5.9-7.9 us.  Two waves on wider projections
// (6144-12288 columns) measured 0.7-1.2x, so those keep the LDS-shared-x
// kernel.
template <int SW, int P, int WK>
__global__ __launch_bounds__(kWave * WK) void decode_fp8_ksplit_kernel(DecodeArgs a, const float* sg,
                                                                      const float* su) {
  decode_tile_fp8<1, SW != 0, P, WK>(a, sg, su, blockIdx.x);
}

struct DecodeFp8KInstance {
  const void* fn;
  int p, wk;
  bool sw;
  const char* name;
};
#define FN_DECODE_F8K(SW, P, WK, NAME) \
  DecodeFp8KInstance { reinterpret_cast<const void*>(&decode_fp8_ksplit_kernel<SW, P, WK>), P, WK, SW != 0, NAME }
static const DecodeFp8KInstance kDecodeFp8K[] = {
    FN_DECODE_F8K(0, 4, 4, "decode_fp8_m16_n16_k4_p4"),
    FN_DECODE_F8K(1, 2, 4, "decode_swiglu_fp8_m16_n16_k4_p2"),
};

int fp8_k_split(int64_t M, int64_t N, bool swiglu) {
  (void)swiglu;
  return M <= 16 && ceil_div(N, 16) <= 256 ? 4 : 0;
}

static const DecodeFp8KInstance* find_fp8k(bool sw, int wk) {
  for (const DecodeFp8KInstance& d : kDecodeFp8K)
    if (d.sw == sw && d.wk == wk) return &d;
  return nullptr;
}

FusedPlan plan_fp8_ksplit(int64_t M, int64_t N, bool swiglu) {
  const DecodeFp8KInstance* d = find_fp8k(swiglu, fp8_k_split(M, N, swiglu));
  FusedPlan p{};
  p.kind = 12;
  p.mf = 1;
  p.nf = 1;
  p.waves = d != nullptr ? d->wk : 0;
  p.grid = dim3((unsigned)ceil_div(N, 16), 1, 1);
  p.block = dim3(kWave * p.waves, 1, 1);
  p.name = d != nullptr ? d->name : "invalid";
  return p;
}

hipError_t launch_fp8_ksplit(const FusedPlan& p, const void* x, const void* wg, const float* sg, const void* wu,
                             const float* su, void* y, int M, int K, int N, float eps, hipStream_t stream) {
  const DecodeFp8KInstance* d = find_fp8k(wu != nullptr, p.waves);
  if (d == nullptr || M > 16 || sg == nullptr || (wu != nullptr && su == nullptr)) return hipErrorInvalidValue;
  DecodeArgs a;
  a.x = x;
  a.wg = static_cast<const u32x4*>(wg);
  a.wu = static_cast<const u32x4*>(wu);
  a.y = y;
  a.M = M;
  a.K = K;
  a.N = N;
  a.kblocks = (int)ceil_div(K, k_per_block(DType::BF16));
  a.nblocks = (int)ceil_div(N, 16);
  a.eps = eps;
  void* args[] = {&a, &sg, &su};
  return hipLaunchKernel(d->fn, p.grid, p.block, args, 0, stream);
}

void grouped_call_fill(void* dst, const void* x, const void* wg, const void* wu, const float* sg, const float* su,
                       void* y, int M, int K, int N, float eps, int first) {
  GroupCall g{};
  g.a.x = x;
  g.a.wg = static_cast<const u32x4*>(wg);
  g.a.wu = static_cast<const u32x4*>(wu);
  g.a.y = y;
  g.a.M = M;
  g.a.K = K;
  g.a.N = N;
  g.a.kblocks = (int)ceil_div(K, k_per_block(DType::BF16));
  g.a.nblocks = (int)ceil_div(N, 16);
  g.a.eps = eps;
  g.sg = sg;
  g.su = su;
  g.first = first;
  g.swiglu = wu != nullptr;
  *static_cast<GroupCall*>(dst) = g;
}

// Kernel instances.  The table maps (dtype, row capacity, SwiGLU, k-split,
// column blocks per wave) to a tile configuration; launch_decode looks the
// instance up by the same key.
struct DecodeInstance {
  const void* fn;
  DType dt;
  int mf, nf, wn, wk, u;
  bool sw;
  const char* name;
};

#define FN_DECODE(TT, DT, MF, NF, SW, WN, WK, U, NAME)                                                    \
  DecodeInstance {                                                                                        \
    reinterpret_cast<const void*>(&decode_kernel<TT, MF, NF, SW, WN, WK, U>), DT, MF, NF, WN, WK, U, SW, NAME \
  }

// Tile choices measured on MI355X (cold weights, >= 1 GiB rotation): at one
// row block and full projection widths a single wave per workgroup
// streaming the whole k range with two 4-k-block stages in flight beats
// splitting k across waves.  Narrow projections -- one GPU's column share
// under tensor parallelism -- have too few column blocks to give every CU a
// wave, and there the k range is split over 4 waves (2 for SwiGLU up to 512
// blocks): measured 12.0 -> 8.1 us for 1536 QKV columns and 21.3 -> 10.9 us
// for 2 x 1376 gate/up columns at 16 rows.  bf16 with more than 16 rows goes
// to the kernel that shares x through LDS (decode_x.hip); fp32 keeps all
// three rungs here.
static const DecodeInstance kDecode[] = {
    FN_DECODE(__bf16, DType::BF16, 1, 1, false, 1, 1, 4, "decode_bf16_m16_n16_k1_u4"),
    FN_DECODE(__bf16, DType::BF16, 1, 1, true, 1, 1, 2, "decode_swiglu_bf16_m16_n16_k1_u2"),
    FN_DECODE(__bf16, DType::BF16, 1, 1, false, 1, 4, 4, "decode_bf16_m16_n16_k4_u4"),
    FN_DECODE(__bf16, DType::BF16, 1, 1, true, 1, 2, 2, "decode_swiglu_bf16_m16_n16_k2_u2"),
    FN_DECODE(__bf16, DType::BF16, 1, 1, true, 1, 4, 2, "decode_swiglu_bf16_m16_n16_k4_u2"),
    // narrow gate/up pairs at 17-64 rows (the LDS-shared-x kernel would run a
    // workgroup per three column blocks, 29 for 1376 columns): the rows in
    // registers, k over 4 waves -- at 2 x 1376 columns 21.9 -> 15.0 us for 32
    // rows, 26.4 -> 22.7 us for 64
    FN_DECODE(__bf16, DType::BF16, 2, 1, true, 1, 4, 2, "decode_swiglu_bf16_m32_n16_k4_u2"),
    FN_DECODE(__bf16, DType::BF16, 4, 1, true, 1, 4, 2, "decode_swiglu_bf16_m64_n16_k4_u2"),
    FN_DECODE(float, DType::F32, 1, 1, false, 1, 4, 2, "decode_f32_m16_n16_k4_u2"),
    FN_DECODE(float, DType::F32, 2, 1, false, 1, 4, 2, "decode_f32_m32_n16_k4_u2"),
    FN_DECODE(float, DType::F32, 4, 1, false, 1, 4, 2, "decode_f32_m64_n16_k4_u2"),
    FN_DECODE(float, DType::F32, 1, 1, true, 1, 4, 2, "decode_swiglu_f32_m16_n16_k4_u2"),
    FN_DECODE(float, DType::F32, 2, 1, true, 1, 4, 2, "decode_swiglu_f32_m32_n16_k4_u2"),
    FN_DECODE(float, DType::F32, 4, 1, true, 1, 4, 2, "decode_swiglu_f32_m64_n16_k4_u2"),
    // very wide projections (an LM head) at up to 16 rows: two column blocks
    // per wave load each x fragment once for two weight fragments, and there
    // are still three or more waves per CU -- measured 48.9 -> 43.9 us for
    // 16 x 4096 -> 32000 and 200 -> 168 us for 16 x 4096 -> 128256 (at 8
    // rows 43.0 -> 43.3 and 166 -> 162 us), the same bits
    FN_DECODE(__bf16, DType::BF16, 1, 2, false, 1, 1, 4, "decode_bf16_m16_n32_k1_u4"),
    FN_DECODE(__bf16, DType::BF16, 1, 2, true, 1, 1, 2, "decode_swiglu_bf16_m16_n32_k1_u2"),
};

// wk 0: the first instance of (dt, mf, sw, nf) in the table (its default).
static const DecodeInstance* find_decode(DType dt, int mf, bool sw, int wk = 0, int nf = 1) {
  for (const DecodeInstance& d : kDecode)
    if (d.dt == dt && d.mf == mf && d.sw == sw && (wk == 0 || d.wk == wk) && d.nf == nf) return &d;
  return nullptr;
}

// Column blocks per wave: two at up to 16 rows of bf16 once there are at
// least 1536 column blocks (768 two-block waves, three per CU).
static int decode_blocks_per_wave(DType dt, int64_t M, int64_t N) {
  return dt == DType::BF16 && M <= 16 && ceil_div(N, 16) >= 1536 ? 2 : 1;
}

// k-split for bf16: 4 waves when there are at most 256 workgroups of one
// wave (fewer than the CUs) at the row rung's tile of 16 * mf rows, 2 for
// SwiGLU up to 512.
static int decode_k_split(DType dt, int64_t M, int64_t N, bool swiglu, int mf) {
  if (dt != DType::BF16) return 0;
  const int64_t wgs = ceil_div(N, 16) * ceil_div(M, 16 * mf);
  if (wgs <= 256) return 4;
  if (swiglu && wgs <= 512) return 2;
  return 1;
}

// M-ladder: the smallest row capacity in {16, 32, 64} that holds M (the
// ladder idea of [FlashInfer #5668], K23_LADDER, without its upper bound:
// a larger M tiles the rows over grid.y).
FusedPlan plan_decode(DType dt, int64_t M, int64_t K, int64_t N, bool swiglu) {
  (void)K;
  const int mf = M <= 16 ? 1 : (M <= 32 ? 2 : 4);
  const int nf = decode_blocks_per_wave(dt, M, N);
  const DecodeInstance* d = nf > 1 ? find_decode(dt, 1, swiglu, 1, nf)
                                   : find_decode(dt, mf, swiglu, decode_k_split(dt, M, N, swiglu, mf));
  if (d == nullptr) d = find_decode(dt, 1, swiglu, decode_k_split(dt, M, N, swiglu, 1));   // bf16 rows tiled
  if (d == nullptr) d = find_decode(dt, 1, swiglu);
  FusedPlan p{};
  p.kind = 0;
  p.mf = d->mf;
  p.nf = d->nf * d->wn;
  p.waves = d->wn * d->wk;
  const int64_t nblocks = ceil_div(N, 16);
  p.grid = dim3((unsigned)ceil_div(nblocks, p.nf), (unsigned)ceil_div(M, 16 * p.mf), 1);
  p.block = dim3(kWave * p.waves, 1, 1);
  p.name = d->name;
  return p;
}

hipError_t launch_decode(DType dt, const FusedPlan& p, const void* x, const void* wg, const void* wu, void* y,
                         int M, int K, int N, float eps, hipStream_t stream) {
  const DecodeInstance* d = find_decode(dt, p.mf, wu != nullptr, p.waves, p.nf);   // one column group: waves = k-split
  if (d == nullptr) return hipErrorInvalidValue;
  DecodeArgs a;
  a.x = x;
  a.wg = static_cast<const u32x4*>(wg);
  a.wu = static_cast<const u32x4*>(wu);
  a.y = y;
  a.M = M;
  a.K = K;
  a.N = N;
  a.kblocks = (int)ceil_div(K, k_per_block(dt));
  a.nblocks = (int)ceil_div(N, 16);
  a.eps = eps;
  void* args[] = {&a};
  return hipLaunchKernel(d->fn, p.grid, p.block, args, 0, stream);
}

}  // namespace fn
