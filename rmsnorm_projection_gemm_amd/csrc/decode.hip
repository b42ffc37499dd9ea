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

template <typename T, int MF, int NF, bool SW, int WN, int WK, int U>
__global__ __launch_bounds__(kWave * WN * WK) void decode_kernel(DecodeArgs a) {
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
  const int nb0 = (blockIdx.x * WN + wn) * NF;
  const int m0 = blockIdx.y * 16 * MF;
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
      for (; kb + 4 * U <= hi; kb += 2 * U) {
        load(s1, kb + U);
        __builtin_amdgcn_sched_barrier(0);
        compute(s0);
        __builtin_amdgcn_sched_barrier(0);
        load(s0, kb + 2 * U);
        __builtin_amdgcn_sched_barrier(0);
        compute(s1);
        __builtin_amdgcn_sched_barrier(0);
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

// Kernel instances.  The table maps (dtype, row capacity, SwiGLU) to a tile
// configuration; launch_decode looks the instance up by the same key.
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
};

// wk 0: the first instance of (dt, mf, sw) in the table (its default).
static const DecodeInstance* find_decode(DType dt, int mf, bool sw, int wk = 0) {
  for (const DecodeInstance& d : kDecode)
    if (d.dt == dt && d.mf == mf && d.sw == sw && (wk == 0 || d.wk == wk)) return &d;
  return nullptr;
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
  const DecodeInstance* d = find_decode(dt, mf, swiglu, decode_k_split(dt, M, N, swiglu, mf));
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
  const DecodeInstance* d = find_decode(dt, p.mf, wu != nullptr, p.waves);   // one column group: waves = k-split
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
