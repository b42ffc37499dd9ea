// Fused RMSNorm + projection (+ SwiGLU) for small row counts (decode).
//
// One launch computes, per output tile, the contraction x * W' on the MFMA
// units and the per-row sum of squares of x on the VALU from the very same
// x registers, then applies the deferred 1/RMS scale (and SiLU * up) to the
// fp32 accumulators and stores the tile once ([FlashNorm digest] proposals
// 1-2; [FlashInfer #5521] "Design" item 2, register-level SwiGLU).  Nothing
// intermediate is written to memory and there is no second stream to join,
// so the stale-buffer race the FlashNorm talk describes (a post-scale step
// reading a product that another stream had not finished) cannot occur.
//
// Decomposition: a workgroup owns NF 16-column blocks of W' (for SwiGLU the
// same columns of W'_gate and W'_up) and MF 16-row blocks of x; its WAVES
// waves split the k-blocks between them and stream their share of W' from
// HBM exactly once.  Partial accumulators and sums of squares meet in LDS,
// where the epilogue finishes them.  W' uses the packed fragment layout, so
// each lane's weight operand is one 16-byte load and a wave reads 1 KiB of
// contiguous memory per fragment.
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

template <typename T, int MF, int NF, bool SW, int WAVES, int U>
__global__ __launch_bounds__(kWave * WAVES) void decode_kernel(DecodeArgs a) {
  constexpr int V = Geo<T>::V;
  constexpr int KB = Geo<T>::KB;
  constexpr int NMAT = SW ? 2 : 1;
  const int lane = threadIdx.x & (kWave - 1);
  const int wave = threadIdx.x / kWave;
  const int lrow = lane & 15;       // operand row (x) / column (W') of this lane
  const int lgrp = lane >> 4;       // k group of this lane
  const int nb0 = blockIdx.x * NF;
  const int m0 = blockIdx.y * 16 * MF;
  const int kb_begin = (int)((int64_t)a.kblocks * wave / WAVES);
  const int kb_end = (int)((int64_t)a.kblocks * (wave + 1) / WAVES);

  const T* xrow[MF];
#pragma unroll
  for (int mf = 0; mf < MF; ++mf) {
    const int row = m0 + 16 * mf + lrow;
    xrow[mf] = row < a.M ? static_cast<const T*>(a.x) + (size_t)row * a.K + lgrp * V : nullptr;
  }
  const u32x4* wp[NMAT][NF];
  bool wok[NF];
#pragma unroll
  for (int nf = 0; nf < NF; ++nf) {
    const int nb = nb0 + nf;
    wok[nf] = nb < a.nblocks;
    const size_t base = ((size_t)(wok[nf] ? nb : 0) * a.kblocks) * kWave + lane;
    wp[0][nf] = a.wg + base;
    if (SW) wp[NMAT - 1][nf] = a.wu + base;
  }

  f32x4 acc[NMAT][MF][NF];
#pragma unroll
  for (int m = 0; m < NMAT; ++m)
#pragma unroll
    for (int mf = 0; mf < MF; ++mf)
#pragma unroll
      for (int nf = 0; nf < NF; ++nf) acc[m][mf][nf] = f32x4{0.f, 0.f, 0.f, 0.f};
  float ss[MF];
#pragma unroll
  for (int mf = 0; mf < MF; ++mf) ss[mf] = 0.f;

  const u32x4 zero = {0u, 0u, 0u, 0u};
  for (int kb = kb_begin; kb < kb_end; kb += U) {
    u32x4 xv[U][MF];
    u32x4 wv[U][NMAT][NF];
#pragma unroll
    for (int u = 0; u < U; ++u) {
      const int k = kb + u;
      const bool kin = k < kb_end;
#pragma unroll
      for (int mf = 0; mf < MF; ++mf) {
        const bool ok = kin && xrow[mf] != nullptr && (k * KB + lgrp * V) < a.K;
        xv[u][mf] = ok ? *reinterpret_cast<const u32x4*>(xrow[mf] + (size_t)k * KB) : zero;
      }
#pragma unroll
      for (int m = 0; m < NMAT; ++m)
#pragma unroll
        for (int nf = 0; nf < NF; ++nf)
          wv[u][m][nf] = (kin && wok[nf]) ? wp[m][nf][(size_t)k * kWave] : zero;
    }
#pragma unroll
    for (int u = 0; u < U; ++u) {
#pragma unroll
      for (int mf = 0; mf < MF; ++mf) {
        ss[mf] += sumsq16<T>(xv[u][mf]);
#pragma unroll
        for (int m = 0; m < NMAT; ++m)
#pragma unroll
          for (int nf = 0; nf < NF; ++nf)
            acc[m][mf][nf] = mfma_chunk<T>(xv[u][mf], wv[u][m][nf], acc[m][mf][nf]);
      }
    }
  }

  // Each row's partial sum of squares is spread over the four k groups.
#pragma unroll
  for (int mf = 0; mf < MF; ++mf) {
    ss[mf] += __shfl_xor(ss[mf], 16);
    ss[mf] += __shfl_xor(ss[mf], 32);
  }

  __shared__ float red_acc[WAVES][NMAT][MF][NF][4][kWave];
  __shared__ float red_ss[WAVES][MF][16];
#pragma unroll
  for (int m = 0; m < NMAT; ++m)
#pragma unroll
    for (int mf = 0; mf < MF; ++mf)
#pragma unroll
      for (int nf = 0; nf < NF; ++nf)
#pragma unroll
        for (int r = 0; r < 4; ++r) red_acc[wave][m][mf][nf][r][lane] = acc[m][mf][nf][r];
  if (lgrp == 0) {
#pragma unroll
    for (int mf = 0; mf < MF; ++mf) red_ss[wave][mf][lrow] = ss[mf];
  }
  __syncthreads();

  // Epilogue: wave w finishes tiles w, w + WAVES, ...  Accumulator element r
  // of lane l is row 4*(l/16) + r, column l%16 of the 16x16 tile.
  const float kf = (float)a.K;
  for (int t = wave; t < MF * NF; t += WAVES) {
    const int mf = t / NF, nf = t % NF;
    const int col = (nb0 + nf) * 16 + lrow;
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      const int i = 4 * lgrp + r;
      const int row = m0 + 16 * mf + i;
      float sum_sq = 0.f, p0 = 0.f, p1 = 0.f;
#pragma unroll
      for (int w = 0; w < WAVES; ++w) {
        sum_sq += red_ss[w][mf][i];
        p0 += red_acc[w][0][mf][nf][r][lane];
        if (SW) p1 += red_acc[w][NMAT - 1][mf][nf][r][lane];
      }
      if (row < a.M && col < a.N) {
        const float inv = inv_rms(sum_sq, kf, a.eps);
        const float v = SW ? silu_times(p0 * inv, p1 * inv) : p0 * inv;
        Store<T>::one(static_cast<T*>(a.y) + (size_t)row * a.N + col, v);
      }
    }
  }
}

namespace {

constexpr int kDecodeWaves = 4;
constexpr int kDecodeUnroll = 4;

template <typename T, int MF, int NF, bool SW>
const void* decode_fn() {
  return reinterpret_cast<const void*>(&decode_kernel<T, MF, NF, SW, kDecodeWaves, kDecodeUnroll>);
}

template <typename T, bool SW>
const void* pick(int mf, int nf) {
  if (nf == 1) {
    if (mf == 1) return decode_fn<T, 1, 1, SW>();
    if (mf == 2) return decode_fn<T, 2, 1, SW>();
    return decode_fn<T, 4, 1, SW>();
  }
  if (mf == 1) return decode_fn<T, 1, 2, SW>();
  if (mf == 2) return decode_fn<T, 2, 2, SW>();
  return decode_fn<T, 4, 2, SW>();
}

const char* decode_name(DType dt, int mf, int nf, bool sw) {
  static const char* names[2][2][3][2] = {
      {{{"decode_f32_m16_n16_w4", "decode_f32_m16_n32_w4"},
        {"decode_f32_m32_n16_w4", "decode_f32_m32_n32_w4"},
        {"decode_f32_m64_n16_w4", "decode_f32_m64_n32_w4"}},
       {{"decode_swiglu_f32_m16_n16_w4", "decode_swiglu_f32_m16_n32_w4"},
        {"decode_swiglu_f32_m32_n16_w4", "decode_swiglu_f32_m32_n32_w4"},
        {"decode_swiglu_f32_m64_n16_w4", "decode_swiglu_f32_m64_n32_w4"}}},
      {{{"decode_bf16_m16_n16_w4", "decode_bf16_m16_n32_w4"},
        {"decode_bf16_m32_n16_w4", "decode_bf16_m32_n32_w4"},
        {"decode_bf16_m64_n16_w4", "decode_bf16_m64_n32_w4"}},
       {{"decode_swiglu_bf16_m16_n16_w4", "decode_swiglu_bf16_m16_n32_w4"},
        {"decode_swiglu_bf16_m32_n16_w4", "decode_swiglu_bf16_m32_n32_w4"},
        {"decode_swiglu_bf16_m64_n16_w4", "decode_swiglu_bf16_m64_n32_w4"}}}};
  const int mi = mf == 1 ? 0 : (mf == 2 ? 1 : 2);
  return names[(int)dt][sw ? 1 : 0][mi][nf - 1];
}

}  // namespace

// M-ladder: the smallest row capacity in {16, 32, 64} that holds M (the
// ladder idea of [FlashInfer #5668], K23_LADDER, without its upper bound:
// larger M tiles the rows over grid.y).
FusedPlan plan_decode(DType dt, int64_t M, int64_t K, int64_t N, bool swiglu) {
  (void)K;
  FusedPlan p{};
  p.kind = 0;
  p.mf = M <= 16 ? 1 : (M <= 32 ? 2 : 4);
  p.nf = 1;
  p.waves = kDecodeWaves;
  const int64_t nblocks = ceil_div(N, 16);
  p.grid = dim3((unsigned)ceil_div(nblocks, p.nf), (unsigned)ceil_div(M, 16 * p.mf), 1);
  p.block = dim3(kWave * kDecodeWaves, 1, 1);
  p.name = decode_name(dt, p.mf, p.nf, swiglu);
  return p;
}

hipError_t launch_decode(DType dt, const FusedPlan& p, const void* x, const void* wg,
                         const void* wu, void* y, int M, int K, int N, float eps,
                         hipStream_t stream) {
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
  const bool sw = wu != nullptr;
  const void* fn;
  if (dt == DType::BF16)
    fn = sw ? pick<__bf16, true>(p.mf, p.nf) : pick<__bf16, false>(p.mf, p.nf);
  else
    fn = sw ? pick<float, true>(p.mf, p.nf) : pick<float, false>(p.mf, p.nf);
  void* args[] = {&a};
  return hipLaunchKernel(fn, p.grid, p.block, args, 0, stream);
}

}  // namespace fn
