// Fused RMSNorm + projection (+ SwiGLU) for 17..64 rows (bf16), with x
// shared through LDS.
//
// Past 16 rows x stops being small next to W': at 64 rows it is 128 KiB per
// 1024 k values, and a kernel that loads x into every wave's registers
// (decode.hip) pushes about as many x bytes through each CU's vector memory
// path as W' bytes, which is what bounds a skinny kernel on this chip (the
// per-CU request rate, not HBM).  Here a workgroup owns NWV weight column
// blocks -- one (or NC) per wave, for SwiGLU with both the gate and the up
// stream -- and its waves walk the k range in lock step.  Per stage of U
// k-blocks the x rows are fetched once for the workgroup, split across its
// waves, straight into an LDS ring slot with direct global-to-LDS buffer
// loads; every wave then reads its MFMA operands with ds_read_b128.  Each
// wave streams its own W' fragments from HBM into registers with
// non-temporal buffer loads, NS-1 stages ahead.
//
// x layout in a slot: each 1 KiB load carries 8 rows x 128 bytes (two
// k-blocks), so every request is a whole cache line; the 16-byte chunks of
// row r are stored permuted by r/2 so that the 16 lanes of each quarter
// wave read 16 distinct bank groups.
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
// k-blocks per stage.
template <int MF, int NC, int NWV, bool SW, int U>
__global__ __launch_bounds__(kWave * NWV) void decode_x_kernel(DecodeXArgs a) {
  constexpr int NS = 4;                    // LDS ring slots
  constexpr int D = NS - 1;                // stages in flight
  constexpr int NMAT = SW ? 2 : 1;
  constexpr int NST = NMAT * NC;           // weight streams per wave
  constexpr int XF = U * MF;               // x loads (1 KiB each) per stage
  constexpr int XPW = (XF + NWV - 1) / NWV;   // x loads each wave issues per stage
  constexpr int LPW = U * NST + XPW;       // vector-memory ops per wave per stage
  // Loads q >= XF (when NWV does not divide XF) fetch nothing and write
  // zeros into the slot's padding, so every wave issues the same count.
  constexpr int SLOT = XPW * NWV * kFragBytes;
  static_assert(U % 2 == 0, "each x load moves two k-blocks of 8 rows");
  static_assert((D - 1) * LPW < 64, "vmcnt range");
  static_assert(NS * SLOT + NWV * XPW * 16 * 4 <= 160 * 1024, "LDS budget");

  __shared__ __attribute__((aligned(1024))) uint8_t ring0[SLOT];
  __shared__ __attribute__((aligned(1024))) uint8_t ring1[SLOT];
  __shared__ __attribute__((aligned(1024))) uint8_t ring2[SLOT];
  __shared__ __attribute__((aligned(1024))) uint8_t ring3[SLOT];
  __shared__ float ssp[NWV][XPW][16];      // Gram diagonals
  auto slot_ptr = [&](int s) __attribute__((always_inline)) -> uint8_t* {
    return s == 0 ? ring0 : (s == 1 ? ring1 : (s == 2 ? ring2 : ring3));
  };

  const int lane = threadIdx.x & (kWave - 1);
  const int w = __builtin_amdgcn_readfirstlane(threadIdx.x / kWave);
  const int lrow = lane & 15, lgrp = lane >> 4;
  const int nb0 = (blockIdx.x * NWV + w) * NC;   // first column block of this wave
  const int64_t kfrag = (int64_t)a.kblocks * kFragBytes;

  const __amdgpu_buffer_rsrc_t xr = make_rsrc_x(a.x, (int64_t)min(MF * 16, a.M) * a.K * 2);
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
#pragma unroll
  for (int i = 0; i < XPW; ++i) {
    const int q = w + NWV * i;
    const int lr = 8 * (q & 1) + (lane >> 3);
    const int c = (lane & 7) ^ (lr >> 1);
    const int row = 16 * ((q >> 1) % MF) + lr;
    xk[i] = q < XF ? (2 * (q / (2 * MF)) + (c >> 2)) * 32 + (c & 3) * 8 : 1 << 30;   // past XF: never in range
    xoff[i] = (uint32_t)(row * a.K + (q < XF ? xk[i] : 0)) * 2u;
  }
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
  auto issue_x = [&](uint8_t* base, int st) __attribute__((always_inline)) {
    const uint32_t live = (uint32_t)((st - a.stages) >> 31);
    const int k0 = st * U * 32;
#pragma unroll
    for (int i = 0; i < XPW; ++i) {
      const uint32_t in = live & (uint32_t)((k0 + xk[i] - a.K) >> 31);
      const uint32_t off = ((xoff[i] + (uint32_t)k0 * 2u) & in) | (kOutOfRangeX & ~in);
      __builtin_amdgcn_raw_ptr_buffer_load_lds(xr, (lds_ptr_x)(base + (w + NWV * i) * kFragBytes), 16, off, 0, 0,
                                               0);
    }
  };
  u32x4 wv[NS][U][NST];
  auto issue_w = [&](int b, int st) __attribute__((always_inline)) {
    const uint32_t live = (uint32_t)((st - a.stages) >> 31);
#pragma unroll
    for (int u = 0; u < U; ++u) {
      const uint32_t off = (uint32_t)((st * U + u) * kFragBytes + lane * 16);
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
    __builtin_amdgcn_s_barrier();
    __builtin_amdgcn_sched_barrier(0);
    const uint8_t* base = slot_ptr(s);
    u32x4 xv[U][MF];
    u32x4 xg[XPW];
#pragma unroll
    for (int u = 0; u < U; ++u)
#pragma unroll
      for (int i = 0; i < MF; ++i) xv[u][i] = *reinterpret_cast<const u32x4*>(base + x_at(u, i));
#pragma unroll
    for (int j = 0; j < XPW; ++j) xg[j] = *reinterpret_cast<const u32x4*>(base + frag_at(w + NWV * j));
    __builtin_amdgcn_sched_barrier(0);
    issue_w((s + D) % NS, st + D);
    issue_x(slot_ptr((s + D) % NS), st + D);
    __builtin_amdgcn_sched_barrier(0);
#pragma unroll
    for (int u = 0; u < U; ++u)
#pragma unroll
      for (int i = 0; i < MF; ++i)
#pragma unroll
        for (int c = 0; c < NST; ++c) acc[c][i] = mfma_chunk<__bf16>(xv[u][i], wv[s][u][c], acc[c][i]);
#pragma unroll
    for (int j = 0; j < XPW; ++j) gram[j] = mfma_chunk<__bf16>(xg[j], xg[j], gram[j]);
  };

#pragma unroll
  for (int p = 0; p < D; ++p) {
    issue_w(p, p);
    issue_x(slot_ptr(p), p);
    __builtin_amdgcn_sched_barrier(0);   // keep the loop's load order: W', then x
  }
  // whole rounds of the ring; stages past the last read as zero
  for (int st = 0; st < a.stages; st += NS) {
    step(0, st);
    step(1, st + 1);
    step(2, st + 2);
    step(3, st + 3);
  }
  wait_vmcnt_x<0>();

  // Accumulator element e of lane l is row 4*(l/16) + e, column l%16 of its
  // 16x16 tile, so the Gram diagonal sits in lanes with (l%16)/4 == l/16.
  if ((lrow >> 2) == lgrp) {
    const int e = lrow & 3;
#pragma unroll
    for (int j = 0; j < XPW; ++j)
      ssp[w][j][lrow] = e == 0 ? gram[j][0] : (e == 1 ? gram[j][1] : (e == 2 ? gram[j][2] : gram[j][3]));
  }
  __syncthreads();

  const float kf = (float)a.K;
#pragma unroll
  for (int i = 0; i < MF; ++i) {
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      const int rr = 4 * lgrp + e;
      const int row = 16 * i + rr;
      // Gram accumulator j of wave v holds fragment q = v + NWV*j, row block q % MF
      float ss = 0.f;
#pragma unroll
      for (int v = 0; v < NWV; ++v)
#pragma unroll
        for (int j = 0; j < XPW; ++j)
          if (v + NWV * j < XF && (v + NWV * j) % MF == i) ss += ssp[v][j][rr];
      const float inv = inv_rms(ss, kf, a.eps);
#pragma unroll
      for (int j = 0; j < NC; ++j) {
        const int col = (nb0 + j) * 16 + lrow;
        if (row < a.M && col < a.N) {
          const float val = SW ? silu_times(acc[j][i][e] * inv, acc[NC + j][i][e] * inv) : acc[j][i][e] * inv;
          Store<__bf16>::one(static_cast<__bf16*>(a.y) + (size_t)row * a.N + col, val);
        }
      }
    }
  }
}

struct DecodeXInstance {
  const void* fn;
  int mf, nc, nwv, u;
  bool sw;
  const char* name;
};

#define FN_DECODE_X(MF, NC, NWV, SW, U, NAME) \
  DecodeXInstance { reinterpret_cast<const void*>(&decode_x_kernel<MF, NC, NWV, SW, U>), MF, NC, NWV, U, SW, NAME }

inline hipError_t launch_decode_x_instance(const DecodeXInstance& d, const void* x, const void* wg, const void* wu,
                                           void* y, int M, int K, int N, float eps, hipStream_t stream) {
  DecodeXArgs a;
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
  return hipLaunchKernel(d.fn, dim3((unsigned)ceil_div(a.nblocks, d.nc * d.nwv)), dim3(kWave * d.nwv), args, 0,
                         stream);
}

#ifndef FN_DECODE_X_NO_TABLE
// Measured on MI355X (cold weights): three one-column-block waves per
// workgroup, two-k-block stages.  A skinny kernel is bounded by each CU's
// vector-memory request rate, so what counts is the bytes each CU moves and
// that every CU moves some: three column blocks per workgroup give 256
// workgroups for 12288 columns (one per CU) and 230 for 11008, with each CU
// fetching x once per three weight streams.  Four waves (192 and 172
// workgroups) measured 10-15% slower, two waves slower still; wider waves,
// deeper stages and k-splits inside the workgroup did not help.
static const DecodeXInstance kDecodeX[] = {
    FN_DECODE_X(2, 1, 3, false, 2, "decode_bf16_m32_xlds_w3_u2"),
    FN_DECODE_X(4, 1, 3, false, 2, "decode_bf16_m64_xlds_w3_u2"),
    FN_DECODE_X(2, 1, 3, true, 2, "decode_swiglu_bf16_m32_xlds_w3_u2"),
    FN_DECODE_X(4, 1, 3, true, 2, "decode_swiglu_bf16_m64_xlds_w3_u2"),
};

static const DecodeXInstance* find_decode_x(int mf, bool sw) {
  for (const DecodeXInstance& d : kDecodeX)
    if (d.mf == mf && d.sw == sw) return &d;
  return nullptr;
}

// Row ladder rungs 32 and 64; one workgroup row, NC*NWV column blocks each.
FusedPlan plan_decode_x(DType dt, int64_t M, int64_t K, int64_t N, bool swiglu) {
  (void)dt;
  (void)K;
  const DecodeXInstance* d = find_decode_x(M <= 32 ? 2 : 4, swiglu);
  FusedPlan p{};
  p.kind = 2;
  p.mf = d->mf;
  p.nf = d->nc * d->nwv;
  p.waves = d->nwv;
  p.grid = dim3((unsigned)ceil_div(ceil_div(N, 16), p.nf), 1, 1);
  p.block = dim3(kWave * p.waves, 1, 1);
  p.name = d->name;
  return p;
}

hipError_t launch_decode_x(DType dt, const FusedPlan& p, const void* x, const void* wg, const void* wu, void* y,
                           int M, int K, int N, float eps, hipStream_t stream) {
  const DecodeXInstance* d = find_decode_x(p.mf, wu != nullptr);
  if (dt != DType::BF16 || d == nullptr || M > 16 * d->mf) return hipErrorInvalidValue;
  return launch_decode_x_instance(*d, x, wg, wu, y, M, K, N, eps, stream);
}
#endif

}  // namespace fn
