// Fused RMSNorm + projection (+ SwiGLU) for many rows (prefill): the
// compute-bound regime, one launch.
//
// A workgroup computes a BM x BN output tile (BM = 16*FM*WM rows, BN =
// 16*FN*WN columns per weight matrix) with WM x WN waves, each owning a
// 16*FM x 16*FN sub-tile whose fp32 accumulators stay in registers for the
// whole k loop.  The instances use 256x256 tiles (256x128 per matrix for
// SwiGLU) with eight waves of 64x128, two waves per SIMD, and a 3-slot ring:
// measured on MI355X this beats four waves of 128x128 by ~40%, the second
// wave hiding the barrier and LDS latency of the first.  Operands stream through an NS-stage LDS ring, one 32-wide
// k-block per stage, filled by direct global-to-LDS buffer loads (no
// register staging).  Every operand lands in LDS already in MFMA fragment
// order -- W' because the packed layout is fragment-major, x because each
// lane of the loading wave fetches exactly the 16 bytes its MFMA lane will
// own -- so each fragment read is one conflict-free ds_read_b128 at lane*16.
// Loads past the matrix edges (rows >= M, columns past the packed width,
// k >= K) use out-of-range buffer offsets, which read as zero.
//
// The per-row sum of squares comes from the x fragments already in
// registers: each of the WN waves that share a row block takes a 1/WN share
// of its row fragments, either on the VALU (convert and FMA) or, in the
// instances, as the diagonal of an x x^T MFMA (GRAM), which measured faster
// than the VALU form once the MFMA pipe is the bottleneck only 1/16 of the
// time it spends on the projection.  The shares meet in LDS before the
// epilogue applies 1/RMS (and SiLU * up) to the accumulators and stores
// ([FlashNorm digest] proposals 1-2; [FlashInfer #5521] "Design" items 1-2,
// tiles kept resident across the k loop and the SwiGLU applied to the
// accumulators in registers).
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

template <int FM, int FN, int WM, int WN, bool SW, int NS, bool GRAM, bool Q8>
__global__ __launch_bounds__(kWave * WM * WN) void prefill_kernel(PrefillArgs a) {
  constexpr int NW = WM * WN;
  constexpr int NMAT = SW ? 2 : 1;
  constexpr int BMF = FM * WM;                   // 16-row fragments per tile
  constexpr int BNF = FN * WN;                   // 16-column fragments per tile and matrix
  constexpr int SFR = BMF + NMAT * BNF;          // fragments per stage (one k-block)
  constexpr int LPW = SFR / NW;                  // loads per wave per stage
  constexpr int ALPW = BMF / NW;                 // of which x fragments
  constexpr int SSF = FM / WN;                   // row fragments whose squares this wave sums
  static_assert(SFR % NW == 0 && BMF % NW == 0 && FM % WN == 0, "tile shape");
  static_assert(NS >= 2 && NS <= 4 && (NS - 2) * LPW < 64, "stage count");

  // One LDS array per ring slot: the compiler can then tell a read of slot s
  // from the direct-to-LDS loads still filling the other slots, instead of
  // waiting for all of them before every read.
  constexpr int SLOT = SFR * kFragBytes;
  __shared__ __attribute__((aligned(1024))) uint8_t ring0[SLOT];
  __shared__ __attribute__((aligned(1024))) uint8_t ring1[SLOT];
  __shared__ __attribute__((aligned(1024))) uint8_t ring2[NS > 2 ? SLOT : 16];
  __shared__ __attribute__((aligned(1024))) uint8_t ring3[NS > 3 ? SLOT : 16];
  __shared__ float ssbuf[BMF * 16];
  // slot s is a literal at every call site, so this folds to one array
  auto slot_ptr = [&](int s) __attribute__((always_inline)) -> uint8_t* { return s == 0 ? ring0 : (s == 1 ? ring1 : (s == 2 ? ring2 : ring3)); };

  const int lane = threadIdx.x & (kWave - 1);
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x / kWave);
  const int wm = wave / WN, wn = wave % WN;
  const int lrow = lane & 15, lgrp = lane >> 4;
  const int m0 = blockIdx.y * BMF * 16;
  const int nb0 = blockIdx.x * BNF;
  const int64_t kfrag = (int64_t)a.kblocks * kFragBytes;   // bytes of one packed column block

  const __amdgpu_buffer_rsrc_t xr =
      make_rsrc(static_cast<const __bf16*>(a.x) + (size_t)m0 * a.K, (int64_t)min(BMF * 16, a.M - m0) * a.K * 2);
  // (two named descriptors: an array of this opaque type would make the
  // host compilation pass drop the kernel's launch stub)
  const int64_t wbytes = (int64_t)min(BNF, a.nblocks - nb0) * kfrag;
  const __amdgpu_buffer_rsrc_t wr0 = make_rsrc(static_cast<const uint8_t*>(a.wg) + nb0 * kfrag, wbytes);
  const __amdgpu_buffer_rsrc_t wr1 = make_rsrc(static_cast<const uint8_t*>(SW ? a.wu : a.wg) + nb0 * kfrag, wbytes);

  // Fragments this wave loads each stage: f = wave + NW * i.  The first ALPW
  // are x fragments (row block f), the rest W' fragments.
  uint32_t xoff[ALPW];    // byte offset of this lane's x chunk at k-block 0
#pragma unroll
  for (int i = 0; i < ALPW; ++i) {
    const int row = 16 * (wave + NW * i) + lrow;
    xoff[i] = (uint32_t)(row * a.K + lgrp * 8) * 2u;
  }
  auto issue = [&](uint8_t* base, int kb) __attribute__((always_inline)) {
    // all-ones while in range, else zero: out-of-range offsets read as zero
    const uint32_t xin = (uint32_t)((kb * 32 + lgrp * 8 - a.K) >> 31);
    const uint32_t win = (uint32_t)((kb - a.kblocks) >> 31);
#pragma unroll
    for (int i = 0; i < LPW; ++i) {
      const int f = wave + NW * i;
      lds_ptr dst = (lds_ptr)(base + f * kFragBytes);
      if (i < ALPW) {
        const uint32_t off = ((xoff[i] + (uint32_t)kb * 64u) & xin) | (kOutOfRange & ~xin);
        __builtin_amdgcn_raw_ptr_buffer_load_lds(xr, dst, 16, off, 0, 0, 0);
      } else {
        const int g = f - BMF;
        const int m = g / BNF, ni = g % BNF;
        const uint32_t off = ((uint32_t)((ni * a.kblocks + kb) * kFragBytes + lane * 16) & win) | (kOutOfRange & ~win);
        __builtin_amdgcn_raw_ptr_buffer_load_lds(m == 0 ? wr0 : wr1, dst, 16, off, 0, 0, 0);
      }
    }
  };

  f32x4 acc[NMAT][FM][FN];
#pragma unroll
  for (int m = 0; m < NMAT; ++m)
#pragma unroll
    for (int i = 0; i < FM; ++i)
#pragma unroll
      for (int j = 0; j < FN; ++j) acc[m][i][j] = f32x4{0.f, 0.f, 0.f, 0.f};
  float ss[SSF];
  f32x4 gram[SSF];
#pragma unroll
  for (int i = 0; i < SSF; ++i) {
    ss[i] = 0.f;
    gram[i] = f32x4{0.f, 0.f, 0.f, 0.f};
  }

  // Register plan: x fragments of two consecutive k-blocks (two sets), one
  // set of W' fragments.  The MFMAs of k-block t run column by column, so the
  // first half of the W' fragments is free by mid-step: there, after the
  // barrier for k-block t+1, go the reads of t+1's x fragments and first W'
  // half plus the refill of the slot t came from; t+1's second W' half is read
  // once t's second half has been issued.  LDS latency and the barrier thus
  // hide behind matrix work instead of stalling it.
  constexpr int NB = NMAT * FN;            // W' fragments per wave and k-block
  u32x4 av[2][FM], bv[NB];
  auto read_a = [&](int r, const uint8_t* base) __attribute__((always_inline)) {
#pragma unroll
    for (int i = 0; i < FM; ++i)
      av[r][i] = *reinterpret_cast<const u32x4*>(base + (wm * FM + i) * kFragBytes + lane * 16);
  };
  auto read_b = [&](int j0, int j1, const uint8_t* base) __attribute__((always_inline)) {
#pragma unroll
    for (int j = j0; j < j1; ++j) {
      const int m = j / FN, jj = j % FN;
      bv[j] = *reinterpret_cast<const u32x4*>(base + (BMF + m * BNF + wn * FN + jj) * kFragBytes + lane * 16);
    }
  };
  auto mfma_cols = [&](int r, int j0, int j1) __attribute__((always_inline)) {
#pragma unroll
    for (int j = j0; j < j1; ++j)
#pragma unroll
      for (int i = 0; i < FM; ++i) acc[j / FN][i][j % FN] = mfma_chunk<__bf16>(av[r][i], bv[j], acc[j / FN][i][j % FN]);
  };
  auto squares = [&](int r) __attribute__((always_inline)) {
#pragma unroll
    for (int i = 0; i < FM; ++i)
      if (i / SSF == wn) {
        if (GRAM) gram[i % SSF] = mfma_chunk<__bf16>(av[r][i], av[r][i], gram[i % SSF]);
        else ss[i % SSF] += sumsq16<__bf16>(av[r][i]);
      }
  };
  // k-block t (in slot s, x operands in register set r).  Memory instructions
  // are spread between the MFMAs (scheduling groups) instead of issued in
  // bursts.  The body has no branches, so the compiler can tell the slot being
  // read from the slots still being filled and adds no wait of its own.
  auto step = [&](int s, int r, int t) __attribute__((always_inline)) {
    const uint8_t* cur = slot_ptr(s);
    const uint8_t* next = slot_ptr((s + 1) % NS);
    // first half: W' columns 0..NB/2 of t, while t's other W' half is read
    __builtin_amdgcn_sched_barrier(0);
    mfma_cols(r, 0, NB / 2);
    read_b(NB / 2, NB, cur);
#pragma unroll
    for (int g = 0; g < NB / 2; ++g) {
      __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);        // one LDS read
      __builtin_amdgcn_sched_group_barrier(0x008, FM, 0);       // FM MFMAs
    }
    __builtin_amdgcn_sched_barrier(0);
    // Every read of slot s has returned before the barrier; k-block t+1 has
    // landed for this wave once at most the NS-2 younger ones are in flight,
    // and the barrier extends both to every wave.
    __builtin_amdgcn_s_waitcnt((15) | (7 << 4) | (0 << 8) | (3 << 14));   // lgkmcnt(0)
    wait_vmcnt<(NS - 2) * LPW>();
    __builtin_amdgcn_s_barrier();
    __builtin_amdgcn_sched_barrier(0);
    // second half: t's other W' columns and squares, while t+1's x fragments
    // and first W' half are read and slot s is refilled with k-block t+NS
    read_a(r ^ 1, next);
    read_b(0, NB / 2, next);
    mfma_cols(r, NB / 2, NB);
    squares(r);
    issue(slot_ptr(s), t + NS);
#pragma unroll
    for (int g = 0; g < FM + NB / 2; ++g) {
      __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);        // one LDS read
      __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);        // one MFMA
    }
#pragma unroll
    for (int g = 0; g < LPW; ++g) {
      __builtin_amdgcn_sched_group_barrier(0x020, 1, 0);        // one global-to-LDS load
      __builtin_amdgcn_sched_group_barrier(0x008, 2, 0);        // two MFMAs
    }
    __builtin_amdgcn_sched_barrier(0);
  };

  static_assert(NS == 4, "the unrolled schedule below assumes four ring slots");
  issue(ring0, 0);
  issue(ring1, 1);
  issue(ring2, 2);
  issue(ring3, 3);
  wait_vmcnt<(NS - 1) * LPW>();
  __builtin_amdgcn_s_barrier();
  read_a(0, ring0);
  read_b(0, NB / 2, ring0);
  // k-blocks past the last one are zero-filled, so rounding the trip count up
  // to whole rounds of the ring adds only zero products.
  for (int t = 0; t < a.kblocks; t += 4) {
    step(0, 0, t);
    step(1, 1, t + 1);
    step(2, 0, t + 2);
    step(3, 1, t + 3);
  }
  wait_vmcnt<0>();   // retire the zero-filled loads issued past the last k-block

  // Sums of squares.  VALU form: lanes l, l^16, l^32, l^48 hold parts of
  // row l%16.  Gram form: the diagonal of x x^T, element l%4 of the lanes
  // whose (l%16)/4 == l/16.
#pragma unroll
  for (int i = 0; i < SSF; ++i) {
    if (GRAM) {
      if ((lrow >> 2) == lgrp) {
        const int r = lrow & 3;
        const f32x4 gv = gram[i];
        ssbuf[(wm * FM + wn * SSF + i) * 16 + lrow] = r == 0 ? gv[0] : (r == 1 ? gv[1] : (r == 2 ? gv[2] : gv[3]));
      }
    } else {
      ss[i] += __shfl_xor(ss[i], 16);
      ss[i] += __shfl_xor(ss[i], 32);
      if (lgrp == 0) ssbuf[(wm * FM + wn * SSF + i) * 16 + lrow] = ss[i];
    }
  }
  __syncthreads();

  const float kf = (float)a.K;
#pragma unroll
  for (int i = 0; i < FM; ++i) {
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      const int rl = (wm * FM + i) * 16 + 4 * lgrp + r;   // row within the tile
      const int row = m0 + rl;
      const float inv = inv_rms(ssbuf[rl], kf, a.eps);
      if constexpr (Q8) {
        // fp8 output: every lane takes part in each block maximum
#pragma unroll
        for (int j = 0; j < FN; ++j) {
          const int nb = nb0 + wn * FN + j;
          const int col = nb * 16 + lrow;
          const float v = SW ? silu_times(acc[0][i][j][r] * inv, acc[NMAT - 1][i][j][r] * inv)
                             : acc[0][i][j][r] * inv;
          store_q8(v, col < a.N, row < a.M, nb < a.nblocks, a.q + (size_t)row * a.N + col,
                   a.qs + (size_t)row * a.nblocks + nb);
        }
      } else if (row < a.M) {
        __bf16* yrow = static_cast<__bf16*>(a.y) + (size_t)row * a.N;
#pragma unroll
        for (int j = 0; j < FN; ++j) {
          const int col = (nb0 + wn * FN + j) * 16 + lrow;
          if (col < a.N) {
            const float v = SW ? silu_times(acc[0][i][j][r] * inv, acc[NMAT - 1][i][j][r] * inv)
                               : acc[0][i][j][r] * inv;
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
  bool sw;
  const char* name;
};

#define FN_PREFILL(FM, FN_, WM, WN, SW, NS, GRAM, Q8, NAME)                                                      \
  PrefillInstance {                                                                                               \
    reinterpret_cast<const void*>(&prefill_kernel<FM, FN_, WM, WN, SW, NS, GRAM, Q8>), FM, FN_, WM, WN, NS, SW, NAME \
  }

static const PrefillInstance kPrefill[] = {
    FN_PREFILL(4, 8, 4, 2, false, 4, true, false, "prefill_bf16_256x256_w4x2_s4"),
    FN_PREFILL(4, 4, 4, 2, true, 4, true, false, "prefill_swiglu_bf16_256x128_w4x2_s4"),
    FN_PREFILL(4, 4, 4, 2, true, 4, true, true, "prefill_swiglu_bf16_q8_256x128_w4x2_s4"),
};

static const PrefillInstance& pick(bool sw, bool q8 = false) { return kPrefill[q8 ? 2 : (sw ? 1 : 0)]; }

FusedPlan plan_prefill(DType dt, int64_t M, int64_t K, int64_t N, bool swiglu, bool q8) {
  (void)dt;
  (void)K;
  const PrefillInstance& d = pick(swiglu, q8);
  FusedPlan p{};
  p.kind = q8 ? 5 : 1;
  p.mf = d.fm * d.wm;
  p.nf = d.fn_ * d.wn;
  p.waves = d.wm * d.wn;
  p.grid = dim3((unsigned)ceil_div(ceil_div(N, 16), p.nf), (unsigned)ceil_div(M, 16 * p.mf), 1);
  p.block = dim3(kWave * p.waves, 1, 1);
  p.name = d.name;
  return p;
}

hipError_t launch_prefill(DType dt, const FusedPlan& p, const void* x, const void* wg, const void* wu, void* y,
                          int M, int K, int N, float eps, hipStream_t stream, uint8_t* q, float* qs) {
  if (dt != DType::BF16 || (q != nullptr && wu == nullptr)) return hipErrorInvalidValue;
  const PrefillInstance& d = pick(wu != nullptr, q != nullptr);
  PrefillArgs a;
  a.q = q;
  a.qs = qs;
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

}  // namespace fn
