// Device-side building blocks shared by the libflashnorm kernels (gfx950).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace fn {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));

constexpr int kWave = 64;      // CDNA wavefront width
constexpr int kFragN = 16;     // output columns per packed fragment
constexpr int kFragBytes = kWave * 16;

// Per-dtype fragment geometry of the packed weight layout: each lane of a
// 1 KiB fragment holds 16 bytes = V consecutive k values of one column.
template <typename T> struct Geo;
template <> struct Geo<__bf16> {
  static constexpr int V = 8;      // values per lane
  static constexpr int KB = 32;    // k rows per fragment (4 lane groups x V)
};
template <> struct Geo<float> {
  static constexpr int V = 4;
  static constexpr int KB = 16;
};

__host__ __device__ inline int64_t ceil_div(int64_t a, int64_t b) { return (a + b - 1) / b; }

// ---- bf16 <-> fp32 -------------------------------------------------------
// Widening is exact: a bf16 value is the top half of an fp32 word.
__device__ inline float bf16_lo(uint32_t w) { return __uint_as_float(w << 16); }
__device__ inline float bf16_hi(uint32_t w) { return __uint_as_float(w & 0xffff0000u); }

// Round-to-nearest-even fp32 -> bf16 (lowers to v_cvt_pk_bf16_f32 on gfx950,
// which rounds by the default round-to-nearest-even mode).
__device__ inline uint16_t to_bf16_bits(float f) {
  __bf16 b = (__bf16)f;
  return __builtin_bit_cast(uint16_t, b);
}
__device__ inline uint32_t pack_bf16x2(float lo, float hi) {
  return (uint32_t)to_bf16_bits(lo) | ((uint32_t)to_bf16_bits(hi) << 16);
}

template <typename T> struct Store;
template <> struct Store<__bf16> {
  __device__ static inline void one(__bf16* p, float v) { *reinterpret_cast<uint16_t*>(p) = to_bf16_bits(v); }
};
template <> struct Store<float> {
  __device__ static inline void one(float* p, float v) { *p = v; }
};

template <typename T> struct Load;
template <> struct Load<__bf16> {
  __device__ static inline float one(const __bf16* p) {
    return __uint_as_float((uint32_t)(*reinterpret_cast<const uint16_t*>(p)) << 16);
  }
};
template <> struct Load<float> {
  __device__ static inline float one(const float* p) { return *p; }
};

// Sum of squares of the V values in one 16-byte lane chunk.
template <typename T> __device__ inline float sumsq16(u32x4 r);
template <> __device__ inline float sumsq16<__bf16>(u32x4 r) {
  float s = 0.f;
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    float a = bf16_lo(r[i]), b = bf16_hi(r[i]);
    s = fmaf(a, a, s);
    s = fmaf(b, b, s);
  }
  return s;
}
template <> __device__ inline float sumsq16<float>(u32x4 r) {
  float s = 0.f;
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    float a = __uint_as_float(r[i]);
    s = fmaf(a, a, s);
  }
  return s;
}

// acc(16x16 fp32) += A(16 x KB) * B(KB x 16) for one pair of 16-byte lane
// chunks.  Lane l holds row/column l%16 and k-group l/16 of each operand; the
// k ordering inside a group is the same for A and B, which is all the
// contraction needs.
template <typename T> __device__ inline f32x4 mfma_chunk(u32x4 a, u32x4 b, f32x4 acc);
template <> __device__ inline f32x4 mfma_chunk<__bf16>(u32x4 a, u32x4 b, f32x4 acc) {
  return __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8, a),
                                                 __builtin_bit_cast(bf16x8, b), acc, 0, 0, 0);
}
template <> __device__ inline f32x4 mfma_chunk<float>(u32x4 a, u32x4 b, f32x4 acc) {
#pragma unroll
  for (int v = 0; v < 4; ++v)
    acc = __builtin_amdgcn_mfma_f32_16x16x4f32(__uint_as_float(a[v]), __uint_as_float(b[v]), acc, 0, 0, 0);
  return acc;
}

// AdaLN-modulated MFMA operand: the 8 bf16 values of a 16-byte chunk times
// their 8 fp32 modulation values (the first four in mlo, the second four in
// mhi), each product rounded to fp32 and then RNE to bf16.
__device__ inline u32x4 modulate8(u32x4 x, u32x4 mlo, u32x4 mhi) {
  u32x4 r;
#pragma unroll
  for (int c = 0; c < 4; ++c) {
    const u32x4 m = c < 2 ? mlo : mhi;   // values 2c and 2c+1
    const int j = 2 * (c & 1);
    r[c] = pack_bf16x2(bf16_lo(x[c]) * __uint_as_float(m[j]), bf16_hi(x[c]) * __uint_as_float(m[j + 1]));
  }
  return r;
}

// The same operand split exactly into two bf16 parts: p = fp32(x * m),
// hi = RNE_bf16(p), lo = RNE_bf16(p - hi) (p - hi is exact in fp32), so
// hi + lo carries p to about 16 significant bits and two MFMAs against the
// same weights give the product of the unrounded operand.
__device__ inline void modulate8_split(u32x4 x, u32x4 mlo, u32x4 mhi, u32x4& hi, u32x4& lo) {
#pragma unroll
  for (int c = 0; c < 4; ++c) {
    const u32x4 m = c < 2 ? mlo : mhi;   // values 2c and 2c+1
    const int j = 2 * (c & 1);
    const float p0 = bf16_lo(x[c]) * __uint_as_float(m[j]), p1 = bf16_hi(x[c]) * __uint_as_float(m[j + 1]);
    const uint32_t h = pack_bf16x2(p0, p1);
    hi[c] = h;
    lo[c] = pack_bf16x2(p0 - bf16_lo(h), p1 - bf16_hi(h));
  }
}

// silu(a) * b = a / (1 + e^-a) * b, with the hardware exp2 and reciprocal
// (v_exp_f32, v_rcp_f32: about 1 ulp each) instead of the libm-accurate
// expf and a correctly rounded division -- a few fp32 ulps, far below the
// bf16 (or E4M3) rounding that follows, for a fraction of the instructions.
// Large negative a: e^-a overflows to inf, rcp(inf) = 0, result -0 or 0.
__device__ inline float silu_times(float a, float b) {
  const float e = __builtin_amdgcn_exp2f(a * -1.44269504088896341f);
  return a * __builtin_amdgcn_rcpf(1.0f + e) * b;
}

// 1 / sqrt(sum_sq / K + eps) in fp32: the deferred per-row scale.
__device__ inline float inv_rms(float sumsq, float k, float eps) {
  return 1.0f / sqrtf(sumsq / k + eps);
}

// ---- OCP fp8 E4M3 ----------------------------------------------------------
// Round-to-nearest-even E4M3 code of v (bias 7, 3 mantissa bits, subnormals
// on the 2^-9 grid, largest finite 448, NaN 0x7F).  Magnitudes that round
// past 448 saturate to it.
// Branch-free: in the normal range the fp32 mantissa is rounded to 3 bits
// (add 2^19 - 1 plus the lowest kept bit, ties to even; a carry moves into
// the exponent) and the exponent rebiased from 127 to 7; below 2^-6 the
// value is counted in units of 2^-9 (exact scaling, rint ties to even).
__device__ inline uint32_t e4m3_rne(float v) {
  const uint32_t bits = __float_as_uint(v);
  const uint32_t sign = (bits >> 24) & 0x80u;
  const uint32_t abits = bits & 0x7fffffffu;
  const float a = __uint_as_float(abits);
  const uint32_t rounded = abits + 0x7FFFFu + ((abits >> 20) & 1u);
  const uint32_t normal = (rounded >> 20) - (120u << 3);      // (exponent - 127 + 7) << 3 | 3 mantissa bits
  const uint32_t sub = (uint32_t)rintf(a * 512.0f);          // 0..8; 8 is the smallest normal's code
  uint32_t code = a < 0.015625f ? sub : normal;
  code = code < 0x7Eu ? code : 0x7Eu;                        // saturate at 448
  return (a != a) ? 0x7Fu : (sign | code);
}

// 16 E4M3 codes (one 16-byte lane chunk of the packed fp8 weights: the
// lane's 8 codes of each k-block of a pair) -> the lane's two bf16 B
// operands, bytes 0..7 for the first k-block and 8..15 for the second.
// v_cvt_scalef32_pk_bf16_fp8 with scale 1 decodes two codes into two bf16
// exactly (every E4M3 value is a bf16 value).
__device__ inline void e4m3x16_to_bf16(u32x4 w, u32x4& lo, u32x4& hi) {
#pragma unroll
  for (int i = 0; i < 2; ++i) {
    lo[2 * i] = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(w[i], 1.0f, false));
    lo[2 * i + 1] = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(w[i], 1.0f, true));
    hi[2 * i] = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(w[2 + i], 1.0f, false));
    hi[2 * i + 1] = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(w[2 + i], 1.0f, true));
  }
}

// Lane permutation inside each 16-lane row of the wave (DPP, no LDS).
template <int CTRL>
__device__ inline float dpp_move(float v) {
  return __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(v), CTRL, 0xF, 0xF, false));
}
// max that propagates NaN from either side
__device__ inline float nan_max(float m, float t) { return (m > t || m != m) ? m : t; }
// Maximum over the 16 lanes of a DPP row: lane ^ 1, lane ^ 2 (quad
// permutes), then the mirror within 8 lanes and within 16 lanes.
__device__ inline float row16_max(float m) {
  m = nan_max(m, dpp_move<0xB1>(m));    // quad_perm [1,0,3,2]
  m = nan_max(m, dpp_move<0x4E>(m));    // quad_perm [2,3,0,1]
  m = nan_max(m, dpp_move<0x141>(m));   // row_half_mirror
  m = nan_max(m, dpp_move<0x140>(m));   // row_mirror
  return m;
}

// fp8 output with one scale per 16-column row block.  In a 16x16
// accumulator tile lane l holds column l%16 of row 4*(l/16)+e, so the 16
// lanes sharing l/16 -- one DPP row -- hold one row's block: its largest
// magnitude is a reduction over that row (NaN propagates).  Then
// r = 448/amax and s = amax/448, both correctly rounded (r = s = 1 for an
// all-zero block), and code = RNE_E4M3(v * r).  Every lane of the wave must
// call this (cross-lane reduction); col_ok and row_ok mask what is stored,
// blk_ok says the block exists (its scale is stored by the block's lane 0).
__device__ inline void store_q8(float v, bool col_ok, bool row_ok, bool blk_ok, uint8_t* code, float* scale) {
  const float m = row16_max(col_ok ? fabsf(v) : 0.f);
  const bool zero = m == 0.f;
  const float r = zero ? 1.f : __fdiv_rn(448.f, m);
  if (row_ok && col_ok) *code = (uint8_t)e4m3_rne(v * r);
  if (row_ok && blk_ok && (threadIdx.x & 15) == 0) *scale = zero ? 1.f : __fdiv_rn(m, 448.f);
}

}  // namespace fn
