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

__device__ inline float silu_times(float a, float b) { return a / (1.0f + expf(-a)) * b; }

// 1 / sqrt(sum_sq / K + eps) in fp32: the deferred per-row scale.
__device__ inline float inv_rms(float sumsq, float k, float eps) {
  return 1.0f / sqrtf(sumsq / k + eps);
}

}  // namespace fn
