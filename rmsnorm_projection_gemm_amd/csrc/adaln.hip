// AdaLN helpers: the bias rows and the gain-folded modulation table
// (offline), and the modulation pre-pass of the two-launch calls.
//
// Bias rows: bias[t][n] = sum_k shift[t][k] * W[k][n] with the
// unfolded W, accumulated in fp32 in k order.  With the modulation
// h = xhat * (1 + scale) + shift after the norm, the shift reaches the
// output as this row of biases ([FlashInfer #5521] "Fused Kernel on SM120":
// the fused FC1 call takes the AdaLN shift beside the pre-processed
// weights).  One thread per (t, n); consecutive threads read consecutive
// columns of W.
#include "fn_device.h"
#include "fn_launch.h"

namespace fn {

template <typename T>
__global__ __launch_bounds__(256) void adaln_bias_kernel(const T* __restrict__ shift, const T* __restrict__ W,
                                                         float* __restrict__ bias, int Tn, int K, int N) {
  const int64_t id = (int64_t)blockIdx.x * 256 + threadIdx.x;
  if (id >= (int64_t)Tn * N) return;
  const int t = (int)(id / N), n = (int)(id % N);
  float acc = 0.f;
  for (int k = 0; k < K; ++k) acc = fmaf(Load<T>::one(shift + (size_t)t * K + k), Load<T>::one(W + (size_t)k * N + n), acc);
  bias[id] = acc;
}

// Offline fold of the gain into the modulation table: mod[t][k] =
// g[k] * (1 + scale[t][k]), the sum and the product in fp64 and one
// rounding to fp32.  With the modulated operand rounded to bf16 for the
// matrix cores anyway, the gain goes here rather than into a rounded W', so
// each product term is rounded once.  One thread per (t, k).
template <typename T>
__global__ __launch_bounds__(256) void adaln_fold_table_kernel(const T* __restrict__ g, const T* __restrict__ scale,
                                                               float* __restrict__ mod, int64_t total, int K) {
  const int64_t id = (int64_t)blockIdx.x * 256 + threadIdx.x;
  if (id >= total) return;
  const double gk = (double)Load<T>::one(g + id % K);
  const double sv = (double)Load<T>::one(scale + id);
  mod[id] = (float)(gk * (1.0 + sv));
}

// Pre-pass of the two-launch AdaLN form, one wave per row of x: the
// modulated operand u = bf16(fp32(x * mod[idx])) (modulate8, the operand the
// one-launch kernel forms; a zero row for an index outside [0, T)) and 1/RMS
// of the raw row in fp32.  split: the operand in two bf16 parts, hi in row
// 2m and lo in row 2m+1 of u ([2M, K]; modulate8_split), for the
// projections that need the unrounded operand.  The projection then runs once on u and applies
// the deferred 1/RMS from rs, so the modulation is done once per row instead
// of once per output tile ([FlashInfer #5521] "Fused Kernel on SM120": the
// page's own AdaLN FC1 also runs as two launches).  Eight 16-byte x chunks
// per lane (and their 32-byte modulation values) are loaded before any is
// used, so each wave keeps 24 KiB of reads in flight.
__global__ __launch_bounds__(256) void adaln_modulate_kernel(const u32x4* __restrict__ x,
                                                             const u32x4* __restrict__ mod,
                                                             const int* __restrict__ idx, int T,
                                                             u32x4* __restrict__ u, float* __restrict__ rs, int M,
                                                             int K8, float k, float eps, int split) {
  const int row = blockIdx.x * 4 + (int)(threadIdx.x / kWave);
  const int lane = threadIdx.x & (kWave - 1);
  if (row >= M) return;   // whole waves only; no workgroup barrier follows
  const int t = idx[row];
  const bool tv = (unsigned)t < (unsigned)T;
  const u32x4* xr = x + (size_t)row * K8;
  const u32x4* mr = mod + (size_t)(tv ? t : 0) * K8 * 2;   // 8 fp32 values = two u32x4 per x chunk
  u32x4* ur = u + (size_t)row * K8 * (split ? 2 : 1);
  u32x4* ul = ur + K8;   // split: the lo row
  constexpr int B = 8;
  float ss = 0.f;
  for (int c0 = lane; c0 < K8; c0 += B * kWave) {
    u32x4 xv[B], ml[B], mh[B];
#pragma unroll
    for (int b = 0; b < B; ++b) {
      const int c = c0 + b * kWave;
      const bool in = c < K8;
      xv[b] = in ? xr[c] : u32x4{0u, 0u, 0u, 0u};
      ml[b] = (tv && in) ? mr[2 * c] : u32x4{0u, 0u, 0u, 0u};
      mh[b] = (tv && in) ? mr[2 * c + 1] : u32x4{0u, 0u, 0u, 0u};
    }
#pragma unroll
    for (int b = 0; b < B; ++b) {
      const int c = c0 + b * kWave;
      ss += sumsq16<__bf16>(xv[b]);
      if (c < K8) {
        if (split) {
          u32x4 hi, lo;
          modulate8_split(xv[b], ml[b], mh[b], hi, lo);
          ur[c] = hi;
          ul[c] = lo;
        } else {
          ur[c] = modulate8(xv[b], ml[b], mh[b]);
        }
      }
    }
  }
  for (int off = kWave / 2; off > 0; off >>= 1) ss += __shfl_xor(ss, off);
  if (lane == 0) rs[row] = inv_rms(ss, k, eps);
}

hipError_t launch_adaln_modulate(const void* x, const float* mod, const int* idx, int T, void* u, float* rs, int M,
                                 int K, float eps, hipStream_t stream, bool split) {
  const u32x4* xp = static_cast<const u32x4*>(x);
  const u32x4* mp = reinterpret_cast<const u32x4*>(mod);
  u32x4* up = static_cast<u32x4*>(u);
  int K8 = K / 8;
  float k = (float)K;
  int sp = split ? 1 : 0;
  void* args[] = {&xp, &mp, &idx, &T, &up, &rs, &M, &K8, &k, &eps, &sp};
  return hipLaunchKernel(reinterpret_cast<const void*>(&adaln_modulate_kernel), dim3((unsigned)ceil_div(M, 4)),
                         dim3(256), args, 0, stream);
}

hipError_t launch_adaln_fold_table(DType dt, const void* g, const void* scale, float* mod, int T, int K,
                                   hipStream_t stream) {
  int64_t total = (int64_t)T * K;
  const dim3 grid((unsigned)ceil_div(total, 256)), block(256);
  if (dt == DType::BF16) {
    const __bf16* gp = static_cast<const __bf16*>(g);
    const __bf16* sp = static_cast<const __bf16*>(scale);
    void* args[] = {&gp, &sp, &mod, &total, &K};
    return hipLaunchKernel(reinterpret_cast<const void*>(&adaln_fold_table_kernel<__bf16>), grid, block, args, 0,
                           stream);
  }
  const float* gp = static_cast<const float*>(g);
  const float* sp = static_cast<const float*>(scale);
  void* args[] = {&gp, &sp, &mod, &total, &K};
  return hipLaunchKernel(reinterpret_cast<const void*>(&adaln_fold_table_kernel<float>), grid, block, args, 0, stream);
}

hipError_t launch_adaln_bias(DType dt, const void* shift, const void* W, float* bias, int T, int K, int N,
                             hipStream_t stream) {
  const dim3 grid((unsigned)ceil_div((int64_t)T * N, 256)), block(256);
  if (dt == DType::BF16) {
    const __bf16* s = static_cast<const __bf16*>(shift);
    const __bf16* w = static_cast<const __bf16*>(W);
    void* args[] = {&s, &w, &bias, &T, &K, &N};
    return hipLaunchKernel(reinterpret_cast<const void*>(&adaln_bias_kernel<__bf16>), grid, block, args, 0, stream);
  }
  const float* s = static_cast<const float*>(shift);
  const float* w = static_cast<const float*>(W);
  void* args[] = {&s, &w, &bias, &T, &K, &N};
  return hipLaunchKernel(reinterpret_cast<const void*>(&adaln_bias_kernel<float>), grid, block, args, 0, stream);
}

}  // namespace fn
