// AdaLN helpers: the bias rows (offline) and the modulation pre-pass of the
// two-launch calls.
//
// Bias rows: bias[t][n] = sum_k shift[t][k] * W[k][n] with the
// unfolded W, accumulated in fp32 in k order.  With the gain folded into W'
// and the modulation h = xhat * (1 + scale) + shift, the shift reaches the
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

// Pre-pass of the two-launch AdaLN form, one wave per row of x: the
// modulated operand u = x + x * scale[idx] (fp32, one rounding, then RNE to
// bf16 -- modulate8, the same operand the one-launch kernels form; scale 0
// for an index outside [0, T)) and 1/RMS of the raw row in fp32.  The
// projection then runs once on u and applies the deferred 1/RMS from rs, so
// the modulation is done once per row instead of once per output tile
// ([FlashInfer #5521] "Fused Kernel on SM120": the page's own AdaLN FC1 also
// runs as two launches).  Eight 16-byte chunks per lane are loaded before
// any is used (a 4096-wide row in one round trip), so each wave keeps 8 KiB
// of reads in flight.
__global__ __launch_bounds__(256) void adaln_modulate_kernel(const u32x4* __restrict__ x,
                                                             const u32x4* __restrict__ scale,
                                                             const int* __restrict__ idx, int T,
                                                             u32x4* __restrict__ u, float* __restrict__ rs, int M,
                                                             int K8, float k, float eps) {
  const int row = blockIdx.x * 4 + (int)(threadIdx.x / kWave);
  const int lane = threadIdx.x & (kWave - 1);
  if (row >= M) return;   // whole waves only; no workgroup barrier follows
  const int t = idx[row];
  const bool tv = (unsigned)t < (unsigned)T;
  const u32x4* xr = x + (size_t)row * K8;
  const u32x4* sr = scale + (size_t)(tv ? t : 0) * K8;
  u32x4* ur = u + (size_t)row * K8;
  constexpr int B = 8;
  float ss = 0.f;
  for (int c0 = lane; c0 < K8; c0 += B * kWave) {
    u32x4 xv[B], sv[B];
#pragma unroll
    for (int b = 0; b < B; ++b) {
      const int c = c0 + b * kWave;
      xv[b] = c < K8 ? xr[c] : u32x4{0u, 0u, 0u, 0u};
      sv[b] = (tv && c < K8) ? sr[c] : u32x4{0u, 0u, 0u, 0u};
    }
#pragma unroll
    for (int b = 0; b < B; ++b) {
      const int c = c0 + b * kWave;
      ss += sumsq16<__bf16>(xv[b]);
      if (c < K8) ur[c] = modulate8(xv[b], sv[b]);
    }
  }
  for (int off = kWave / 2; off > 0; off >>= 1) ss += __shfl_xor(ss, off);
  if (lane == 0) rs[row] = inv_rms(ss, k, eps);
}

hipError_t launch_adaln_modulate(const void* x, const void* scale, const int* idx, int T, void* u, float* rs, int M,
                                 int K, float eps, hipStream_t stream) {
  const u32x4* xp = static_cast<const u32x4*>(x);
  const u32x4* sp = static_cast<const u32x4*>(scale);
  u32x4* up = static_cast<u32x4*>(u);
  int K8 = K / 8;
  float k = (float)K;
  void* args[] = {&xp, &sp, &idx, &T, &up, &rs, &M, &K8, &k, &eps};
  return hipLaunchKernel(reinterpret_cast<const void*>(&adaln_modulate_kernel), dim3((unsigned)ceil_div(M, 4)),
                         dim3(256), args, 0, stream);
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
