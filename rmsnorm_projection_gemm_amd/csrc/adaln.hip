// AdaLN bias rows, offline: bias[t][n] = sum_k shift[t][k] * W[k][n] with the
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
