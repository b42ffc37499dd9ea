// The unfused "segmented chain" the fused kernels are measured against
// ([FlashInfer #5521] "MiniMax-H3 Fused FC1 + SwiGLU", section "Segmented
// Chain"): a normalisation kernel that writes xhat to HBM, a separate GEMM
// (hipBLASLt through torch, outside this library), and for the FFN variant a
// silu_and_mul kernel over the GEMM's [M, 2N] output.  Each step writes its
// result to HBM and the next reads it back; that round trip and the extra
// launches are what the fused path removes.
#include "fn_device.h"
#include "fn_launch.h"

namespace fn {

// One workgroup per row: reduce sum(x^2), then write xhat = x * inv_rms * g,
// rounded once to T.
template <typename T>
__global__ __launch_bounds__(256) void rmsnorm_kernel(const T* __restrict__ x, const T* __restrict__ g,
                                                      T* __restrict__ xhat, int K, float eps) {
  const int row = blockIdx.x;
  const T* xr = x + (size_t)row * K;
  T* outr = xhat + (size_t)row * K;
  float s = 0.f;
  for (int k = threadIdx.x; k < K; k += blockDim.x) {
    const float v = Load<T>::one(xr + k);
    s = fmaf(v, v, s);
  }
  for (int off = kWave / 2; off > 0; off >>= 1) s += __shfl_xor(s, off);
  __shared__ float part[256 / kWave];
  const int lane = threadIdx.x & (kWave - 1), wave = threadIdx.x / kWave;
  if (lane == 0) part[wave] = s;
  __syncthreads();
  float total = 0.f;
  for (int w = 0; w < (int)(blockDim.x / kWave); ++w) total += part[w];
  const float inv = inv_rms(total, (float)K, eps);
  for (int k = threadIdx.x; k < K; k += blockDim.x)
    Store<T>::one(outr + k, Load<T>::one(xr + k) * inv * Load<T>::one(g + k));
}

// out[m][n] = silu(h[m][n]) * h[m][N + n], rounded once to T.
template <typename T>
__global__ __launch_bounds__(256) void silu_mul_kernel(const T* __restrict__ h, T* __restrict__ out,
                                                       int N, int64_t total) {
  const int64_t idx = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  if (idx >= total) return;
  const int64_t m = idx / N;
  const int n = (int)(idx - m * N);
  const T* hr = h + (size_t)m * 2 * N;
  Store<T>::one(out + idx, silu_times(Load<T>::one(hr + n), Load<T>::one(hr + N + n)));
}

hipError_t launch_rmsnorm(DType dt, const void* x, const void* g, void* xhat, int M, int K, float eps,
                          hipStream_t stream) {
  const dim3 grid((unsigned)M), block(256);
  void* args[] = {(void*)&x, (void*)&g, &xhat, &K, &eps};
  const void* fn = dt == DType::BF16 ? reinterpret_cast<const void*>(&rmsnorm_kernel<__bf16>)
                                     : reinterpret_cast<const void*>(&rmsnorm_kernel<float>);
  return hipLaunchKernel(fn, grid, block, args, 0, stream);
}

hipError_t launch_silu_mul(DType dt, const void* h, void* out, int M, int N, hipStream_t stream) {
  const int64_t total = (int64_t)M * N;
  const dim3 grid((unsigned)ceil_div(total, 256)), block(256);
  void* args[] = {(void*)&h, &out, &N, (void*)&total};
  const void* fn = dt == DType::BF16 ? reinterpret_cast<const void*>(&silu_mul_kernel<__bf16>)
                                     : reinterpret_cast<const void*>(&silu_mul_kernel<float>);
  return hipLaunchKernel(fn, grid, block, args, 0, stream);
}

}  // namespace fn
