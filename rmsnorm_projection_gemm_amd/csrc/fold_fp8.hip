// Offline fold + per-column E4M3 quantisation of the projection weights.
//
// W'[k][n] = round_dt(g[k] * W[k][n]) exactly as fold.hip computes it, then
// per output column n: amax = max_k |W'[k][n]|, r = 448 / amax, s = amax /
// 448 (both one correctly rounded fp32 division; r = s = 1 for a zero
// column) and code q[k][n] = RNE_E4M3(W'[k][n] * r) with one fp32 multiply.
// The weights then stream at one byte per element, decoded in registers
// right before the matrix product ([Fused-kernel memory hierarchy] "Fused
// 커널은 왜 3~4배 빠른가", section "트릭 2"; [FlashNorm digest], folded
// checkpoints stay valid for quantised models).
//
// One workgroup per 16-column block: pass 1 reduces the 16 column maxima,
// pass 2 writes the block's packed fragments, one 16-byte lane chunk per
// thread (the lane's 8 codes of two consecutive 32-row k-blocks).
#include "fn_device.h"
#include "fn_launch.h"

namespace fn {

// Stored folded weight as an fp32 value (zero outside the matrix).
template <typename T>
__device__ inline float folded_value(const T* g, const T* W, int k, int n, int K, int N) {
  if (k >= K || n >= N) return 0.f;
  float w = Load<T>::one(W + (size_t)k * N + n);
  if (g != nullptr) w = Load<T>::one(g + k) * w;
  if constexpr (sizeof(T) == 2) w = __uint_as_float((uint32_t)to_bf16_bits(w) << 16);
  return w;
}

template <typename T>
__global__ __launch_bounds__(256) void fold_fp8_kernel(const T* __restrict__ g, const T* __restrict__ W,
                                                       u32x4* __restrict__ W8, float* __restrict__ scales,
                                                       int K, int N, int kpairs) {
  __shared__ float part[16][17];
  __shared__ float rcol[16];
  const int t = threadIdx.x;
  const int nb = blockIdx.x;
  {
    const int c = t & 15, rg = t >> 4;
    float amax = 0.f;
    for (int k = rg; k < K; k += 16) amax = fmaxf(amax, fabsf(folded_value(g, W, k, nb * 16 + c, K, N)));
    part[rg][c] = amax;
  }
  __syncthreads();
  if (t < 16) {
    float m = 0.f;
#pragma unroll
    for (int i = 0; i < 16; ++i) m = fmaxf(m, part[i][t]);
    const bool zero = !(m > 0.f);
    rcol[t] = zero ? 1.f : __fdiv_rn(448.f, m);
    if (nb * 16 + t < N) scales[nb * 16 + t] = zero ? 1.f : __fdiv_rn(m, 448.f);
  }
  __syncthreads();
  for (int idx = t; idx < kpairs * kWave; idx += 256) {
    const int f = idx / kWave, lane = idx % kWave;
    const int col = nb * 16 + (lane & 15);
    const float r = rcol[lane & 15];
    u32x4 out = {0u, 0u, 0u, 0u};
#pragma unroll
    for (int b = 0; b < 16; ++b) {   // byte b: k-block 2f + b/8, row (lane/16)*8 + b%8 of it
      const int k = f * 64 + (b / 8) * 32 + (lane >> 4) * 8 + (b % 8);
      out[b / 4] |= e4m3_rne(folded_value(g, W, k, col, K, N) * r) << ((b % 4) * 8);
    }
    W8[(size_t)nb * kpairs * kWave + idx] = out;
  }
}

hipError_t launch_fold_fp8(DType dt, const void* g, const void* W, void* W8, float* scales, int K, int N,
                           hipStream_t stream) {
  const int kpairs = (int)ceil_div(K, 64);
  const dim3 grid((unsigned)ceil_div(N, kFragN)), block(256);
  u32x4* out = static_cast<u32x4*>(W8);
  if (dt == DType::BF16) {
    const __bf16* gp = static_cast<const __bf16*>(g);
    const __bf16* wp = static_cast<const __bf16*>(W);
    void* args[] = {&gp, &wp, &out, &scales, &K, &N, (void*)&kpairs};
    return hipLaunchKernel(reinterpret_cast<const void*>(&fold_fp8_kernel<__bf16>), grid, block, args, 0, stream);
  }
  const float* gp = static_cast<const float*>(g);
  const float* wp = static_cast<const float*>(W);
  void* args[] = {&gp, &wp, &out, &scales, &K, &N, (void*)&kpairs};
  return hipLaunchKernel(reinterpret_cast<const void*>(&fold_fp8_kernel<float>), grid, block, args, 0, stream);
}

}  // namespace fn
