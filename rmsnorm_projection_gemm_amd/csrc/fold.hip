// Weightless normalisation, offline ([FlashNorm digest] proposal 1): fold the
// RMSNorm gain into the projection, W'[k][n] = round(g[k] * W[k][n]), and
// write W' in the packed fragment layout the fused kernels stream.
//
// One thread writes one 16-byte lane chunk: V consecutive k of one column.
// The product is taken once in fp32 (exact for two bf16 values, correctly
// rounded for two fp32 values) and rounded once to the storage type.
#include "fn_device.h"
#include "fn_launch.h"

namespace fn {

template <typename T>
__global__ __launch_bounds__(256) void fold_kernel(const T* __restrict__ g, const T* __restrict__ W,
                                                   u32x4* __restrict__ Wp, int K, int N,
                                                   int kblocks, int64_t total_chunks) {
  constexpr int V = Geo<T>::V;
  constexpr int KB = Geo<T>::KB;
  const int64_t idx = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  if (idx >= total_chunks) return;
  const int lane = (int)(idx & (kWave - 1));
  const int64_t frag = idx / kWave;
  const int kb = (int)(frag % kblocks);
  const int nb = (int)(frag / kblocks);
  const int n = nb * kFragN + (lane & 15);
  const int k0 = kb * KB + (lane >> 4) * V;
  float v[V];
#pragma unroll
  for (int i = 0; i < V; ++i) {
    const int k = k0 + i;
    float w = 0.f;
    if (k < K && n < N) {
      w = Load<T>::one(W + (size_t)k * N + n);
      if (g != nullptr) w = Load<T>::one(g + k) * w;
    }
    v[i] = w;
  }
  u32x4 out;
  if constexpr (V == 8) {
#pragma unroll
    for (int i = 0; i < 4; ++i) out[i] = pack_bf16x2(v[2 * i], v[2 * i + 1]);
  } else {
#pragma unroll
    for (int i = 0; i < 4; ++i) out[i] = __float_as_uint(v[i]);
  }
  Wp[idx] = out;
}

hipError_t launch_fold(DType dt, const void* g, const void* W, void* W_packed, int K, int N,
                       hipStream_t stream) {
  const int kblocks = (int)ceil_div(K, k_per_block(dt));
  const int64_t nblocks = ceil_div(N, kFragN);
  const int64_t total = nblocks * kblocks * kWave;
  const dim3 block(256);
  const dim3 grid((unsigned)ceil_div(total, 256));
  u32x4* out = static_cast<u32x4*>(W_packed);
  if (dt == DType::BF16) {
    const __bf16* gp = static_cast<const __bf16*>(g);
    const __bf16* wp = static_cast<const __bf16*>(W);
    void* args[] = {&gp, &wp, &out, &K, &N, (void*)&kblocks, (void*)&total};
    return hipLaunchKernel(reinterpret_cast<const void*>(&fold_kernel<__bf16>), grid, block, args, 0, stream);
  }
  const float* gp = static_cast<const float*>(g);
  const float* wp = static_cast<const float*>(W);
  void* args[] = {&gp, &wp, &out, &K, &N, (void*)&kblocks, (void*)&total};
  return hipLaunchKernel(reinterpret_cast<const void*>(&fold_kernel<float>), grid, block, args, 0, stream);
}

}  // namespace fn
