// Measurement probes, not part of the fused path: the attainable peaks the
// roofline fractions are also reported against -- a streaming HBM read and
// an MFMA-only loop -- so that a fraction of the vendor's peak can be read
// next to a fraction of what this GPU sustains at its clocks under load.
#include "fn_device.h"
#include "fn_launch.h"

namespace fn {

// Every thread streams 16-byte chunks of the source with non-temporal loads
// over a grid-wide stride (measured: faster than cached loads, and than
// unrolling); the XOR of the words keeps the loads, and the workgroup's first
// thread writes it to sink[workgroup].
__global__ __launch_bounds__(256) void probe_read_kernel(const u32x4* __restrict__ src, int64_t n16,
                                                         uint32_t* __restrict__ sink) {
  const int64_t stride = (int64_t)gridDim.x * blockDim.x;
  u32x4 acc = {0u, 0u, 0u, 0u};
  for (int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; i < n16; i += stride)
    acc ^= __builtin_nontemporal_load(src + i);
  uint32_t v = acc[0] ^ acc[1] ^ acc[2] ^ acc[3];
  for (int off = kWave / 2; off > 0; off >>= 1) v ^= __shfl_xor(v, off);
  __shared__ uint32_t part[256 / kWave];
  if ((threadIdx.x & (kWave - 1)) == 0) part[threadIdx.x / kWave] = v;
  __syncthreads();
  if (threadIdx.x == 0) {
    uint32_t t = 0;
    for (int w = 0; w < (int)(blockDim.x / kWave); ++w) t ^= part[w];
    sink[blockIdx.x] = t;
  }
}

// Eight independent accumulator chains of v_mfma_f32_16x16x32_bf16 per wave,
// operands in registers: iters * 8 MFMAs (16384 FLOPs each) per wave, four
// waves per workgroup.  Each workgroup writes one value to sink.
__global__ __launch_bounds__(256) void probe_mfma_kernel(float* __restrict__ sink, int iters) {
  bf16x8 a, b;
#pragma unroll
  for (int i = 0; i < 8; ++i) {
    a[i] = (__bf16)(float)((threadIdx.x + i) & 7);
    b[i] = (__bf16)(float)((i - (int)threadIdx.x) & 7);
  }
  f32x4 acc[8];
#pragma unroll
  for (int j = 0; j < 8; ++j) acc[j] = f32x4{0.f, 0.f, 0.f, (float)j};
  for (int it = 0; it < iters; ++it) {
#pragma unroll
    for (int j = 0; j < 8; ++j) acc[j] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, acc[j], 0, 0, 0);
  }
  float s = 0.f;
#pragma unroll
  for (int j = 0; j < 8; ++j) s += acc[j][0] + acc[j][1] + acc[j][2] + acc[j][3];
  for (int off = kWave / 2; off > 0; off >>= 1) s += __shfl_xor(s, off);
  __shared__ float part[256 / kWave];
  if ((threadIdx.x & (kWave - 1)) == 0) part[threadIdx.x / kWave] = s;
  __syncthreads();
  if (threadIdx.x == 0) {
    float t = 0.f;
    for (int w = 0; w < (int)(blockDim.x / kWave); ++w) t += part[w];
    sink[blockIdx.x] = t;
  }
}

hipError_t launch_probe_read(const void* src, int64_t bytes, void* sink, int workgroups, hipStream_t stream) {
  const u32x4* s = static_cast<const u32x4*>(src);
  int64_t n16 = bytes / 16;
  uint32_t* out = static_cast<uint32_t*>(sink);
  void* args[] = {&s, &n16, &out};
  return hipLaunchKernel(reinterpret_cast<const void*>(&probe_read_kernel), dim3((unsigned)workgroups), dim3(256),
                         args, 0, stream);
}

hipError_t launch_probe_mfma(void* sink, int iters, int workgroups, hipStream_t stream) {
  float* out = static_cast<float*>(sink);
  void* args[] = {&out, &iters};
  return hipLaunchKernel(reinterpret_cast<const void*>(&probe_mfma_kernel), dim3((unsigned)workgroups), dim3(256),
                         args, 0, stream);
}

}  // namespace fn
