// Host-side launch interface between the C ABI (api.cpp) and the kernels.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace fn {

enum class DType : int { F32 = 0, BF16 = 1 };

inline int elem_bytes(DType t) { return t == DType::F32 ? 4 : 2; }
inline int k_per_block(DType t) { return t == DType::F32 ? 16 : 32; }   // KB of the packed layout

// Kernel instance chosen for one fused call.
struct FusedPlan {
  int kind;           // 0 = decode (<= 16 rows, or fp32), 1 = prefill (tiled), 2 = decode with x in LDS,
                      // 3 = fp8 weights (x in LDS, rows tiled over grid.y),
                      // 4 = SwiGLU with fp8 output (x in LDS), 5 = the same on the prefill kernel,
                      // 6 = AdaLN prologue (x and modulation rows in LDS, up to 16 rows),
                      // 8 = prefill on an operand modulated by the AdaLN pre-pass,
                      // 9 = the same on the LDS-shared-x decode kernel, 10 = the same with fp8 output,
                      // 11 = the prefill kernel with fp8 weights
  int mf;             // 16-row fragments per workgroup (decode)
  int nf;             // 16-column fragments per workgroup (decode)
  int waves;          // waves per workgroup
  dim3 grid;
  dim3 block;
  const char* name;   // static string
};

FusedPlan plan_fused(DType dt, int64_t M, int64_t K, int64_t N, bool swiglu);
FusedPlan plan_decode(DType dt, int64_t M, int64_t K, int64_t N, bool swiglu);
hipError_t launch_decode(DType dt, const FusedPlan& plan, const void* x, const void* w_gate,
                         const void* w_up, void* y, int M, int K, int N, float eps,
                         hipStream_t stream);

FusedPlan plan_decode_x(DType dt, int64_t M, int64_t K, int64_t N, bool swiglu);
hipError_t launch_decode_x(DType dt, const FusedPlan& plan, const void* x, const void* w_gate,
                           const void* w_up, void* y, int M, int K, int N, float eps,
                           hipStream_t stream);

// AdaLN prologue: h = RMSNorm_g(x) * (1 + scale[idx]) + shift[idx] before
// the projection; the gain is folded into the modulation table
// mod = g * (1 + scale) ([T, K], fp32), the weights are the plain W, and the
// shift enters as bias rows shift @ W ([T, N], fp32).
struct AdalnArgs {
  const float* mod;      // [T, K] fp32
  const int* idx;        // [M] table row of each x row
  const float* bias_g;   // [T, N]
  const float* bias_u;   // [T, N], SwiGLU only
  int T;
};

// q8: SwiGLU with fp8 output (codes q, row-block scales qs; y unused).
// ex: the prefill kernel on an operand the AdaLN pre-pass modulated (1/RMS
// per row from the pre-pass, bias rows in the epilogue).
// f8: fp8 (E4M3) weights with column scales (launch_prefill_fp8, or
// launch_prefill_premod with scales).
FusedPlan plan_prefill(DType dt, int64_t M, int64_t K, int64_t N, bool swiglu, bool q8 = false, bool ex = false,
                       bool f8 = false);
hipError_t launch_prefill_fp8(const FusedPlan& plan, const void* x, const void* wg, const float* sg, const void* wu,
                              const float* su, void* y, int M, int K, int N, float eps, hipStream_t stream,
                              uint8_t* q = nullptr, float* qs = nullptr);
hipError_t launch_prefill(DType dt, const FusedPlan& plan, const void* x, const void* w_gate,
                          const void* w_up, void* y, int M, int K, int N, float eps,
                          hipStream_t stream, uint8_t* q = nullptr, float* qs = nullptr);
// Two-launch AdaLN: the pre-pass writes u = bf16(fp32(x * mod[idx])) [M,K]
// (a zero row for an index outside the table) and rs = 1/RMS(x) [M]; the
// projection kernel then runs on u (plan from plan_prefill(..., ex = true)
// or plan_decode_premod; ad.mod unused).
// split: u is [2M, K], row 2m the bf16 operand (hi) and row 2m+1 its
// rounding remainder (lo), for the SwiGLU projections.
hipError_t launch_adaln_modulate(const void* x, const float* mod, const int* idx, int T, void* u, float* rs, int M,
                                 int K, float eps, hipStream_t stream, bool split = false);
// Offline: mod[t][k] = fp32(g[k] * (1 + scale[t][k])) computed in fp64.
hipError_t launch_adaln_fold_table(DType dt, const void* g, const void* scale, float* mod, int T, int K,
                                   hipStream_t stream);
// q, qs: SwiGLU with fp8 row-block output (y unused); sg, su: fp8 weights.
hipError_t launch_prefill_premod(const FusedPlan& plan, const void* u, const float* rs, const void* wg,
                                 const void* wu, void* y, int M, int K, int N, const AdalnArgs& ad,
                                 hipStream_t stream, uint8_t* q = nullptr, float* qs = nullptr,
                                 const float* sg = nullptr, const float* su = nullptr);
// SwiGLU with fp8 output on the pre-modulated operand (bf16 weights up to 64
// rows, fp8 weights every M).
FusedPlan plan_decode_q8_premod(bool f8_weights, int64_t M, int64_t N);
hipError_t launch_decode_q8_premod(bool f8_weights, const FusedPlan& plan, const void* u, const float* rs,
                                   const void* wg, const float* sg, const void* wu, const float* su, uint8_t* q,
                                   float* qs, int M, int K, int N, const AdalnArgs& ad, hipStream_t stream);
// bf16 weights: 17..64 rows; fp8 weights (column scales sg, su): every M.
FusedPlan plan_decode_premod(int64_t M, int64_t N, bool swiglu, bool f8 = false);
hipError_t launch_decode_premod(const FusedPlan& plan, const void* u, const float* rs, const void* wg,
                                const float* sg, const void* wu, const float* su, void* y, int M, int K, int N,
                                const AdalnArgs& ad, hipStream_t stream);

// Grouped launch of independent calls of at most 16 rows, all with bf16
// weights or all with fp8 weights (sg, su: column scales): one one-wave
// workgroup per grouped_blocks() column blocks of every call.  calls:
// device array of grouped_call_bytes() records (grouped_call_fill on the
// host, then copied; first = the call's first workgroup); item_call: device
// array [items] of uint16 call indices.
constexpr int kGroupedBlocks = 2;            // bf16 weights
constexpr int kGroupedBlocksFp8 = 2;         // fp8 weights, projection
constexpr int kGroupedBlocksFp8Swiglu = 2;   // fp8 weights, gate/up pair
constexpr int kGroupedPairsFp8 = 4;          // fp8: k-block pairs per stage
inline int grouped_blocks(bool fp8, bool swiglu) {
  return fp8 ? (swiglu ? kGroupedBlocksFp8Swiglu : kGroupedBlocksFp8) : kGroupedBlocks;
}
size_t grouped_call_bytes();
void grouped_call_fill(void* dst, const void* x, const void* wg, const void* wu, const float* sg, const float* su,
                       void* y, int M, int K, int N, float eps, int first);
hipError_t launch_decode_grouped(const void* calls, const void* item_call, int items, bool fp8, hipStream_t stream);
// The same for steps with calls of 17..64 rows (decode_x.hip): every call in
// workgroups of kGroupedXWaves waves of kGroupedXCols column blocks each,
// sharing x through LDS, kGroupedXStage k-blocks per stage;
// grouped_x_call_bytes() records.
constexpr int kGroupedXWaves = 12;
constexpr int kGroupedXCols = 1;
constexpr int kGroupedXStage = 2;
constexpr int kGroupedXBlocks = kGroupedXWaves * kGroupedXCols;   // column blocks per workgroup
size_t grouped_x_call_bytes();
void grouped_x_call_fill(void* dst, const void* x, const void* wg, const void* wu, const float* sg, const float* su,
                         void* y, int M, int K, int N, float eps, int first);
hipError_t launch_decode_x_grouped(const void* calls, const void* item_call, int items, bool fp8,
                                   hipStream_t stream);

hipError_t launch_fold(DType dt, const void* g, const void* W, void* W_packed,
                       int K, int N, hipStream_t stream);

// fp8 (E4M3) weights: fold + quantise, and the fused calls (bf16 activations).
hipError_t launch_fold_fp8(DType dt, const void* g, const void* W, void* W8, float* scales,
                           int K, int N, hipStream_t stream);
FusedPlan plan_fp8(int64_t M, int64_t K, int64_t N, bool swiglu);
hipError_t launch_fp8(const FusedPlan& plan, const void* x, const void* wg, const float* sg,
                      const void* wu, const float* su, void* y, int M, int K, int N, float eps,
                      hipStream_t stream);
// Narrow projections at up to 16 rows with fp8 weights: the register-x tile
// with its k range split over waves (decode.hip); 0 when the call is not
// such a case, else the waves per column block.
int fp8_k_split(int64_t M, int64_t N, bool swiglu);
FusedPlan plan_fp8_ksplit(int64_t M, int64_t N, bool swiglu);
hipError_t launch_fp8_ksplit(const FusedPlan& plan, const void* x, const void* wg, const float* sg,
                             const void* wu, const float* su, void* y, int M, int K, int N, float eps,
                             hipStream_t stream);

// SwiGLU with fp8 output (E4M3 codes, one scale per 16-column row block):
// the LDS-shared-x decode kernel (bf16 weights up to 64 rows, fp8 weights
// any M).
FusedPlan plan_decode_q8(bool f8_weights, int64_t M, int64_t N);
hipError_t launch_decode_q8(bool f8_weights, const FusedPlan& plan, const void* x, const void* wg,
                            const float* sg, const void* wu, const float* su, uint8_t* q, float* qs,
                            int M, int K, int N, float eps, hipStream_t stream);

// One-launch AdaLN, up to 16 rows.
FusedPlan plan_adaln(int64_t M, int64_t N, bool swiglu);
hipError_t launch_adaln(const FusedPlan& plan, const void* x, const void* wg, const void* wu, void* y, int M,
                        int K, int N, float eps, const AdalnArgs& ad, hipStream_t stream);
// Measurement probes (a streaming read, an MFMA-only loop).
hipError_t launch_probe_read(const void* src, int64_t bytes, void* sink, int workgroups, hipStream_t stream);
hipError_t launch_probe_mfma(void* sink, int iters, int workgroups, hipStream_t stream);

hipError_t launch_adaln_bias(DType dt, const void* shift, const void* W, float* bias, int T, int K, int N,
                             hipStream_t stream);

hipError_t launch_fused(DType dt, const FusedPlan& plan, const void* x,
                        const void* w_gate, const void* w_up, void* y,
                        int M, int K, int N, float eps, hipStream_t stream);

hipError_t launch_rmsnorm(DType dt, const void* x, const void* g, void* xhat,
                          int M, int K, float eps, hipStream_t stream);

hipError_t launch_silu_mul(DType dt, const void* h, void* out, int M, int N,
                           hipStream_t stream);

}  // namespace fn
