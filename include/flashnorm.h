/*
 * libflashnorm: fused RMSNorm + linear projection for AMD Instinct MI355X
 * (gfx950), after FlashNorm.
 *
 * The method ([FlashNorm digest] "RMS norm는 연산량 1할인데 왜 33번 호출로
 * 속도를 갉아먹나", news.juniverse.app, summary bullets proposal 1-3):
 *   - weightless normalisation: the RMSNorm gain g is folded offline into the
 *     projection, W' = diag(g) * W, so the run-time norm has no weights;
 *   - deferred normalisation: the per-row division by RMS(x) moves after the
 *     product, y = (x * W') / RMS(x), so the sum of squares (vector units)
 *     and the contraction (matrix units) proceed together.
 * With RMS(x) = sqrt(mean_k x^2 + eps), the result equals the unfolded
 * definition y = (x / RMS(x) * g) * W.  The SwiGLU variant
 * ([FlashInfer #5521] "MiniMax-H3 Fused FC1 + SwiGLU", section "Design",
 * register-level SwiGLU) computes silu(a) * b with a and b the normalised
 * gate and up projections, applied to the accumulators before the store.
 *
 * Conventions shared by every entry point
 * ---------------------------------------
 * Memory:   every data pointer is device memory owned by the caller.  The
 *           library allocates nothing, frees nothing and never synchronises;
 *           each call enqueues its work on `stream` (0 = the null stream)
 *           and returns.  Results are ready when the stream reaches them.
 *           Exceptions, each stated at its declaration: creating a recorded
 *           or grouped step allocates (and copies its call table
 *           synchronously), and fn_norm_proj_swiglu_adaln_static works in
 *           the library's own static device array.
 * Layouts:  x[M,K], y[M,N], W[K,N] are dense row-major (leading dimensions
 *           K, N and N).  g[K] is a vector.  All tensors of one call share
 *           the storage dtype `dt`; y and out use it too.
 * Packed weights: the folded weights W' live in the library's packed,
 *           fragment-major layout (fn_fold_weights writes it, the fused
 *           calls read it).  With e the element size, V = 16/e values per
 *           lane (8 for bf16, 4 for fp32) and KB = 4*V rows per k-block
 *           (32 for bf16, 16 for fp32), element W'[k][n] sits at byte
 *             (((n/16) * ceil(K/KB) + k/KB) * 64 + ((k%KB)/V) * 16 + n%16) * 16
 *               + (k%V) * e
 *           and padding elements (k >= K or n >= N) are zero.  Its size is
 *           fn_packed_weight_bytes(K, N, dt).
 * Rounding: sums of squares and products accumulate in fp32.  A bf16 result
 *           is rounded once, to nearest with ties to even, from the fp32
 *           value ([FlashInfer #4040] "Fused SwiGLU 및 NVFP4 양자화", section
 *           "하드웨어 최적화"; [FlashInfer #5668] "Kimi-K3 TP12 LatentMoE
 *           Tail", round once after an fp32 sum).
 * Errors:   arguments are checked before any HIP call; on failure nothing is
 *           enqueued and a status other than FN_OK is returned, with detail
 *           in fn_last_error() (per thread).  Launch failures return
 *           FN_ERR_HIP.  No C++ exception crosses this interface.
 * Limits:   1 <= K <= 2^20 with K % 8 == 0; 0 <= M <= 2^22; 0 <= N <= 2^24.
 *           M == 0 or N == 0 is a valid empty call: nothing is launched and
 *           no pointer is read.  x, W', y, out must be 16-byte aligned; g, W
 *           and h (the unfused helpers) need the alignment of their dtype.
 *           eps must be finite and >= 0.  An output may not overlap an input.
 * Threads:  the library holds no state between calls beyond the per-thread
 *           error text (and the static array of the no-allocation call);
 *           calls on different streams may run concurrently.
 */
#ifndef FLASHNORM_H
#define FLASHNORM_H

#include <stddef.h>
#include <stdint.h>
#include <hip/hip_runtime_api.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum fn_status {
  FN_OK = 0,
  FN_ERR_NULL = 1,   /* a required pointer is NULL                        */
  FN_ERR_SHAPE = 2,  /* M, K or N outside the limits above                 */
  FN_ERR_ALIGN = 3,  /* a pointer lacks the required alignment             */
  FN_ERR_DTYPE = 4,  /* dt is not a member of fn_dtype                     */
  FN_ERR_EPS = 5,    /* eps is negative, NaN or infinite                   */
  FN_ERR_ALIAS = 6,  /* an output buffer overlaps an input buffer          */
  FN_ERR_HIP = 7,    /* the HIP runtime rejected a launch                  */
  FN_ERR_WORKSPACE = 8 /* a caller workspace is NULL, misaligned or short */
} fn_status;

typedef enum fn_dtype {
  FN_F32 = 0,        /* IEEE binary32                                      */
  FN_BF16 = 1        /* bfloat16 (8 significant bits, fp32 exponent range) */
} fn_dtype;

/* Bytes of the packed folded weights for a [K,N] matrix; 0 if K, N or dt is
 * outside the limits. */
size_t fn_packed_weight_bytes(int64_t K, int64_t N, fn_dtype dt);

/* Weightless normalisation, offline ([FlashNorm digest] proposal 1):
 *   W'[k][n] = round_dt(g[k] * W[k][n])
 * computed as one fp32 product (exact for bf16 operands; the correctly
 * rounded product for fp32) rounded once to dt, written in the packed layout.
 * g:        [K] device vector, or NULL to pack W unchanged (W' = W).
 * W:        [K,N] row-major device matrix.
 * W_packed: device buffer of fn_packed_weight_bytes(K, N, dt) bytes, fully
 *           overwritten (padding included).  Must not overlap g or W.
 * Not on the per-token path: run once per weight matrix. */
fn_status fn_fold_weights(const void* g, const void* W, void* W_packed,
                          int64_t K, int64_t N, fn_dtype dt, hipStream_t stream);

/* Fused RMSNorm + projection, one launch ([FlashNorm digest] proposals 1-2):
 *   y[m][n] = round_dt( (sum_k x[m][k] * W'[k][n]) / sqrt(sum_k x[m][k]^2 / K + eps) )
 * x:        [M,K] row-major.
 * W_packed: folded weights from fn_fold_weights for this K and N.
 * y:        [M,N] row-major output, fully overwritten.
 * eps:      added to the mean square inside the root.
 * Rows are independent: a non-finite value in row m affects row m only. */
fn_status fn_norm_proj(const void* x, const void* W_packed, void* y,
                       int64_t M, int64_t K, int64_t N, float eps,
                       fn_dtype dt, hipStream_t stream);

/* Fused RMSNorm + gate/up projections + SwiGLU, one launch
 * ([FlashNorm digest] proposals 1-2; [FlashInfer #5521] section "Design",
 * register-level SwiGLU):
 *   a = (x * W'_gate)[m][n] / r[m],  b = (x * W'_up)[m][n] / r[m],
 *   out[m][n] = round_dt( a / (1 + exp(-a)) * b ),
 *   r[m] = sqrt(sum_k x[m][k]^2 / K + eps).
 * The 1/r factor reaches a and b before the SiLU (it cannot be moved past a
 * nonlinearity).  W_gate_packed and W_up_packed are two packed [K,N]
 * matrices; out is [M,N] row-major. */
fn_status fn_norm_proj_swiglu(const void* x, const void* W_gate_packed,
                              const void* W_up_packed, void* out,
                              int64_t M, int64_t K, int64_t N, float eps,
                              fn_dtype dt, hipStream_t stream);

/* Unfused baseline, step 1 of the segmented chain ([FlashInfer #5521],
 * section "Segmented Chain"): xhat[m][k] = round_dt(x[m][k] / r[m] * g[k]),
 * written to HBM for a following GEMM.  x, xhat: [M,K]; g: [K]. */
fn_status fn_rmsnorm(const void* x, const void* g, void* xhat,
                     int64_t M, int64_t K, float eps, fn_dtype dt,
                     hipStream_t stream);

/* Unfused baseline, last step of the segmented chain (silu_and_mul over a
 * [M, 2N] product whose first N columns are the gate and last N the up
 * projection): out[m][n] = round_dt(silu(h[m][n]) * h[m][N + n]).
 * h: [M, 2N] row-major; out: [M, N].  K is not involved (pass any valid
 * shape: only M and N are checked, with N >= 1 and M >= 0). */
fn_status fn_silu_mul(const void* h, void* out, int64_t M, int64_t N,
                      fn_dtype dt, hipStream_t stream);

/* Measurement probes, not part of the method: the attainable peaks that
 * roofline fractions are also reported against (a fraction of the vendor
 * peak and a fraction of what this GPU sustains).
 *
 * fn_probe_hbm_read: `workgroups` workgroups of 256 threads stream all of
 * [src, src + bytes) once with 16-byte loads and write one 32-bit XOR of
 * what they read to sink[w] (sink: workgroups x 4 bytes, caller-owned
 * device memory).  bytes must be a multiple of 16 and src 16-byte aligned;
 * 1 <= workgroups <= 65536.  Bytes read per call = bytes.
 *
 * fn_probe_mfma_bf16: `workgroups` workgroups of four waves; every wave runs
 * iters x 8 v_mfma_f32_16x16x32_bf16 on register operands (eight
 * independent accumulator chains) and each workgroup writes one float to
 * sink[w] (workgroups x 4 bytes).  FLOPs per call = workgroups * iters *
 * 524288.  1 <= iters <= 2^20, 1 <= workgroups <= 65536.
 *
 * Both enqueue one launch on `stream`; errors: FN_ERR_NULL, FN_ERR_ALIGN,
 * FN_ERR_SHAPE (sizes out of range), FN_ERR_HIP. */
fn_status fn_probe_hbm_read(const void* src, int64_t bytes, void* sink,
                            int64_t workgroups, hipStream_t stream);
fn_status fn_probe_mfma_bf16(void* sink, int64_t iters, int64_t workgroups,
                             hipStream_t stream);

/* ---------------------------------------------------------------------------
 * fp8 weights (E4M3, one scale per output column)
 *
 * Folded checkpoints stay valid for quantised models ([FlashNorm digest],
 * compatibility bullet); the pages' fused FC1 + SwiGLU kernel has an FP8
 * variant ([FlashInfer #5521], results, "FP8 Variant"), and low-precision
 * weights are decoded in registers right before the matrix product
 * ([Fused-kernel memory hierarchy] "Fused 커널은 왜 3~4배 빠른가", section
 * "트릭 2").  Reading taken here: the folded, stored W' (as fn_fold_weights
 * computes it in dt) is quantised per output column to OCP FP8 E4M3
 * (1 sign, 4 exponent bits with bias 7, 3 mantissa bits, subnormals, largest
 * finite 448), with every step one IEEE fp32 operation:
 *   amax[n] = max_k |W'[k][n]|,  r[n] = 448 / amax[n],  s[n] = amax[n] / 448
 *   (r = s = 1 for an all-zero column),
 *   q[k][n] = RNE_E4M3(W'[k][n] * r[n])   (ties to even, saturating at 448).
 * The fused calls then compute, in fp32,
 *   y[m][n] = round_bf16( s[n] * (sum_k x[m][k] * q[k][n]) / RMS(x[m]) )
 * decoding q exactly (every E4M3 value is a bf16 value).  Only bf16
 * activations (x, y, out) are supported.
 *
 * Packed fp8 layout: fragment-major 1 KiB fragments of 16 columns x 64 rows;
 * code q[k][n] sits at byte
 *   (((n/16) * ceil(K/64) + k/64) * 64 + ((k%32)/8) * 16 + n%16) * 16
 *     + (k%64 >= 32 ? 8 : 0) + k%8
 * so one 16-byte lane load carries the lane's 8 values of two consecutive
 * 32-row k-blocks.  Padding codes (k >= K or n >= N) are zero.  Weights must
 * be finite; the codes of a column holding a NaN or an infinity are
 * unspecified.
 * ------------------------------------------------------------------------- */

/* Bytes of the packed fp8 weights for a [K,N] matrix; 0 if K or N is
 * outside the limits. */
size_t fn_packed_fp8_bytes(int64_t K, int64_t N);

/* Fold (as fn_fold_weights, in dt), then quantise per column as above.
 * g:         [K] device vector in dt, or NULL (W' = W).
 * W:         [K,N] row-major device matrix in dt (FN_BF16 or FN_F32).
 * W8_packed: device buffer of fn_packed_fp8_bytes(K, N) bytes, fully
 *            overwritten (padding included).
 * scales:    device buffer of N floats, receives s[n].
 * The outputs may not overlap g, W or each other.  Offline, once per
 * weight matrix. */
fn_status fn_fold_weights_fp8(const void* g, const void* W, void* W8_packed, float* scales,
                              int64_t K, int64_t N, fn_dtype dt, hipStream_t stream);

/* Fused RMSNorm + projection with fp8 weights, one launch:
 *   y[m][n] = round_bf16( s[n] * (sum_k x[m][k] * q[k][n]) / sqrt(sum_k x[m][k]^2 / K + eps) )
 * x: [M,K] bf16; W8_packed, scales: from fn_fold_weights_fp8 for this K, N;
 * y: [M,N] bf16, fully overwritten.  scales must be 4-byte aligned.
 * Instances: the LDS-shared-x decode kernel up to 64 rows (up to 256 on
 * projections of at least 512 column blocks, the row blocks tiled), the
 * prefill kernel with fp8 weights above (the codes decoded exactly to bf16
 * operands inside the k loop). */
fn_status fn_norm_proj_fp8(const void* x, const void* W8_packed, const float* scales, void* y,
                           int64_t M, int64_t K, int64_t N, float eps, hipStream_t stream);

/* Fused RMSNorm + gate/up projections + SwiGLU with fp8 weights:
 *   a = s_gate[n] (x * q_gate)[m][n] / r[m],  b = s_up[n] (x * q_up)[m][n] / r[m],
 *   out[m][n] = round_bf16( a / (1 + exp(-a)) * b ). */
fn_status fn_norm_proj_swiglu_fp8(const void* x, const void* W8_gate, const float* s_gate,
                                  const void* W8_up, const float* s_up, void* out,
                                  int64_t M, int64_t K, int64_t N, float eps, hipStream_t stream);

/* Name of the kernel instance fn_norm_proj_fp8 (swiglu == 0) or
 * fn_norm_proj_swiglu_fp8 (swiglu != 0) would launch for this shape; a
 * static string, "invalid" for bad shapes. */
const char* fn_kernel_name_fp8(int64_t M, int64_t K, int64_t N, int swiglu);

/* Name of the kernel instance fn_norm_proj (swiglu == 0) or
 * fn_norm_proj_swiglu (swiglu != 0) would launch for this shape, e.g.
 * "decode_bf16_m16_n1_w4"; a static string, "invalid" for bad shapes. */
const char* fn_kernel_name(int64_t M, int64_t K, int64_t N, int swiglu, fn_dtype dt);

/* ---------------------------------------------------------------------------
 * SwiGLU with fp8 output (E4M3 codes, one scale per 16-column row block)
 *
 * The SwiGLU result quantised where it is computed, so the next projection
 * (the down projection) reads one byte per value and nothing else is
 * written ([FlashInfer #4040] "Fused SwiGLU 및 NVFP4 양자화 최적화 분석",
 * sections "들어가며" and "Fused Kernel 구현": the activation quantised in
 * registers, one scale factor per vector of consecutive values).  Reading
 * taken here (the page's format is NVFP4): OCP E4M3 codes as in the fp8
 * weight section, blocks of 16 consecutive columns of one row (the last
 * block of a row is shorter when N % 16 != 0); per block, from the fp32
 * values v = silu(a) * b of the fused call,
 *   amax = max |v|,  r = 448 / amax,  s = amax / 448   (one correctly
 *   rounded fp32 division each; r = s = 1 for an all-zero block),
 *   code = RNE_E4M3(v * r)   (one fp32 multiply; ties to even, saturating),
 * and a consumer reads back s * decode(code).  A NaN in a block makes its
 * scale and all its codes NaN (0x7F).
 * out_codes:  [M,N] row-major bytes, fully overwritten (no alignment needed).
 * out_scales: [M, ceil(N/16)] row-major fp32, 4-byte aligned, fully
 *             overwritten.
 * x is bf16.  Instances: the LDS-shared-x decode kernel up to 64 rows (on
 * projections of at least 512 column blocks up to 128 rows with bf16
 * weights and 256 with fp8, 64-row blocks tiled), the prefill kernel above
 * (bf16 or fp8 weights).
 * ------------------------------------------------------------------------- */

/* bf16 packed weights (fn_fold_weights with FN_BF16). */
fn_status fn_norm_proj_swiglu_q8(const void* x, const void* W_gate_packed, const void* W_up_packed, void* out_codes,
                                 float* out_scales, int64_t M, int64_t K, int64_t N, float eps, hipStream_t stream);

/* fp8 weights (fn_fold_weights_fp8): fp8 in, fp8 out. */
fn_status fn_norm_proj_swiglu_fp8_q8(const void* x, const void* W8_gate, const float* s_gate, const void* W8_up,
                                     const float* s_up, void* out_codes, float* out_scales, int64_t M, int64_t K,
                                     int64_t N, float eps, hipStream_t stream);

/* Kernel instance the two calls above would launch (fp8_weights selects
 * the second); "invalid" for bad shapes. */
const char* fn_kernel_name_q8(int64_t M, int64_t K, int64_t N, int fp8_weights);

/* ---------------------------------------------------------------------------
 * AdaLN prologue (adaptive-norm modulation after the RMSNorm)
 *
 * The diffusion FC1 of [FlashInfer #5521] ("MiniMax-H3 Fused FC1 + SwiGLU",
 * sections "Segmented Chain" and "Fused Kernel on SM120") runs RMSNorm +
 * AdaLN before the projection, and its fused call takes raw x, the norm
 * weight, an AdaLN scale and shift and a per-input index into them.  The
 * page does not write the modulation; the reading taken here:
 *   h[m][k] = RMSNorm_g(x)[m][k] * (1 + scale[idx[m]][k]) + shift[idx[m]][k]
 *   y = h * W,  or  out = silu(h * W_gate) * (h * W_up).
 * The modulation is picked at run time, so it cannot be folded into the
 * weights.  The gain still folds offline ([FlashNorm digest] proposal 1),
 * here into the modulation table rather than into W: the matrix-core
 * operand x * (1 + scale) has to be rounded to bf16 anyway, and a rounded
 * W' as well would round every product term twice.  So the AdaLN calls take
 *   mod[t][k] = g[k] * (1 + scale[t][k])   (fn_adaln_fold_table, fp32)
 *   the plain weights W, packed by fn_fold_weights with g = NULL (or
 *     quantised by fn_fold_weights_fp8 with g = NULL),
 *   bias[t] = shift[t] * W                  (fn_adaln_shift_bias, fp32)
 * and compute, with RMS(x) of the unmodulated x,
 *   y[m] = ((x[m] * mod[idx[m]]) * W) / RMS(x[m]) + bias[idx[m]].
 * Arithmetic: the operand x * mod is formed in fp32 and rounded once (RNE)
 * to bf16 for the matrix cores (the one rounding a bf16 W' has in the plain
 * path); sums in fp32; bf16 output rounded once.  bf16 only.
 * mod: [T,K] fp32, 16-byte aligned.  idx: [M] int32, 4-byte aligned; an
 * index outside [0, T) selects no table row: that row's h is 0 (its output
 * is 0).  bias: [T,N] fp32, 4-byte aligned.  T >= 1 and T*K*4 < 2^31.
 * ------------------------------------------------------------------------- */

/* mod[t][k] = fp32(g[k] * (1 + scale[t][k])), the sum and product taken in
 * fp64 and rounded once.  g: [K], scale: [T,K] row-major, both in dt with
 * their element alignment; mod: [T,K] fp32, 4-byte aligned (the AdaLN calls
 * need 16), overwritten, overlapping neither input.  Offline, once per
 * table.  Errors: FN_ERR_DTYPE, FN_ERR_SHAPE (K % 8, T*K*4 >= 2^31),
 * FN_ERR_NULL, FN_ERR_ALIGN, FN_ERR_ALIAS, FN_ERR_HIP. */
fn_status fn_adaln_fold_table(const void* g, const void* scale, float* mod, int64_t T, int64_t K, fn_dtype dt,
                              hipStream_t stream);

/* bias[t][n] = sum_k shift[t][k] * W[k][n] in fp32 (k in order).  shift:
 * [T,K], W: [K,N] row-major (unfolded), both in dt; bias: [T,N] fp32,
 * overwritten.  Offline, once per table and weight matrix.  T*N < 2^31. */
fn_status fn_adaln_shift_bias(const void* shift, const void* W, float* bias, int64_t T, int64_t K, int64_t N,
                              fn_dtype dt, hipStream_t stream);

/* Fused RMSNorm + AdaLN + projection, one launch (bf16), for M <= 16: the
 * LDS-shared-x decode kernel with one modulation-table row per x row loaded
 * beside x and the operand modulated in registers.  More rows return
 * FN_ERR_SHAPE: the two-launch calls below serve them, faster than one
 * launch would (the modulation is done once per row instead of once per
 * output tile). */
fn_status fn_norm_proj_adaln(const void* x, const float* mod, const int* idx, const void* W_packed, const float* bias,
                             void* y, int64_t M, int64_t K, int64_t N, int64_t T, float eps, hipStream_t stream);

/* Fused RMSNorm + AdaLN + gate/up projections + SwiGLU, one launch (bf16),
 * M <= 16 as above. */
fn_status fn_norm_proj_swiglu_adaln(const void* x, const float* mod, const int* idx, const void* W_gate_packed,
                                    const float* bias_gate, const void* W_up_packed, const float* bias_up, void* out,
                                    int64_t M, int64_t K, int64_t N, int64_t T, float eps, hipStream_t stream);

/* Kernel instance of the two one-launch AdaLN calls; "invalid" for bad
 * shapes and for M > 16. */
const char* fn_kernel_name_adaln(int64_t M, int64_t K, int64_t N, int64_t T, int swiglu);

/* Two-launch form of the two AdaLN calls above, any M.  A pre-pass
 * (fn_adaln_modulate below) writes the modulated operand and 1/RMS of each
 * raw row into a caller workspace; the plain projection kernel of the row
 * count (the LDS-shared-x decode kernel up to 64 rows -- up to 128 rows,
 * 64-row blocks tiled, on projections of at least 512 column blocks except
 * for the SwiGLU pair -- the prefill kernel above) then projects that
 * operand and applies the deferred 1/RMS and the bias rows in its
 * epilogue.  The modulation is done once per row, and any T is served.  The
 * page's own AdaLN FC1 kernel runs as two launches as well ([FlashInfer
 * #5521] "Fused Kernel on SM120").  Same arithmetic and
 * arguments as fn_norm_proj_adaln / fn_norm_proj_swiglu_adaln, plus:
 * workspace: device memory of at least fn_adaln_workspace_bytes(M, K)
 *   bytes, 256-byte aligned, overlapping no other argument.  The call writes
 *   it and reads it back in stream order; its contents afterwards are
 *   unspecified, and calls in flight at the same time need separate
 *   workspaces.  With the workspace given the calls allocate nothing, so a
 *   caller may capture them into a HIP graph.  For M <= 16 the call is the
 *   one-launch call (the workspace is not touched and may be NULL, with
 *   workspace_bytes 0).
 * Errors as the one-launch calls (without their row limit), plus
 * FN_ERR_WORKSPACE (M > 16 and the workspace NULL, misaligned or smaller
 * than needed) and FN_ERR_ALIAS (the workspace overlaps an argument). */
fn_status fn_norm_proj_adaln_ws(const void* x, const float* mod, const int* idx, const void* W_packed,
                                const float* bias, void* y, int64_t M, int64_t K, int64_t N, int64_t T, float eps,
                                void* workspace, int64_t workspace_bytes, hipStream_t stream);
fn_status fn_norm_proj_swiglu_adaln_ws(const void* x, const float* mod, const int* idx, const void* W_gate_packed,
                                       const float* bias_gate, const void* W_up_packed, const float* bias_up,
                                       void* out, int64_t M, int64_t K, int64_t N, int64_t T, float eps,
                                       void* workspace, int64_t workspace_bytes, hipStream_t stream);

/* fn_norm_proj_swiglu_adaln_ws without a workspace argument, for callers
 * that cannot allocate device memory (code under HIP graph capture, tight
 * serving loops, harnesses that forbid hipMalloc): the call's workspace is
 * a device array of this library's own, fn_norm_proj_swiglu_adaln_static_max_bytes()
 * bytes (64 MiB + 64 KiB) on each GPU the library runs on, held until the
 * process ends; the call allocates and frees nothing.  Arguments, arithmetic
 * and results are those of fn_norm_proj_swiglu_adaln_ws (bit for bit: the
 * same kernels).  Calls whose workspace would exceed the array
 * (fn_adaln_workspace_bytes(M, K) > the maximum, e.g. M * K > 2^24) return
 * FN_ERR_SHAPE before any HIP call.  Every call on one GPU shares that GPU's
 * array, so calls that overlap in time on one GPU (on different streams,
 * or from different threads) race and must not be issued; calls on
 * different GPUs do not interact.  M <= 16 uses no scratch (one launch). */
fn_status fn_norm_proj_swiglu_adaln_static(const void* x, const float* mod, const int* idx, const void* W_gate_packed,
                                           const float* bias_gate, const void* W_up_packed, const float* bias_up,
                                           void* out, int64_t M, int64_t K, int64_t N, int64_t T, float eps,
                                           hipStream_t stream);
int64_t fn_norm_proj_swiglu_adaln_static_max_bytes(void);

/* Workspace bytes the two calls above need: the operand and one fp32 per
 * row, each rounded up to 256 bytes; 0 when M <= 16 (one launch) or when M
 * or K is outside the limits.  The SwiGLU call multiplies the operand split
 * in two bf16 parts (the rounded product and its remainder, 2*M*K bf16) with
 * the same weights, so that its two products are those of the unrounded
 * operand: the SiLU times up of two once-rounded products has no margin
 * left against the bf16 tolerance at prefill sizes, the projection (M*K
 * bf16, one rounding per term) has.  The size returned is the split one,
 * enough for either call. */
int64_t fn_adaln_workspace_bytes(int64_t M, int64_t K);

/* Projection kernel instance of the two-launch calls (their one-launch
 * kernel for M <= 16); "invalid" for bad shapes. */
const char* fn_kernel_name_adaln_ws(int64_t M, int64_t K, int64_t N, int64_t T, int swiglu);

/* AdaLN with fp8 weights (fn_fold_weights_fp8 of the plain W, g = NULL:
 * E4M3 codes, one scale per output column), in two launches for every M:
 * the pre-pass above, then the fp8-weight kernel of the row count on the
 * modulated operand (decode up to 64 rows -- on projections of at least
 * 512 column blocks up to 256, 128 for the SwiGLU pair, 64-row blocks
 * tiled -- prefill above), with
 *   y[m] = s * (u[m] * q) / RMS(x[m]) + bias[idx[m]].
 * The pages' AdaLN FC1 kernel is an fp8 kernel with pre-processed weights
 * and scales ([FlashInfer #5521] "Fused Kernel on SM120").  bias rows come
 * from fn_adaln_shift_bias on the bf16 W.  Arguments as fn_norm_proj_fp8 /
 * fn_norm_proj_swiglu_fp8 plus mod, idx, bias and T as in the AdaLN calls
 * above; workspace: at least fn_adaln_prepass_bytes(M, K) bytes, 256-byte
 * aligned, overlapping no other argument (always needed).  Errors as the
 * calls above. */
fn_status fn_norm_proj_adaln_fp8_ws(const void* x, const float* mod, const int* idx, const void* W8_packed,
                                    const float* scales, const float* bias, void* y, int64_t M, int64_t K, int64_t N,
                                    int64_t T, float eps, void* workspace, int64_t workspace_bytes,
                                    hipStream_t stream);
fn_status fn_norm_proj_swiglu_adaln_fp8_ws(const void* x, const float* mod, const int* idx, const void* W8_gate,
                                           const float* s_gate, const float* bias_gate, const void* W8_up,
                                           const float* s_up, const float* bias_up, void* out, int64_t M, int64_t K,
                                           int64_t N, int64_t T, float eps, void* workspace, int64_t workspace_bytes,
                                           hipStream_t stream);

/* Workspace bytes of the AdaLN calls that always run the pre-pass (the two
 * fp8-weight calls above, the SwiGLU one on the split operand, and the two
 * fp8-output calls below, on the operand rounded once): the size of
 * fn_adaln_workspace_bytes for every M >= 1; 0 for M < 1 or M, K outside
 * the limits. */
int64_t fn_adaln_prepass_bytes(int64_t M, int64_t K);

/* Projection kernel instance of the fp8 AdaLN calls; "invalid" for bad
 * shapes. */
const char* fn_kernel_name_adaln_fp8(int64_t M, int64_t K, int64_t N, int64_t T, int swiglu);

/* AdaLN + gate/up projections + SwiGLU with fp8 row-block output (E4M3
 * codes, one fp32 scale per 16-column row block, as fn_norm_proj_swiglu_q8),
 * in two launches for every M: the pre-pass, then the q8 kernel of the row
 * count on the modulated operand (the LDS-shared-x decode kernel up to 64
 * rows -- on projections of at least 512 column blocks up to 128 rows with
 * bf16 weights and 256 with fp8, 64-row blocks tiled -- the prefill kernel
 * above, with bf16 or fp8 weights).  The AdaLN FC1
 * block of [FlashInfer #5521] ("Segmented Chain": norm + AdaLN, FC1, SwiGLU,
 * quantisation for the next projection) with the output format of
 * [FlashInfer #4040] as read for fn_norm_proj_swiglu_q8.  The block values
 * are
 *   v = silu(a) * b,  a = (u * W_gate) / RMS(x) + bias_gate[idx],  b likewise,
 * u the pre-pass operand; arguments and errors as the calls above plus
 * out_codes [M,N] (uint8) and out_scales [M, ceil(N/16)] (fp32, 4-byte
 * aligned); workspace: fn_adaln_prepass_bytes(M, K) bytes. */
fn_status fn_norm_proj_swiglu_adaln_q8_ws(const void* x, const float* mod, const int* idx, const void* W_gate_packed,
                                          const float* bias_gate, const void* W_up_packed, const float* bias_up,
                                          void* out_codes, float* out_scales, int64_t M, int64_t K, int64_t N,
                                          int64_t T, float eps, void* workspace, int64_t workspace_bytes,
                                          hipStream_t stream);
fn_status fn_norm_proj_swiglu_adaln_fp8_q8_ws(const void* x, const float* mod, const int* idx, const void* W8_gate,
                                              const float* s_gate, const float* bias_gate, const void* W8_up,
                                              const float* s_up, const float* bias_up, void* out_codes,
                                              float* out_scales, int64_t M, int64_t K, int64_t N, int64_t T,
                                              float eps, void* workspace, int64_t workspace_bytes,
                                              hipStream_t stream);

/* Kernel instance of the two fp8-output AdaLN calls; "invalid" for bad
 * shapes. */
const char* fn_kernel_name_adaln_q8(int64_t M, int64_t K, int64_t N, int64_t T, int fp8_weights);

/* The pre-pass alone: for each row m, with mo = mod[idx[m]] (all zero when
 * idx[m] is outside [0, T)),
 *   u[m][k] = bf16_rne(fp32(x[m][k] * mo[k]))
 *   rs[m]   = 1 / sqrt(sum_k x[m][k]^2 / K + eps)         (fp32, raw x)
 * -- the operand the one-launch AdaLN kernel forms in registers, and the
 * deferred scale.  x, mod: as above; u: [M,K] bf16, 16-byte aligned; rs: [M]
 * fp32, 4-byte aligned; neither may overlap an input or the other. */
fn_status fn_adaln_modulate(const void* x, const float* mod, const int* idx, void* u, float* rs, int64_t M,
                            int64_t K, int64_t T, float eps, hipStream_t stream);

/* ---------------------------------------------------------------------------
 * Recorded steps: a sequence of fused calls replayed with one launch
 *
 * A decode step starts the norm + projection once per layer, dozens of
 * times, and on a GPU the starts and waits between small kernels cost more
 * than their arithmetic ([FlashNorm digest], summary bullets "problem
 * definition" and "GPU weakness"; [Fused kernels] closing summary, item 3:
 * launch overhead matters for small units of work).  fn_step_create records
 * the calls, in order, into a HIP graph once; fn_step_launch replays them
 * with a single graph launch.
 *
 * Every pointer and size is fixed when the step is recorded: a replay reads
 * whatever the x buffers hold at that time and overwrites the same outputs,
 * so a caller refreshes its inputs in place between replays.  The calls of a
 * step run in the order given, each after the previous one has finished
 * (stream order), so a later call may read an earlier call's output.
 * ------------------------------------------------------------------------- */

typedef enum {
  FN_CALL_NORM_PROJ = 0,            /* fn_norm_proj: w_gate = W_packed */
  FN_CALL_NORM_PROJ_SWIGLU = 1,     /* fn_norm_proj_swiglu: w_gate, w_up */
  FN_CALL_NORM_PROJ_FP8 = 2,        /* fn_norm_proj_fp8: w_gate = W8_packed, s_gate = scales */
  FN_CALL_NORM_PROJ_SWIGLU_FP8 = 3, /* fn_norm_proj_swiglu_fp8: w_gate, s_gate, w_up, s_up */
  FN_CALL_NORM_PROJ_SWIGLU_Q8 = 4,  /* fn_norm_proj_swiglu_q8: y = out_codes, y_scales = out_scales */
  FN_CALL_NORM_PROJ_SWIGLU_FP8_Q8 = 5 /* fn_norm_proj_swiglu_fp8_q8: as kind 3, outputs as kind 4 */
} fn_call_kind;

/* One call of a step: the arguments of the entry point `kind` names.
 * Fields a kind does not use are ignored (w_up for single projections,
 * s_gate / s_up for bf16 and fp32 weights, y_scales except for the fp8
 * output kinds, dt for kinds 2..5, which take bf16 activations). */
typedef struct {
  fn_call_kind kind;
  const void* x;
  const void* w_gate;
  const void* w_up;
  const float* s_gate;
  const float* s_up;
  void* y;
  int64_t M, K, N;
  float eps;
  fn_dtype dt;
  float* y_scales;
} fn_call;

typedef struct fn_step_s* fn_step;   /* opaque handle */

/* Validate every call exactly as its entry point would (no HIP call is made
 * before all of them pass), then record them into a HIP graph on a private
 * stream and instantiate it.  calls: host array of n_calls >= 1 entries,
 * copied; *out receives the handle.  Calls with M == 0 or N == 0 record
 * nothing.  Unlike the per-call entry points this allocates: host memory
 * for the handle and the HIP runtime's graph objects (freed by
 * fn_step_destroy).  An invalid call returns its status with
 * "call i: ..." in fn_last_error() and *out = NULL. */
fn_status fn_step_create(const fn_call* calls, int64_t n_calls, fn_step* out);

/* A step of independent calls run as ONE kernel launch: the column blocks
 * of every call are the workgroups of the same grid, in call order, so the
 * calls follow one another on the CUs with no drain and ramp between
 * kernels (a graph replay still runs one kernel per call, each ending in a
 * tail where CUs idle; [FlashNorm digest], summary bullets on the dozens of
 * norm launches per decode step; [Fused kernels] closing summary, item 3).
 * When every call has at most 16 rows, each workgroup
 * is one wave streaming the whole of k for two column blocks of its call,
 * x in registers (one x fragment load serves both); when some call has
 * 17..128 rows, every call runs in workgroups of 64 rows and twelve waves,
 * one column block each, sharing x through LDS (the entry point's
 * 17..64-row kernel with more column blocks per workgroup than a single
 * call could fill the GPU with).  The products follow the entry point's k order.  bf16 weights
 * up to 16 rows: the same bits as the call's own entry point where that
 * entry point also runs one wave over the whole of k (more than 256 column
 * blocks for a projection, more than 512 for a SwiGLU pair); narrower
 * calls, which the entry point splits over k across waves, agree with it
 * to the fp32 sum order.  Otherwise the sum of squares may be added in
 * another order than in the entry point (one chain, or other per-wave
 * partials), so an output can differ from the entry point's by one bf16
 * rounding step, rarely.  Takes FN_CALL_NORM_PROJ and
 * FN_CALL_NORM_PROJ_SWIGLU calls with FN_BF16, or FN_CALL_NORM_PROJ_FP8 and
 * FN_CALL_NORM_PROJ_SWIGLU_FP8 calls, all of one weight type, each with
 * M <= 128 (FN_ERR_SHAPE otherwise), 1 <= n_calls <= 65535; calls with
 * M == 0 or N == 0 add nothing (a step of only such calls launches
 * nothing).  The calls run at the same time, so no call may write a buffer
 * another call reads or writes (column scales included): FN_ERR_ALIAS
 * otherwise (a model's chained calls need the recorded graph of
 * fn_step_create).  Allocates host memory for the handle
 * and device memory for the call table (n_calls small records and two
 * bytes per workgroup), copied synchronously here; launching allocates
 * nothing. */
fn_status fn_step_create_grouped(const fn_call* calls, int64_t n_calls, fn_step* out);

/* Replay the recorded calls on `stream`: one graph launch, or for a
 * grouped step one kernel launch; allocates nothing.  A step must not be
 * replayed on two streams at once (its replays share the outputs). */
fn_status fn_step_launch(fn_step step, hipStream_t stream);

/* Kernel launches per replay of the step: the calls recorded (those with M,
 * N >= 1), or 1 for a grouped step (0 if all its calls are empty); -1 for
 * NULL. */
int64_t fn_step_num_kernels(fn_step step);

/* Release the graph (or the grouped step's device tables) and the handle;
 * NULL is a no-op.  The caller makes sure no replay is still running (e.g.
 * synchronises its stream). */
fn_status fn_step_destroy(fn_step step);

/* Static description of a status code. */
const char* fn_status_string(fn_status s);

/* Detail of the last failing call on this thread ("" if none). */
const char* fn_last_error(void);

#ifdef __cplusplus
}
#endif

#endif /* FLASHNORM_H */
