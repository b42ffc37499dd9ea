// libflashnorm C ABI: argument checks, kernel-instance choice, launches.
// The contract of every function is documented in include/flashnorm.h.
#include "../../include/flashnorm.h"

#include <cmath>
#include <cstdarg>
#include <cstdio>
#include <cstring>
#include <algorithm>
#include <mutex>
#include <new>
#include <vector>

#include "fn_launch.h"

namespace {

constexpr int64_t kMaxK = int64_t(1) << 20;
constexpr int64_t kMaxM = int64_t(1) << 22;
constexpr int64_t kMaxN = int64_t(1) << 24;

thread_local char g_last_error[256] = "";

fn_status fail(fn_status s, const char* fmt, ...) {
  va_list ap;
  va_start(ap, fmt);
  vsnprintf(g_last_error, sizeof g_last_error, fmt, ap);
  va_end(ap);
  return s;
}

bool dtype_ok(fn_dtype dt) { return dt == FN_F32 || dt == FN_BF16; }
fn::DType to_dt(fn_dtype dt) { return dt == FN_F32 ? fn::DType::F32 : fn::DType::BF16; }
int64_t esize(fn_dtype dt) { return dt == FN_F32 ? 4 : 2; }

bool aligned(const void* p, uintptr_t a) { return (reinterpret_cast<uintptr_t>(p) & (a - 1)) == 0; }

bool overlap(const void* a, int64_t abytes, const void* b, int64_t bbytes) {
  if (a == nullptr || b == nullptr || abytes <= 0 || bbytes <= 0) return false;
  const uintptr_t a0 = reinterpret_cast<uintptr_t>(a), b0 = reinterpret_cast<uintptr_t>(b);
  return a0 < b0 + (uintptr_t)bbytes && b0 < a0 + (uintptr_t)abytes;
}

int64_t packed_bytes(int64_t K, int64_t N, fn_dtype dt) {
  const int64_t kb = dt == FN_F32 ? 16 : 32;
  return ((N + 15) / 16) * ((K + kb - 1) / kb) * 1024;
}

fn_status check_k(int64_t K) {
  if (K < 1 || K > kMaxK) return fail(FN_ERR_SHAPE, "K=%lld must be in [1, %lld]", (long long)K, (long long)kMaxK);
  if (K % 8 != 0) return fail(FN_ERR_SHAPE, "K=%lld must be a multiple of 8", (long long)K);
  return FN_OK;
}

fn_status check_mn(int64_t M, int64_t N) {
  if (M < 0 || M > kMaxM) return fail(FN_ERR_SHAPE, "M=%lld must be in [0, %lld]", (long long)M, (long long)kMaxM);
  if (N < 0 || N > kMaxN) return fail(FN_ERR_SHAPE, "N=%lld must be in [0, %lld]", (long long)N, (long long)kMaxN);
  return FN_OK;
}

fn_status check_eps(float eps) {
  if (!std::isfinite(eps) || eps < 0.f) return fail(FN_ERR_EPS, "eps=%g must be finite and >= 0", (double)eps);
  return FN_OK;
}

fn_status hip_status(hipError_t e, const char* what) {
  if (e != hipSuccess) return fail(FN_ERR_HIP, "%s: %s", what, hipGetErrorString(e));
  return FN_OK;
}

#define FN_TRY(expr)                  \
  do {                                \
    const fn_status s_ = (expr);      \
    if (s_ != FN_OK) return s_;       \
  } while (0)

// check_only: validate and return without launching (recorded steps check
// every call before recording any).
fn_status fused_common(const void* x, const void* wg, const void* wu, void* y, int64_t M, int64_t K,
                       int64_t N, float eps, fn_dtype dt, hipStream_t stream, bool swiglu, bool check_only = false) {
  g_last_error[0] = '\0';
  if (!dtype_ok(dt)) return fail(FN_ERR_DTYPE, "unknown dtype %d", (int)dt);
  FN_TRY(check_k(K));
  FN_TRY(check_mn(M, N));
  FN_TRY(check_eps(eps));
  if (M == 0 || N == 0) return FN_OK;
  if (x == nullptr) return fail(FN_ERR_NULL, "x is NULL");
  if (wg == nullptr) return fail(FN_ERR_NULL, swiglu ? "W_gate_packed is NULL" : "W_packed is NULL");
  if (swiglu && wu == nullptr) return fail(FN_ERR_NULL, "W_up_packed is NULL");
  if (y == nullptr) return fail(FN_ERR_NULL, swiglu ? "out is NULL" : "y is NULL");
  if (!aligned(x, 16)) return fail(FN_ERR_ALIGN, "x must be 16-byte aligned");
  if (!aligned(wg, 16) || (swiglu && !aligned(wu, 16)))
    return fail(FN_ERR_ALIGN, "packed weights must be 16-byte aligned");
  if (!aligned(y, 16)) return fail(FN_ERR_ALIGN, "output must be 16-byte aligned");
  const int64_t e = esize(dt);
  const int64_t xb = M * K * e, yb = M * N * e, wb = packed_bytes(K, N, dt);
  if (overlap(y, yb, x, xb) || overlap(y, yb, wg, wb) || (swiglu && overlap(y, yb, wu, wb)))
    return fail(FN_ERR_ALIAS, "output overlaps an input");
  if (check_only) return FN_OK;
  const fn::DType t = to_dt(dt);
  const fn::FusedPlan plan = fn::plan_fused(t, M, K, N, swiglu);
  return hip_status(fn::launch_fused(t, plan, x, wg, swiglu ? wu : nullptr, y, (int)M, (int)K, (int)N, eps, stream),
                    plan.name);
}

int64_t packed_fp8_bytes(int64_t K, int64_t N) { return ((N + 15) / 16) * ((K + 63) / 64) * 1024; }

// Row counts past 64 that still take the LDS-shared-x decode kernel, its row
// blocks tiled over grid.y (each streams the weights again, mostly from L2),
// instead of the prefill kernel.
// Wide projections (at least 512 column blocks): a 128-row rung for bf16
// weights, 64- or 128-row blocks for fp8; the prefill kernel's 256-row tiles
// would leave most of each tile empty and give too few workgroups (96 for
// 12288 columns).  Measured on MI355X, K = 4096: QKV 62 -> 36 us (bf16,
// 65-128 rows), 64-67 -> 26-57 us (fp8, 65-256 rows); gate/up pairs 77 ->
// 47-51 us (bf16, 65-128 rows) and 81-87 -> 39-64 us (fp8, 65-256 rows).
// Beyond 128 rows with bf16 weights and 256 with fp8 the prefill kernel is
// faster.
// Narrow projections (one GPU's share under tensor parallelism): the prefill
// kernel gives them a few dozen 256 x 128 tiles, each streaming its x and
// weight panels at one CU's request rate, 48-106 us whatever the row count
// up to 1-2 thousand rows; the decode kernel's 64-row blocks spread them
// over the CUs.  Measured, K = 4096, prefill -> tiled decode: 1536 columns
// 59-61 -> 20-22 us (bf16, 65-512 rows), 54-65 -> 20-28 us (fp8, to 1024);
// 2 x 1376 75-78 -> 24-40 us (bf16), 80-84 -> 39-44 us (fp8); 6144 columns
// 61-64 -> 21-39 us (bf16, to 256 rows), 64-67 -> 21-54 us (fp8, to 512);
// the fp8-output and AdaLN forms 1.2-3.7x.  The gain ends where the row
// blocks' repeated weight streams catch up: with bf16 weights about 256 rows
// (512 at 192 column blocks or fewer); with fp8 256 rows above 384 column
// blocks (8176 columns at 384 rows: 67 against 71 us), 512 up to 384 and
// 1024 up to 192.
bool decode_rows_tiled(int64_t M, int64_t N, bool f8) {
  const int64_t nb = (N + 15) / 16;
  if (M <= 64) return false;
  if (nb >= 512) return M <= (f8 ? 256 : 128);
  if (!f8) return M <= (nb <= 192 ? 512 : 256);
  return M <= (nb <= 192 ? 1024 : (nb <= 384 ? 512 : 256));
}

// The same rows for the forms whose decode kernels have no 128-row rung --
// SwiGLU with fp8 output and the AdaLN two-launch calls -- run its 64-row
// instances tiled over the rows.  Measured on MI355X, K = 4096, 65-256 rows:
// fp8 output 90-104 -> 45-75 us (fp8 weights) and 90-91 -> 65-67 us (bf16,
// up to 128 rows); AdaLN QKV 87-93 -> 32-66 us (fp8) and 78-79 -> 43-52 us
// (bf16); AdaLN with fp8 output 98-108 -> 50-82 us and 94-95 -> 70-74 us.
// The AdaLN SwiGLU pair with bf16 output carries its operand as a hi + lo
// pair, twice the x bytes per row block: with fp8 weights it gains up to 128
// rows (86-89 -> 65-74 us) and loses beyond (95-101 -> 111-129 us), with bf16
// weights it loses (81-86 -> 87-93 us), so those stay on the prefill kernel.
bool premod_rows_tiled(int64_t M, int64_t N, bool f8, bool split) {
  return decode_rows_tiled(M, N, f8) && (!split || (f8 && M <= 128));
}

fn_status fp8_common(const void* x, const void* wg, const float* sg, const void* wu, const float* su, void* y,
                     int64_t M, int64_t K, int64_t N, float eps, hipStream_t stream, bool swiglu,
                     bool check_only = false) {
  g_last_error[0] = '\0';
  FN_TRY(check_k(K));
  FN_TRY(check_mn(M, N));
  FN_TRY(check_eps(eps));
  if (M == 0 || N == 0) return FN_OK;
  if (x == nullptr) return fail(FN_ERR_NULL, "x is NULL");
  if (wg == nullptr || sg == nullptr)
    return fail(FN_ERR_NULL, swiglu ? "W8_gate or s_gate is NULL" : "W8_packed or scales is NULL");
  if (swiglu && (wu == nullptr || su == nullptr)) return fail(FN_ERR_NULL, "W8_up or s_up is NULL");
  if (y == nullptr) return fail(FN_ERR_NULL, swiglu ? "out is NULL" : "y is NULL");
  if (!aligned(x, 16)) return fail(FN_ERR_ALIGN, "x must be 16-byte aligned");
  if (!aligned(wg, 16) || (swiglu && !aligned(wu, 16)))
    return fail(FN_ERR_ALIGN, "packed fp8 weights must be 16-byte aligned");
  if (!aligned(sg, 4) || (swiglu && !aligned(su, 4))) return fail(FN_ERR_ALIGN, "scales must be 4-byte aligned");
  if (!aligned(y, 16)) return fail(FN_ERR_ALIGN, "output must be 16-byte aligned");
  const int64_t xb = M * K * 2, yb = M * N * 2, wb = packed_fp8_bytes(K, N), sb = N * 4;
  if (overlap(y, yb, x, xb) || overlap(y, yb, wg, wb) || overlap(y, yb, sg, sb) ||
      (swiglu && (overlap(y, yb, wu, wb) || overlap(y, yb, su, sb))))
    return fail(FN_ERR_ALIAS, "output overlaps an input");
  if (check_only) return FN_OK;
  if (M > 64 && !decode_rows_tiled(M, N, true)) {
    const fn::FusedPlan plan = fn::plan_prefill(fn::DType::BF16, M, K, N, swiglu, false, false, true);
    return hip_status(fn::launch_prefill_fp8(plan, x, wg, sg, swiglu ? wu : nullptr, swiglu ? su : nullptr, y, (int)M,
                                             (int)K, (int)N, eps, stream),
                      plan.name);
  }
  if (fn::fp8_k_split(M, N, swiglu) != 0) {
    const fn::FusedPlan plan = fn::plan_fp8_ksplit(M, N, swiglu);
    return hip_status(fn::launch_fp8_ksplit(plan, x, wg, sg, swiglu ? wu : nullptr, swiglu ? su : nullptr, y, (int)M,
                                            (int)K, (int)N, eps, stream),
                      plan.name);
  }
  const fn::FusedPlan plan = fn::plan_fp8(M, K, N, swiglu);
  return hip_status(fn::launch_fp8(plan, x, wg, sg, swiglu ? wu : nullptr, swiglu ? su : nullptr, y, (int)M, (int)K,
                                   (int)N, eps, stream),
                    plan.name);
}

// SwiGLU with fp8 output: bf16 activations, bf16 packed weights (f8 false)
// or E4M3 codes with column scales (f8 true); codes [M,N] and row-block
// scales [M, ceil(N/16)] out.
fn_status q8_common(const void* x, const void* wg, const float* sg, const void* wu, const float* su, void* codes,
                    float* scales, int64_t M, int64_t K, int64_t N, float eps, hipStream_t stream, bool f8,
                    bool check_only = false) {
  g_last_error[0] = '\0';
  FN_TRY(check_k(K));
  FN_TRY(check_mn(M, N));
  FN_TRY(check_eps(eps));
  if (M == 0 || N == 0) return FN_OK;
  if (x == nullptr) return fail(FN_ERR_NULL, "x is NULL");
  if (wg == nullptr || wu == nullptr) return fail(FN_ERR_NULL, "gate or up weights are NULL");
  if (f8 && (sg == nullptr || su == nullptr)) return fail(FN_ERR_NULL, "s_gate or s_up is NULL");
  if (codes == nullptr || scales == nullptr) return fail(FN_ERR_NULL, "out_codes or out_scales is NULL");
  if (!aligned(x, 16)) return fail(FN_ERR_ALIGN, "x must be 16-byte aligned");
  if (!aligned(wg, 16) || !aligned(wu, 16)) return fail(FN_ERR_ALIGN, "packed weights must be 16-byte aligned");
  if (f8 && (!aligned(sg, 4) || !aligned(su, 4))) return fail(FN_ERR_ALIGN, "scales must be 4-byte aligned");
  if (!aligned(scales, 4)) return fail(FN_ERR_ALIGN, "out_scales must be 4-byte aligned");
  const int64_t xb = M * K * 2, cb = M * N, qb = M * ((N + 15) / 16) * 4;
  const int64_t wb = f8 ? packed_fp8_bytes(K, N) : packed_bytes(K, N, FN_BF16), sb = f8 ? N * 4 : 0;
  for (const void* out : {static_cast<const void*>(codes), static_cast<const void*>(scales)}) {
    const int64_t ob = out == codes ? cb : qb;
    if (overlap(out, ob, x, xb) || overlap(out, ob, wg, wb) || overlap(out, ob, wu, wb) ||
        (f8 && (overlap(out, ob, sg, sb) || overlap(out, ob, su, sb))))
      return fail(FN_ERR_ALIAS, "an output overlaps an input");
  }
  if (overlap(codes, cb, scales, qb)) return fail(FN_ERR_ALIAS, "out_codes overlaps out_scales");
  if (check_only) return FN_OK;
  uint8_t* q = static_cast<uint8_t*>(codes);
  if (M > 64 && !decode_rows_tiled(M, N, f8)) {
    const fn::FusedPlan plan = fn::plan_prefill(fn::DType::BF16, M, K, N, true, true, false, f8);
    if (f8)
      return hip_status(fn::launch_prefill_fp8(plan, x, wg, sg, wu, su, nullptr, (int)M, (int)K, (int)N, eps, stream, q,
                                               scales),
                        plan.name);
    return hip_status(fn::launch_prefill(fn::DType::BF16, plan, x, wg, wu, nullptr, (int)M, (int)K, (int)N, eps,
                                         stream, q, scales),
                      plan.name);
  }
  const fn::FusedPlan plan = fn::plan_decode_q8(f8, M, N);
  return hip_status(fn::launch_decode_q8(f8, plan, x, wg, sg, wu, su, q, scales, (int)M, (int)K, (int)N, eps, stream),
                    plan.name);
}

constexpr int64_t kAdalnOneLaunchRows = 16;   // the one-launch AdaLN kernel's rows; the _ws calls run it up to here

// AdaLN prologue (bf16): x [M,K], modulation table mod [T,K] fp32 (the gain
// folded in), idx [M], packed plain W (gate and up for SwiGLU), bias rows
// [T,N] fp32, y [M,N].  check_only validates the arguments every AdaLN call
// shares; the one-launch call itself takes at most 16 rows.
fn_status adaln_common(const void* x, const float* mod, const int* idx, const void* wg, const float* bg,
                       const void* wu, const float* bu, void* y, int64_t M, int64_t K, int64_t N, int64_t T,
                       float eps, hipStream_t stream, bool swiglu, bool check_only = false) {
  g_last_error[0] = '\0';
  FN_TRY(check_k(K));
  FN_TRY(check_mn(M, N));
  FN_TRY(check_eps(eps));
  if (T < 1 || T > INT32_MAX || T * K * 4 > INT32_MAX)
    return fail(FN_ERR_SHAPE, "T=%lld must be >= 1 with T*K*4 < 2^31", (long long)T);
  if (!check_only && M > kAdalnOneLaunchRows)
    return fail(FN_ERR_SHAPE,
                "M=%lld: the one-launch AdaLN calls take at most %lld rows; more rows run faster in two launches "
                "(fn_norm_proj_adaln_ws / fn_norm_proj_swiglu_adaln_ws with a workspace)",
                (long long)M, (long long)kAdalnOneLaunchRows);
  if (M == 0 || N == 0) return FN_OK;
  if (x == nullptr || mod == nullptr || idx == nullptr) return fail(FN_ERR_NULL, "x, mod or idx is NULL");
  if (wg == nullptr || bg == nullptr) return fail(FN_ERR_NULL, "W_packed or bias is NULL");
  if (swiglu && (wu == nullptr || bu == nullptr)) return fail(FN_ERR_NULL, "W_up_packed or bias_up is NULL");
  if (y == nullptr) return fail(FN_ERR_NULL, "y is NULL");
  if (!aligned(x, 16) || !aligned(mod, 16)) return fail(FN_ERR_ALIGN, "x and mod must be 16-byte aligned");
  if (!aligned(wg, 16) || (swiglu && !aligned(wu, 16)))
    return fail(FN_ERR_ALIGN, "packed weights must be 16-byte aligned");
  if (!aligned(idx, 4) || !aligned(bg, 4) || (swiglu && !aligned(bu, 4)))
    return fail(FN_ERR_ALIGN, "idx and bias must be 4-byte aligned");
  if (!aligned(y, 16)) return fail(FN_ERR_ALIGN, "output must be 16-byte aligned");
  const int64_t yb = M * N * 2, wb = packed_bytes(K, N, FN_BF16), bb = T * N * 4;
  if (overlap(y, yb, x, M * K * 2) || overlap(y, yb, mod, T * K * 4) || overlap(y, yb, idx, M * 4) ||
      overlap(y, yb, wg, wb) || overlap(y, yb, bg, bb) || (swiglu && (overlap(y, yb, wu, wb) || overlap(y, yb, bu, bb))))
    return fail(FN_ERR_ALIAS, "output overlaps an input");
  if (check_only) return FN_OK;
  const fn::AdalnArgs ad{mod, idx, bg, swiglu ? bu : nullptr, (int)T};
  const fn::FusedPlan plan = fn::plan_adaln(M, N, swiglu);
  return hip_status(fn::launch_adaln(plan, x, wg, swiglu ? wu : nullptr, y, (int)M, (int)K, (int)N, eps, ad, stream),
                    plan.name);
}

int64_t align256(int64_t b) { return (b + 255) / 256 * 256; }

// Two-launch AdaLN workspace: the modulated operand u [M,K] bf16 (split in
// two parts for SwiGLU with bf16 output: [2M,K]), then 1/RMS per row [M]
// fp32, each at a 256-byte boundary.  The exported sizes are those of the
// split form, enough for every call.
int64_t adaln_u_bytes(int64_t M, int64_t K, bool split) { return align256(M * K * 2 * (split ? 2 : 1)); }
int64_t adaln_ws_need(int64_t M, int64_t K, bool split = true) {
  return adaln_u_bytes(M, K, split) + align256(M * 4);
}

fn_status adaln_ws_common(const void* x, const float* mod, const int* idx, const void* wg, const float* bg,
                          const void* wu, const float* bu, void* y, int64_t M, int64_t K, int64_t N, int64_t T,
                          float eps, void* ws, int64_t ws_bytes, hipStream_t stream, bool swiglu) {
  FN_TRY(adaln_common(x, mod, idx, wg, bg, wu, bu, y, M, K, N, T, eps, stream, swiglu, true));
  if (M == 0 || N == 0) return FN_OK;
  if (M <= kAdalnOneLaunchRows)
    return adaln_common(x, mod, idx, wg, bg, wu, bu, y, M, K, N, T, eps, stream, swiglu);
  const int64_t need = adaln_ws_need(M, K, swiglu);
  if (ws == nullptr) return fail(FN_ERR_WORKSPACE, "workspace is NULL (the call needs %lld bytes)", (long long)need);
  if (!aligned(ws, 256)) return fail(FN_ERR_WORKSPACE, "workspace must be 256-byte aligned");
  if (ws_bytes < need)
    return fail(FN_ERR_WORKSPACE, "workspace_bytes=%lld, the call needs %lld", (long long)ws_bytes, (long long)need);
  const int64_t wb = packed_bytes(K, N, FN_BF16), bb = T * N * 4;
  if (overlap(ws, need, x, M * K * 2) || overlap(ws, need, mod, T * K * 4) || overlap(ws, need, idx, M * 4) ||
      overlap(ws, need, wg, wb) || overlap(ws, need, bg, bb) || overlap(ws, need, y, M * N * 2) ||
      (swiglu && (overlap(ws, need, wu, wb) || overlap(ws, need, bu, bb))))
    return fail(FN_ERR_ALIAS, "workspace overlaps an argument");
  void* u = ws;
  float* rs = reinterpret_cast<float*>(static_cast<uint8_t*>(ws) + adaln_u_bytes(M, K, swiglu));
  FN_TRY(hip_status(fn::launch_adaln_modulate(x, mod, idx, (int)T, u, rs, (int)M, (int)K, eps, stream, swiglu),
                    "adaln_modulate"));
  const fn::AdalnArgs ad{nullptr, idx, bg, swiglu ? bu : nullptr, (int)T};
  if (M <= 64 || premod_rows_tiled(M, N, false, swiglu)) {
    const fn::FusedPlan plan = fn::plan_decode_premod(M, N, swiglu);
    return hip_status(fn::launch_decode_premod(plan, u, rs, wg, nullptr, swiglu ? wu : nullptr, nullptr, y, (int)M,
                                               (int)K, (int)N, ad, stream),
                      plan.name);
  }
  const fn::FusedPlan plan = fn::plan_prefill(fn::DType::BF16, M, K, N, swiglu, false, true);
  return hip_status(fn::launch_prefill_premod(plan, u, rs, wg, swiglu ? wu : nullptr, y, (int)M, (int)K, (int)N, ad,
                                              stream),
                    plan.name);
}

// Two-launch AdaLN with fp8 weights (E4M3 codes + column scales), every M:
// the pre-pass, then the fp8 decode or prefill kernel on the modulated
// operand.
fn_status adaln_fp8_ws_common(const void* x, const float* mod, const int* idx, const void* wg, const float* sg,
                              const float* bg, const void* wu, const float* su, const float* bu, void* y, int64_t M,
                              int64_t K, int64_t N, int64_t T, float eps, void* ws, int64_t ws_bytes,
                              hipStream_t stream, bool swiglu) {
  g_last_error[0] = '\0';
  FN_TRY(check_k(K));
  FN_TRY(check_mn(M, N));
  FN_TRY(check_eps(eps));
  if (T < 1 || T > INT32_MAX || T * K * 4 > INT32_MAX)
    return fail(FN_ERR_SHAPE, "T=%lld must be >= 1 with T*K*4 < 2^31", (long long)T);
  if (M == 0 || N == 0) return FN_OK;
  if (x == nullptr || mod == nullptr || idx == nullptr) return fail(FN_ERR_NULL, "x, mod or idx is NULL");
  if (wg == nullptr || sg == nullptr || bg == nullptr)
    return fail(FN_ERR_NULL, swiglu ? "W8_gate, s_gate or bias_gate is NULL" : "W8_packed, scales or bias is NULL");
  if (swiglu && (wu == nullptr || su == nullptr || bu == nullptr))
    return fail(FN_ERR_NULL, "W8_up, s_up or bias_up is NULL");
  if (y == nullptr) return fail(FN_ERR_NULL, swiglu ? "out is NULL" : "y is NULL");
  if (!aligned(x, 16) || !aligned(mod, 16)) return fail(FN_ERR_ALIGN, "x and mod must be 16-byte aligned");
  if (!aligned(wg, 16) || (swiglu && !aligned(wu, 16)))
    return fail(FN_ERR_ALIGN, "packed fp8 weights must be 16-byte aligned");
  if (!aligned(idx, 4) || !aligned(sg, 4) || !aligned(bg, 4) || (swiglu && (!aligned(su, 4) || !aligned(bu, 4))))
    return fail(FN_ERR_ALIGN, "idx, scales and bias must be 4-byte aligned");
  if (!aligned(y, 16)) return fail(FN_ERR_ALIGN, "output must be 16-byte aligned");
  const int64_t yb = M * N * 2, wb = packed_fp8_bytes(K, N), sb = N * 4, bb = T * N * 4;
  const void* ins[] = {x, mod, idx, wg, sg, bg, swiglu ? wu : nullptr, swiglu ? su : nullptr,
                       swiglu ? bu : nullptr};
  const int64_t inb[] = {M * K * 2, T * K * 4, M * 4, wb, sb, bb, wb, sb, bb};
  for (int i = 0; i < 9; ++i)
    if (overlap(y, yb, ins[i], inb[i])) return fail(FN_ERR_ALIAS, "output overlaps an input");
  const int64_t need = adaln_ws_need(M, K, swiglu);
  if (ws == nullptr) return fail(FN_ERR_WORKSPACE, "workspace is NULL (the call needs %lld bytes)", (long long)need);
  if (!aligned(ws, 256)) return fail(FN_ERR_WORKSPACE, "workspace must be 256-byte aligned");
  if (ws_bytes < need)
    return fail(FN_ERR_WORKSPACE, "workspace_bytes=%lld, the call needs %lld", (long long)ws_bytes, (long long)need);
  for (int i = 0; i < 9; ++i)
    if (overlap(ws, need, ins[i], inb[i])) return fail(FN_ERR_ALIAS, "workspace overlaps an argument");
  if (overlap(ws, need, y, yb)) return fail(FN_ERR_ALIAS, "workspace overlaps an argument");
  void* u = ws;
  float* rs = reinterpret_cast<float*>(static_cast<uint8_t*>(ws) + adaln_u_bytes(M, K, swiglu));
  FN_TRY(hip_status(fn::launch_adaln_modulate(x, mod, idx, (int)T, u, rs, (int)M, (int)K, eps, stream, swiglu),
                    "adaln_modulate"));
  const fn::AdalnArgs ad{nullptr, idx, bg, swiglu ? bu : nullptr, (int)T};
  if (M > 64 && !premod_rows_tiled(M, N, true, swiglu)) {
    const fn::FusedPlan plan = fn::plan_prefill(fn::DType::BF16, M, K, N, swiglu, false, true, true);
    return hip_status(fn::launch_prefill_premod(plan, u, rs, wg, swiglu ? wu : nullptr, y, (int)M, (int)K, (int)N, ad,
                                                stream, nullptr, nullptr, sg, swiglu ? su : nullptr),
                      plan.name);
  }
  const fn::FusedPlan plan = fn::plan_decode_premod(M, N, swiglu, true);
  return hip_status(fn::launch_decode_premod(plan, u, rs, wg, sg, swiglu ? wu : nullptr, swiglu ? su : nullptr, y,
                                             (int)M, (int)K, (int)N, ad, stream),
                    plan.name);
}

// Two-launch AdaLN + SwiGLU with fp8 row-block output, every M: bf16 weights
// (f8 false) or E4M3 codes with column scales (f8 true).
fn_status adaln_q8_ws_common(const void* x, const float* mod, const int* idx, const void* wg, const float* sg,
                             const float* bg, const void* wu, const float* su, const float* bu, void* codes,
                             float* qscales, int64_t M, int64_t K, int64_t N, int64_t T, float eps, void* ws,
                             int64_t ws_bytes, hipStream_t stream, bool f8) {
  g_last_error[0] = '\0';
  FN_TRY(check_k(K));
  FN_TRY(check_mn(M, N));
  FN_TRY(check_eps(eps));
  if (T < 1 || T > INT32_MAX || T * K * 4 > INT32_MAX)
    return fail(FN_ERR_SHAPE, "T=%lld must be >= 1 with T*K*4 < 2^31", (long long)T);
  if (M == 0 || N == 0) return FN_OK;
  if (x == nullptr || mod == nullptr || idx == nullptr) return fail(FN_ERR_NULL, "x, mod or idx is NULL");
  if (wg == nullptr || wu == nullptr || bg == nullptr || bu == nullptr)
    return fail(FN_ERR_NULL, "gate or up weights or bias rows are NULL");
  if (f8 && (sg == nullptr || su == nullptr)) return fail(FN_ERR_NULL, "s_gate or s_up is NULL");
  if (codes == nullptr || qscales == nullptr) return fail(FN_ERR_NULL, "out_codes or out_scales is NULL");
  if (!aligned(x, 16) || !aligned(mod, 16)) return fail(FN_ERR_ALIGN, "x and mod must be 16-byte aligned");
  if (!aligned(wg, 16) || !aligned(wu, 16)) return fail(FN_ERR_ALIGN, "packed weights must be 16-byte aligned");
  if (!aligned(idx, 4) || !aligned(bg, 4) || !aligned(bu, 4) || (f8 && (!aligned(sg, 4) || !aligned(su, 4))))
    return fail(FN_ERR_ALIGN, "idx, scales and bias must be 4-byte aligned");
  if (!aligned(qscales, 4)) return fail(FN_ERR_ALIGN, "out_scales must be 4-byte aligned");
  const int64_t wb = f8 ? packed_fp8_bytes(K, N) : packed_bytes(K, N, FN_BF16), sb = f8 ? N * 4 : 0, bb = T * N * 4;
  const void* ins[] = {x, mod, idx, wg, wu, bg, bu, f8 ? sg : nullptr, f8 ? su : nullptr};
  const int64_t inb[] = {M * K * 2, T * K * 4, M * 4, wb, wb, bb, bb, sb, sb};
  const int64_t cb = M * N, qb = M * ((N + 15) / 16) * 4;
  for (int i = 0; i < 9; ++i)
    if (overlap(codes, cb, ins[i], inb[i]) || overlap(qscales, qb, ins[i], inb[i]))
      return fail(FN_ERR_ALIAS, "an output overlaps an input");
  if (overlap(codes, cb, qscales, qb)) return fail(FN_ERR_ALIAS, "out_codes overlaps out_scales");
  const int64_t need = adaln_ws_need(M, K, false);
  if (ws == nullptr) return fail(FN_ERR_WORKSPACE, "workspace is NULL (the call needs %lld bytes)", (long long)need);
  if (!aligned(ws, 256)) return fail(FN_ERR_WORKSPACE, "workspace must be 256-byte aligned");
  if (ws_bytes < need)
    return fail(FN_ERR_WORKSPACE, "workspace_bytes=%lld, the call needs %lld", (long long)ws_bytes, (long long)need);
  for (int i = 0; i < 9; ++i)
    if (overlap(ws, need, ins[i], inb[i])) return fail(FN_ERR_ALIAS, "workspace overlaps an argument");
  if (overlap(ws, need, codes, cb) || overlap(ws, need, qscales, qb))
    return fail(FN_ERR_ALIAS, "workspace overlaps an argument");
  void* u = ws;
  float* rs = reinterpret_cast<float*>(static_cast<uint8_t*>(ws) + adaln_u_bytes(M, K, false));
  FN_TRY(hip_status(fn::launch_adaln_modulate(x, mod, idx, (int)T, u, rs, (int)M, (int)K, eps, stream),
                    "adaln_modulate"));
  const fn::AdalnArgs ad{nullptr, idx, bg, bu, (int)T};
  uint8_t* q = static_cast<uint8_t*>(codes);
  if (M > 64 && !premod_rows_tiled(M, N, f8, false)) {
    const fn::FusedPlan plan = fn::plan_prefill(fn::DType::BF16, M, K, N, true, true, true, f8);
    return hip_status(fn::launch_prefill_premod(plan, u, rs, wg, wu, nullptr, (int)M, (int)K, (int)N, ad, stream, q,
                                                qscales, f8 ? sg : nullptr, f8 ? su : nullptr),
                      plan.name);
  }
  const fn::FusedPlan plan = fn::plan_decode_q8_premod(f8, M, N);
  return hip_status(fn::launch_decode_q8_premod(f8, plan, u, rs, wg, f8 ? sg : nullptr, wu, f8 ? su : nullptr, q,
                                                qscales, (int)M, (int)K, (int)N, ad, stream),
                    plan.name);
}

// One recorded call: validate (check_only) or enqueue it on `stream`.
fn_status run_call(const fn_call& c, hipStream_t stream, bool check_only) {
  switch (c.kind) {
    case FN_CALL_NORM_PROJ:
      return fused_common(c.x, c.w_gate, nullptr, c.y, c.M, c.K, c.N, c.eps, c.dt, stream, false, check_only);
    case FN_CALL_NORM_PROJ_SWIGLU:
      return fused_common(c.x, c.w_gate, c.w_up, c.y, c.M, c.K, c.N, c.eps, c.dt, stream, true, check_only);
    case FN_CALL_NORM_PROJ_FP8:
      return fp8_common(c.x, c.w_gate, c.s_gate, nullptr, nullptr, c.y, c.M, c.K, c.N, c.eps, stream, false,
                        check_only);
    case FN_CALL_NORM_PROJ_SWIGLU_FP8:
      return fp8_common(c.x, c.w_gate, c.s_gate, c.w_up, c.s_up, c.y, c.M, c.K, c.N, c.eps, stream, true,
                        check_only);
    case FN_CALL_NORM_PROJ_SWIGLU_Q8:
      return q8_common(c.x, c.w_gate, nullptr, c.w_up, nullptr, c.y, c.y_scales, c.M, c.K, c.N, c.eps, stream,
                       false, check_only);
    case FN_CALL_NORM_PROJ_SWIGLU_FP8_Q8:
      return q8_common(c.x, c.w_gate, c.s_gate, c.w_up, c.s_up, c.y, c.y_scales, c.M, c.K, c.N, c.eps, stream,
                       true, check_only);
  }
  return fail(FN_ERR_DTYPE, "unknown call kind %d", (int)c.kind);
}

// Prefix the current error text with the index of the failing call.
fn_status call_failed(fn_status s, int64_t i) {
  char detail[sizeof g_last_error];
  std::memcpy(detail, g_last_error, sizeof detail);
  return fail(s, "call %lld: %s", (long long)i, detail);
}

}  // namespace

struct fn_step_s {
  hipGraph_t graph = nullptr;
  hipGraphExec_t exec = nullptr;
  int64_t kernels = 0;
  void* calls = nullptr;   // grouped: the call records (device)
  void* items = nullptr;   // grouped: the call of each workgroup (device)
  int64_t nitems = 0;      // grouped: workgroups of the one launch
  bool grouped = false;
  bool fp8 = false;        // grouped: the calls take fp8 weights
  bool wide = false;       // grouped: some call has more than 16 rows (the LDS-shared-x tile)
};

namespace fn {

// The row ladder.  bf16: up to 16 rows the skinny decode kernel with x in
// registers; 17..64 rows the decode kernel that shares x through LDS (both
// weight streaming, HBM-bound), and its 128-row rung up to 128 rows of wide
// projections (decode_rows_tiled); more rows the tiled prefill kernel
// (MFMA-bound).  fp32 at any M stays on the register decode kernel, tiled
// over rows.
FusedPlan plan_fused(DType dt, int64_t M, int64_t K, int64_t N, bool swiglu) {
  if (dt == DType::BF16 && M > 64 && !decode_rows_tiled(M, N, false)) return plan_prefill(dt, M, K, N, swiglu);
  // narrow SwiGLU pairs at 17-64 rows, and past 64 rows while the 64-row
  // blocks give at most 256 workgroups: the register-x kernel with a 4-wave
  // k-split (2 x 1376 columns, 65-128 rows: 24 us against 27-28 on the
  // LDS-shared-x kernel)
  const int64_t nb = (N + 15) / 16;
  if (dt == DType::BF16 && swiglu && M > 16 && nb <= 256 && (M <= 64 || nb * ((M + 63) / 64) <= 256))
    return plan_decode(dt, M, K, N, swiglu);
  if (dt == DType::BF16 && M > 16) return plan_decode_x(dt, M, K, N, swiglu);
  return plan_decode(dt, M, K, N, swiglu);
}

hipError_t launch_fused(DType dt, const FusedPlan& plan, const void* x, const void* w_gate,
                        const void* w_up, void* y, int M, int K, int N, float eps, hipStream_t stream) {
  if (plan.kind == 1) return launch_prefill(dt, plan, x, w_gate, w_up, y, M, K, N, eps, stream);
  if (plan.kind == 2) return launch_decode_x(dt, plan, x, w_gate, w_up, y, M, K, N, eps, stream);
  return launch_decode(dt, plan, x, w_gate, w_up, y, M, K, N, eps, stream);
}

}  // namespace fn

extern "C" {

size_t fn_packed_weight_bytes(int64_t K, int64_t N, fn_dtype dt) {
  if (!dtype_ok(dt) || K < 1 || K > kMaxK || K % 8 != 0 || N < 0 || N > kMaxN) return 0;
  return (size_t)packed_bytes(K, N, dt);
}

fn_status fn_fold_weights(const void* g, const void* W, void* W_packed, int64_t K, int64_t N, fn_dtype dt,
                          hipStream_t stream) {
  g_last_error[0] = '\0';
  if (!dtype_ok(dt)) return fail(FN_ERR_DTYPE, "unknown dtype %d", (int)dt);
  FN_TRY(check_k(K));
  FN_TRY(check_mn(0, N));
  if (N == 0) return FN_OK;
  if (W == nullptr) return fail(FN_ERR_NULL, "W is NULL");
  if (W_packed == nullptr) return fail(FN_ERR_NULL, "W_packed is NULL");
  const int64_t e = esize(dt);
  if ((g != nullptr && !aligned(g, (uintptr_t)e)) || !aligned(W, (uintptr_t)e))
    return fail(FN_ERR_ALIGN, "g and W must be aligned to their element size");
  if (!aligned(W_packed, 16)) return fail(FN_ERR_ALIGN, "W_packed must be 16-byte aligned");
  const int64_t pb = packed_bytes(K, N, dt);
  if (overlap(W_packed, pb, W, K * N * e) || overlap(W_packed, pb, g, K * e))
    return fail(FN_ERR_ALIAS, "W_packed overlaps g or W");
  return hip_status(fn::launch_fold(to_dt(dt), g, W, W_packed, (int)K, (int)N, stream), "fold_weights");
}

fn_status fn_norm_proj(const void* x, const void* W_packed, void* y, int64_t M, int64_t K, int64_t N, float eps,
                       fn_dtype dt, hipStream_t stream) {
  return fused_common(x, W_packed, nullptr, y, M, K, N, eps, dt, stream, false);
}

fn_status fn_norm_proj_swiglu(const void* x, const void* W_gate_packed, const void* W_up_packed, void* out,
                              int64_t M, int64_t K, int64_t N, float eps, fn_dtype dt, hipStream_t stream) {
  return fused_common(x, W_gate_packed, W_up_packed, out, M, K, N, eps, dt, stream, true);
}

fn_status fn_rmsnorm(const void* x, const void* g, void* xhat, int64_t M, int64_t K, float eps, fn_dtype dt,
                     hipStream_t stream) {
  g_last_error[0] = '\0';
  if (!dtype_ok(dt)) return fail(FN_ERR_DTYPE, "unknown dtype %d", (int)dt);
  FN_TRY(check_k(K));
  FN_TRY(check_mn(M, 0));
  FN_TRY(check_eps(eps));
  if (M == 0) return FN_OK;
  if (x == nullptr || g == nullptr || xhat == nullptr) return fail(FN_ERR_NULL, "x, g and xhat must be non-NULL");
  const int64_t e = esize(dt);
  if (!aligned(x, (uintptr_t)e) || !aligned(g, (uintptr_t)e) || !aligned(xhat, (uintptr_t)e))
    return fail(FN_ERR_ALIGN, "x, g and xhat must be aligned to their element size");
  if (overlap(xhat, M * K * e, x, M * K * e) || overlap(xhat, M * K * e, g, K * e))
    return fail(FN_ERR_ALIAS, "xhat overlaps x or g");
  return hip_status(fn::launch_rmsnorm(to_dt(dt), x, g, xhat, (int)M, (int)K, eps, stream), "rmsnorm");
}

fn_status fn_silu_mul(const void* h, void* out, int64_t M, int64_t N, fn_dtype dt, hipStream_t stream) {
  g_last_error[0] = '\0';
  if (!dtype_ok(dt)) return fail(FN_ERR_DTYPE, "unknown dtype %d", (int)dt);
  FN_TRY(check_mn(M, N));
  if (M == 0 || N == 0) return FN_OK;
  if (h == nullptr || out == nullptr) return fail(FN_ERR_NULL, "h and out must be non-NULL");
  const int64_t e = esize(dt);
  if (!aligned(h, (uintptr_t)e) || !aligned(out, (uintptr_t)e))
    return fail(FN_ERR_ALIGN, "h and out must be aligned to their element size");
  if (overlap(out, M * N * e, h, M * 2 * N * e)) return fail(FN_ERR_ALIAS, "out overlaps h");
  return hip_status(fn::launch_silu_mul(to_dt(dt), h, out, (int)M, (int)N, stream), "silu_mul");
}

fn_status fn_probe_hbm_read(const void* src, int64_t bytes, void* sink, int64_t workgroups, hipStream_t stream) {
  g_last_error[0] = '\0';
  if (bytes < 16 || bytes % 16 != 0) return fail(FN_ERR_SHAPE, "bytes must be a positive multiple of 16");
  if (workgroups < 1 || workgroups > 65536) return fail(FN_ERR_SHAPE, "workgroups must be in [1, 65536]");
  if (src == nullptr || sink == nullptr) return fail(FN_ERR_NULL, "src and sink must be non-NULL");
  if (!aligned(src, 16) || !aligned(sink, 4)) return fail(FN_ERR_ALIGN, "src must be 16-byte and sink 4-byte aligned");
  return hip_status(fn::launch_probe_read(src, bytes, sink, (int)workgroups, stream), "probe_read");
}

fn_status fn_probe_mfma_bf16(void* sink, int64_t iters, int64_t workgroups, hipStream_t stream) {
  g_last_error[0] = '\0';
  if (iters < 1 || iters > (1 << 20)) return fail(FN_ERR_SHAPE, "iters must be in [1, 2^20]");
  if (workgroups < 1 || workgroups > 65536) return fail(FN_ERR_SHAPE, "workgroups must be in [1, 65536]");
  if (sink == nullptr) return fail(FN_ERR_NULL, "sink must be non-NULL");
  if (!aligned(sink, 4)) return fail(FN_ERR_ALIGN, "sink must be 4-byte aligned");
  return hip_status(fn::launch_probe_mfma(sink, (int)iters, (int)workgroups, stream), "probe_mfma");
}

size_t fn_packed_fp8_bytes(int64_t K, int64_t N) {
  if (K < 1 || K > kMaxK || K % 8 != 0 || N < 0 || N > kMaxN) return 0;
  return (size_t)packed_fp8_bytes(K, N);
}

fn_status fn_fold_weights_fp8(const void* g, const void* W, void* W8_packed, float* scales, int64_t K, int64_t N,
                              fn_dtype dt, hipStream_t stream) {
  g_last_error[0] = '\0';
  if (!dtype_ok(dt)) return fail(FN_ERR_DTYPE, "unknown dtype %d", (int)dt);
  FN_TRY(check_k(K));
  FN_TRY(check_mn(0, N));
  if (N == 0) return FN_OK;
  if (W == nullptr) return fail(FN_ERR_NULL, "W is NULL");
  if (W8_packed == nullptr || scales == nullptr) return fail(FN_ERR_NULL, "W8_packed or scales is NULL");
  const int64_t e = esize(dt);
  if ((g != nullptr && !aligned(g, (uintptr_t)e)) || !aligned(W, (uintptr_t)e))
    return fail(FN_ERR_ALIGN, "g and W must be aligned to their element size");
  if (!aligned(W8_packed, 16)) return fail(FN_ERR_ALIGN, "W8_packed must be 16-byte aligned");
  if (!aligned(scales, 4)) return fail(FN_ERR_ALIGN, "scales must be 4-byte aligned");
  const int64_t pb = packed_fp8_bytes(K, N);
  if (overlap(W8_packed, pb, W, K * N * e) || overlap(W8_packed, pb, g, K * e) ||
      overlap(scales, N * 4, W, K * N * e) || overlap(scales, N * 4, g, K * e) || overlap(scales, N * 4, W8_packed, pb))
    return fail(FN_ERR_ALIAS, "W8_packed or scales overlaps an input or each other");
  return hip_status(fn::launch_fold_fp8(to_dt(dt), g, W, W8_packed, scales, (int)K, (int)N, stream),
                    "fold_weights_fp8");
}

fn_status fn_norm_proj_fp8(const void* x, const void* W8_packed, const float* scales, void* y, int64_t M, int64_t K,
                           int64_t N, float eps, hipStream_t stream) {
  return fp8_common(x, W8_packed, scales, nullptr, nullptr, y, M, K, N, eps, stream, false);
}

fn_status fn_norm_proj_swiglu_fp8(const void* x, const void* W8_gate, const float* s_gate, const void* W8_up,
                                  const float* s_up, void* out, int64_t M, int64_t K, int64_t N, float eps,
                                  hipStream_t stream) {
  return fp8_common(x, W8_gate, s_gate, W8_up, s_up, out, M, K, N, eps, stream, true);
}

fn_status fn_norm_proj_swiglu_q8(const void* x, const void* W_gate_packed, const void* W_up_packed, void* out_codes,
                                 float* out_scales, int64_t M, int64_t K, int64_t N, float eps, hipStream_t stream) {
  return q8_common(x, W_gate_packed, nullptr, W_up_packed, nullptr, out_codes, out_scales, M, K, N, eps, stream,
                   false);
}

fn_status fn_norm_proj_swiglu_fp8_q8(const void* x, const void* W8_gate, const float* s_gate, const void* W8_up,
                                     const float* s_up, void* out_codes, float* out_scales, int64_t M, int64_t K,
                                     int64_t N, float eps, hipStream_t stream) {
  return q8_common(x, W8_gate, s_gate, W8_up, s_up, out_codes, out_scales, M, K, N, eps, stream, true);
}

const char* fn_kernel_name_q8(int64_t M, int64_t K, int64_t N, int fp8_weights) {
  if (K < 1 || K > kMaxK || K % 8 != 0 || M < 1 || M > kMaxM || N < 1 || N > kMaxN) return "invalid";
  if (M > 64 && !decode_rows_tiled(M, N, fp8_weights != 0))
    return fn::plan_prefill(fn::DType::BF16, M, K, N, true, true, false, fp8_weights != 0).name;
  return fn::plan_decode_q8(fp8_weights != 0, M, N).name;
}

fn_status fn_adaln_shift_bias(const void* shift, const void* W, float* bias, int64_t T, int64_t K, int64_t N,
                              fn_dtype dt, hipStream_t stream) {
  g_last_error[0] = '\0';
  if (!dtype_ok(dt)) return fail(FN_ERR_DTYPE, "unknown dtype %d", (int)dt);
  FN_TRY(check_k(K));
  FN_TRY(check_mn(0, N));
  if (T < 0 || T > INT32_MAX || T * K * esize(dt) > INT32_MAX || T * N > INT32_MAX)
    return fail(FN_ERR_SHAPE, "T=%lld out of range (T*K*e and T*N must stay below 2^31)", (long long)T);
  if (T == 0 || N == 0) return FN_OK;
  if (shift == nullptr || W == nullptr || bias == nullptr) return fail(FN_ERR_NULL, "shift, W or bias is NULL");
  const int64_t e = esize(dt);
  if (!aligned(shift, (uintptr_t)e) || !aligned(W, (uintptr_t)e) || !aligned(bias, 4))
    return fail(FN_ERR_ALIGN, "shift and W need their element alignment, bias 4 bytes");
  if (overlap(bias, T * N * 4, shift, T * K * e) || overlap(bias, T * N * 4, W, K * N * e))
    return fail(FN_ERR_ALIAS, "bias overlaps shift or W");
  return hip_status(fn::launch_adaln_bias(to_dt(dt), shift, W, bias, (int)T, (int)K, (int)N, stream), "adaln_bias");
}

fn_status fn_adaln_fold_table(const void* g, const void* scale, float* mod, int64_t T, int64_t K, fn_dtype dt,
                              hipStream_t stream) {
  g_last_error[0] = '\0';
  if (!dtype_ok(dt)) return fail(FN_ERR_DTYPE, "unknown dtype %d", (int)dt);
  FN_TRY(check_k(K));
  if (T < 0 || T > INT32_MAX || T * K * 4 > INT32_MAX)
    return fail(FN_ERR_SHAPE, "T=%lld out of range (T*K*4 must stay below 2^31)", (long long)T);
  if (T == 0) return FN_OK;
  if (g == nullptr || scale == nullptr || mod == nullptr) return fail(FN_ERR_NULL, "g, scale or mod is NULL");
  const int64_t e = esize(dt);
  if (!aligned(g, (uintptr_t)e) || !aligned(scale, (uintptr_t)e) || !aligned(mod, 4))
    return fail(FN_ERR_ALIGN, "g and scale need their element alignment, mod 4 bytes");
  if (overlap(mod, T * K * 4, g, K * e) || overlap(mod, T * K * 4, scale, T * K * e))
    return fail(FN_ERR_ALIAS, "mod overlaps g or scale");
  return hip_status(fn::launch_adaln_fold_table(to_dt(dt), g, scale, mod, (int)T, (int)K, stream), "adaln_fold_table");
}

fn_status fn_norm_proj_adaln(const void* x, const float* mod, const int* idx, const void* W_packed, const float* bias,
                             void* y, int64_t M, int64_t K, int64_t N, int64_t T, float eps, hipStream_t stream) {
  return adaln_common(x, mod, idx, W_packed, bias, nullptr, nullptr, y, M, K, N, T, eps, stream, false);
}

fn_status fn_norm_proj_swiglu_adaln(const void* x, const float* mod, const int* idx, const void* W_gate_packed,
                                    const float* bias_gate, const void* W_up_packed, const float* bias_up, void* out,
                                    int64_t M, int64_t K, int64_t N, int64_t T, float eps, hipStream_t stream) {
  return adaln_common(x, mod, idx, W_gate_packed, bias_gate, W_up_packed, bias_up, out, M, K, N, T, eps, stream,
                      true);
}

const char* fn_kernel_name_adaln(int64_t M, int64_t K, int64_t N, int64_t T, int swiglu) {
  if (K < 1 || K > kMaxK || K % 8 != 0 || M < 1 || M > kAdalnOneLaunchRows || N < 1 || N > kMaxN || T < 1)
    return "invalid";
  return fn::plan_adaln(M, N, swiglu != 0).name;
}

int64_t fn_adaln_workspace_bytes(int64_t M, int64_t K) {
  if (K < 1 || K > kMaxK || K % 8 != 0 || M < 0 || M > kMaxM || M <= kAdalnOneLaunchRows) return 0;
  return adaln_ws_need(M, K);
}

fn_status fn_norm_proj_adaln_ws(const void* x, const float* mod, const int* idx, const void* W_packed,
                                const float* bias, void* y, int64_t M, int64_t K, int64_t N, int64_t T, float eps,
                                void* workspace, int64_t workspace_bytes, hipStream_t stream) {
  return adaln_ws_common(x, mod, idx, W_packed, bias, nullptr, nullptr, y, M, K, N, T, eps, workspace,
                         workspace_bytes, stream, false);
}

fn_status fn_norm_proj_swiglu_adaln_ws(const void* x, const float* mod, const int* idx, const void* W_gate_packed,
                                       const float* bias_gate, const void* W_up_packed, const float* bias_up,
                                       void* out, int64_t M, int64_t K, int64_t N, int64_t T, float eps,
                                       void* workspace, int64_t workspace_bytes, hipStream_t stream) {
  return adaln_ws_common(x, mod, idx, W_gate_packed, bias_gate, W_up_packed, bias_up, out, M, K, N, T, eps,
                         workspace, workspace_bytes, stream, true);
}

// ---------------------------------------------------------------------------
// The same SwiGLU AdaLN call for callers that cannot allocate: its workspace
// is this library's own device array.  In host code `scratch` names a
// host-side stand-in, not the device memory: the device address of each
// GPU's copy is looked up once per device (hipGetSymbolAddress, with that
// device current) and only that address is passed to kernels.
// ---------------------------------------------------------------------------
constexpr int64_t kScratchBytes = (int64_t(64) << 20) + (int64_t(64) << 10);
static __device__ __align__(256) uint8_t scratch[kScratchBytes];

namespace {
constexpr int kMaxDevices = 64;
std::mutex g_scratch_mutex;
void* g_scratch_ptr[kMaxDevices] = {};

// The current device's copy of `scratch`, looked up on its first use there.
fn_status scratch_for_current_device(void** out) {
  int dev = -1;
  FN_TRY(hip_status(hipGetDevice(&dev), "hipGetDevice"));
  if (dev < 0 || dev >= kMaxDevices) return fail(FN_ERR_HIP, "device %d out of the supported range", dev);
  std::lock_guard<std::mutex> lock(g_scratch_mutex);
  if (g_scratch_ptr[dev] == nullptr) {
    void* p = nullptr;
    FN_TRY(hip_status(hipGetSymbolAddress(&p, HIP_SYMBOL(scratch)), "hipGetSymbolAddress(scratch)"));
    if (p == nullptr) return fail(FN_ERR_HIP, "hipGetSymbolAddress(scratch) returned NULL");
    g_scratch_ptr[dev] = p;
  }
  *out = g_scratch_ptr[dev];
  return FN_OK;
}
}  // namespace

int64_t fn_norm_proj_swiglu_adaln_static_max_bytes(void) { return kScratchBytes; }

fn_status fn_norm_proj_swiglu_adaln_static(const void* x, const float* mod, const int* idx, const void* W_gate_packed,
                                           const float* bias_gate, const void* W_up_packed, const float* bias_up,
                                           void* out, int64_t M, int64_t K, int64_t N, int64_t T, float eps,
                                           hipStream_t stream) {
  g_last_error[0] = '\0';
  // arguments first (no HIP call on a bad call), then the size limit
  FN_TRY(adaln_common(x, mod, idx, W_gate_packed, bias_gate, W_up_packed, bias_up, out, M, K, N, T, eps, stream,
                      true, true));
  if (M == 0 || N == 0) return FN_OK;
  if (M <= kAdalnOneLaunchRows)
    return adaln_common(x, mod, idx, W_gate_packed, bias_gate, W_up_packed, bias_up, out, M, K, N, T, eps, stream,
                        true);
  const int64_t need = adaln_ws_need(M, K, true);
  if (need > kScratchBytes)
    return fail(FN_ERR_SHAPE, "M=%lld, K=%lld need %lld bytes of scratch; the static scratch holds %lld",
                (long long)M, (long long)K, (long long)need, (long long)kScratchBytes);
  void* ws = nullptr;
  FN_TRY(scratch_for_current_device(&ws));
  return adaln_ws_common(x, mod, idx, W_gate_packed, bias_gate, W_up_packed, bias_up, out, M, K, N, T, eps, ws,
                         kScratchBytes, stream, true);
}

const char* fn_kernel_name_adaln_ws(int64_t M, int64_t K, int64_t N, int64_t T, int swiglu) {
  if (K < 1 || K > kMaxK || K % 8 != 0 || M < 1 || M > kMaxM || N < 1 || N > kMaxN || T < 1) return "invalid";
  if (M > 64 && !premod_rows_tiled(M, N, false, swiglu != 0))
    return fn::plan_prefill(fn::DType::BF16, M, K, N, swiglu != 0, false, true).name;
  if (M > kAdalnOneLaunchRows) return fn::plan_decode_premod(M, N, swiglu != 0).name;
  return fn_kernel_name_adaln(M, K, N, T, swiglu);
}

int64_t fn_adaln_prepass_bytes(int64_t M, int64_t K) {
  if (K < 1 || K > kMaxK || K % 8 != 0 || M < 1 || M > kMaxM) return 0;
  return adaln_ws_need(M, K);
}

fn_status fn_norm_proj_adaln_fp8_ws(const void* x, const float* mod, const int* idx, const void* W8_packed,
                                    const float* scales, const float* bias, void* y, int64_t M, int64_t K, int64_t N,
                                    int64_t T, float eps, void* workspace, int64_t workspace_bytes,
                                    hipStream_t stream) {
  return adaln_fp8_ws_common(x, mod, idx, W8_packed, scales, bias, nullptr, nullptr, nullptr, y, M, K, N, T, eps,
                             workspace, workspace_bytes, stream, false);
}

fn_status fn_norm_proj_swiglu_adaln_fp8_ws(const void* x, const float* mod, const int* idx, const void* W8_gate,
                                           const float* s_gate, const float* bias_gate, const void* W8_up,
                                           const float* s_up, const float* bias_up, void* out, int64_t M, int64_t K,
                                           int64_t N, int64_t T, float eps, void* workspace, int64_t workspace_bytes,
                                           hipStream_t stream) {
  return adaln_fp8_ws_common(x, mod, idx, W8_gate, s_gate, bias_gate, W8_up, s_up, bias_up, out, M, K, N, T, eps,
                             workspace, workspace_bytes, stream, true);
}

const char* fn_kernel_name_adaln_fp8(int64_t M, int64_t K, int64_t N, int64_t T, int swiglu) {
  if (K < 1 || K > kMaxK || K % 8 != 0 || M < 1 || M > kMaxM || N < 1 || N > kMaxN || T < 1) return "invalid";
  if (M > 64 && !premod_rows_tiled(M, N, true, swiglu != 0))
    return fn::plan_prefill(fn::DType::BF16, M, K, N, swiglu != 0, false, true, true).name;
  return fn::plan_decode_premod(M, N, swiglu != 0, true).name;
}

fn_status fn_norm_proj_swiglu_adaln_q8_ws(const void* x, const float* mod, const int* idx, const void* W_gate_packed,
                                          const float* bias_gate, const void* W_up_packed, const float* bias_up,
                                          void* out_codes, float* out_scales, int64_t M, int64_t K, int64_t N,
                                          int64_t T, float eps, void* workspace, int64_t workspace_bytes,
                                          hipStream_t stream) {
  return adaln_q8_ws_common(x, mod, idx, W_gate_packed, nullptr, bias_gate, W_up_packed, nullptr, bias_up, out_codes,
                            out_scales, M, K, N, T, eps, workspace, workspace_bytes, stream, false);
}

fn_status fn_norm_proj_swiglu_adaln_fp8_q8_ws(const void* x, const float* mod, const int* idx, const void* W8_gate,
                                              const float* s_gate, const float* bias_gate, const void* W8_up,
                                              const float* s_up, const float* bias_up, void* out_codes,
                                              float* out_scales, int64_t M, int64_t K, int64_t N, int64_t T,
                                              float eps, void* workspace, int64_t workspace_bytes,
                                              hipStream_t stream) {
  return adaln_q8_ws_common(x, mod, idx, W8_gate, s_gate, bias_gate, W8_up, s_up, bias_up, out_codes, out_scales, M,
                            K, N, T, eps, workspace, workspace_bytes, stream, true);
}

const char* fn_kernel_name_adaln_q8(int64_t M, int64_t K, int64_t N, int64_t T, int fp8_weights) {
  if (K < 1 || K > kMaxK || K % 8 != 0 || M < 1 || M > kMaxM || N < 1 || N > kMaxN || T < 1) return "invalid";
  if (M > 64 && !premod_rows_tiled(M, N, fp8_weights != 0, false))
    return fn::plan_prefill(fn::DType::BF16, M, K, N, true, true, true, fp8_weights != 0).name;
  return fn::plan_decode_q8_premod(fp8_weights != 0, M, N).name;
}

fn_status fn_adaln_modulate(const void* x, const float* mod, const int* idx, void* u, float* rs, int64_t M,
                            int64_t K, int64_t T, float eps, hipStream_t stream) {
  g_last_error[0] = '\0';
  FN_TRY(check_k(K));
  FN_TRY(check_mn(M, 0));
  FN_TRY(check_eps(eps));
  if (T < 1 || T > INT32_MAX || T * K * 4 > INT32_MAX)
    return fail(FN_ERR_SHAPE, "T=%lld must be >= 1 with T*K*4 < 2^31", (long long)T);
  if (M == 0) return FN_OK;
  if (x == nullptr || mod == nullptr || idx == nullptr) return fail(FN_ERR_NULL, "x, mod or idx is NULL");
  if (u == nullptr || rs == nullptr) return fail(FN_ERR_NULL, "u or rs is NULL");
  if (!aligned(x, 16) || !aligned(mod, 16) || !aligned(u, 16))
    return fail(FN_ERR_ALIGN, "x, mod and u must be 16-byte aligned");
  if (!aligned(idx, 4) || !aligned(rs, 4)) return fail(FN_ERR_ALIGN, "idx and rs must be 4-byte aligned");
  const int64_t xb = M * K * 2;
  if (overlap(u, xb, x, xb) || overlap(u, xb, mod, T * K * 4) || overlap(u, xb, idx, M * 4) ||
      overlap(rs, M * 4, x, xb) || overlap(rs, M * 4, mod, T * K * 4) || overlap(rs, M * 4, idx, M * 4) ||
      overlap(u, xb, rs, M * 4))
    return fail(FN_ERR_ALIAS, "output overlaps an input");
  return hip_status(fn::launch_adaln_modulate(x, mod, idx, (int)T, u, rs, (int)M, (int)K, eps, stream),
                    "adaln_modulate");
}

fn_status fn_step_create(const fn_call* calls, int64_t n_calls, fn_step* out) {
  g_last_error[0] = '\0';
  if (out == nullptr) return fail(FN_ERR_NULL, "out is NULL");
  *out = nullptr;
  if (calls == nullptr) return fail(FN_ERR_NULL, "calls is NULL");
  if (n_calls < 1 || n_calls > (int64_t(1) << 20))
    return fail(FN_ERR_SHAPE, "n_calls=%lld must be in [1, 2^20]", (long long)n_calls);
  int64_t kernels = 0;
  for (int64_t i = 0; i < n_calls; ++i) {
    const fn_status s = run_call(calls[i], nullptr, true);
    if (s != FN_OK) return call_failed(s, i);
    if (calls[i].M > 0 && calls[i].N > 0) ++kernels;
  }
  // Record on a private stream (default priority), then instantiate.
  hipStream_t cs = nullptr;
  FN_TRY(hip_status(hipStreamCreateWithFlags(&cs, hipStreamNonBlocking), "step: stream"));
  fn_status st = hip_status(hipStreamBeginCapture(cs, hipStreamCaptureModeThreadLocal), "step: begin capture");
  if (st == FN_OK) {
    for (int64_t i = 0; i < n_calls && st == FN_OK; ++i) {
      st = run_call(calls[i], cs, false);
      if (st != FN_OK) st = call_failed(st, i);
    }
    hipGraph_t graph = nullptr;
    const fn_status end = hip_status(hipStreamEndCapture(cs, &graph), "step: end capture");
    if (st == FN_OK) st = end;
    hipGraphExec_t exec = nullptr;
    if (st == FN_OK) st = hip_status(hipGraphInstantiate(&exec, graph, nullptr, nullptr, 0), "step: instantiate");
    if (st == FN_OK) {
      fn_step h = new (std::nothrow) fn_step_s;
      if (h == nullptr) {
        st = fail(FN_ERR_HIP, "step: out of host memory");
      } else {
        h->graph = graph;
        h->exec = exec;
        h->kernels = kernels;
        *out = h;
      }
    }
    if (st != FN_OK) {
      if (exec != nullptr) (void)hipGraphExecDestroy(exec);
      if (graph != nullptr) (void)hipGraphDestroy(graph);
    }
  }
  (void)hipStreamDestroy(cs);
  return st;
}

namespace {
struct Span {
  uintptr_t lo, hi;
  bool out;
  int64_t call;
};

// Furthest end reached so far, kept per call: the largest end, its call,
// and the largest end among the other calls, so that the furthest reach of
// every call but a given one is known.
struct Reach {
  uintptr_t end1 = 0, end2 = 0;
  int64_t call1 = -1;
  void add(uintptr_t e, int64_t c) {
    if (c == call1) {
      end1 = std::max(end1, e);
    } else if (e > end1) {
      end2 = end1;
      end1 = e;
      call1 = c;
    } else {
      end2 = std::max(end2, e);
    }
  }
  uintptr_t other_than(int64_t c) const { return c == call1 ? end2 : end1; }
};

// True if an output of one call overlaps any buffer of another call: sorted
// by start, a span overlaps an earlier span of another call exactly when it
// starts before that call's furthest end; an output is checked against
// every earlier span, any span against earlier outputs.
bool outputs_overlap(std::vector<Span>& v) {
  std::sort(v.begin(), v.end(), [](const Span& a, const Span& b) { return a.lo < b.lo; });
  Reach outs, any;
  for (const Span& s : v) {
    if (s.lo < outs.other_than(s.call)) return true;
    if (s.out && s.lo < any.other_than(s.call)) return true;
    if (s.out) outs.add(s.hi, s.call);
    any.add(s.hi, s.call);
  }
  return false;
}
}  // namespace

namespace {
fn_status step_create_grouped(const fn_call* calls, int64_t n_calls, fn_step* out);
}  // namespace

fn_status fn_step_create_grouped(const fn_call* calls, int64_t n_calls, fn_step* out) {
  g_last_error[0] = '\0';
  // host tables of up to 2^31 entries: allocation failure is a status, not an exception
  try {
    return step_create_grouped(calls, n_calls, out);
  } catch (const std::bad_alloc&) {
    return fail(FN_ERR_HIP, "grouped step: out of host memory");
  }
}

namespace {
fn_status step_create_grouped(const fn_call* calls, int64_t n_calls, fn_step* out) {
  if (out == nullptr) return fail(FN_ERR_NULL, "out is NULL");
  *out = nullptr;
  if (calls == nullptr) return fail(FN_ERR_NULL, "calls is NULL");
  if (n_calls < 1 || n_calls > 65535) return fail(FN_ERR_SHAPE, "n_calls=%lld must be in [1, 65535]", (long long)n_calls);
  std::vector<Span> spans;
  int64_t items = 0;
  const bool f8 = calls[0].kind == FN_CALL_NORM_PROJ_FP8 || calls[0].kind == FN_CALL_NORM_PROJ_SWIGLU_FP8;
  for (int64_t i = 0; i < n_calls; ++i) {
    const fn_call& c = calls[i];
    const fn_status s = run_call(c, nullptr, true);
    if (s != FN_OK) return call_failed(s, i);
    const bool bf = c.kind == FN_CALL_NORM_PROJ || c.kind == FN_CALL_NORM_PROJ_SWIGLU;
    const bool c8 = c.kind == FN_CALL_NORM_PROJ_FP8 || c.kind == FN_CALL_NORM_PROJ_SWIGLU_FP8;
    if (!bf && !c8)
      return call_failed(fail(FN_ERR_SHAPE, "a grouped step takes fn_norm_proj, fn_norm_proj_swiglu and their fp8 "
                                            "forms"), i);
    if (c8 != f8)
      return call_failed(fail(FN_ERR_SHAPE, "a grouped step takes calls of one weight type (all bf16 or all fp8)"),
                         i);
    if ((bf && c.dt != FN_BF16) || c.M > 128)
      return call_failed(fail(FN_ERR_SHAPE, "a grouped step takes bf16 activations of at most 128 rows (M=%lld)",
                              (long long)c.M), i);
    if (c.M == 0 || c.N == 0) continue;
    const bool sw = c.kind == FN_CALL_NORM_PROJ_SWIGLU || c.kind == FN_CALL_NORM_PROJ_SWIGLU_FP8;
    const int64_t wb = f8 ? packed_fp8_bytes(c.K, c.N) : packed_bytes(c.K, c.N, FN_BF16);
    auto add = [&](const void* p, int64_t bytes, bool o) {
      const uintptr_t lo = reinterpret_cast<uintptr_t>(p);
      spans.push_back(Span{lo, lo + (uintptr_t)bytes, o, i});
    };
    add(c.x, c.M * c.K * 2, false);
    add(c.w_gate, wb, false);
    if (sw) add(c.w_up, wb, false);
    if (f8) {
      add(c.s_gate, c.N * 4, false);
      if (sw) add(c.s_up, c.N * 4, false);
    }
    add(c.y, c.M * c.N * 2, true);
  }
  // up to 16 rows in every call: the one-wave register-x tiles; else every
  // call takes the LDS-shared-x tile, 64 rows per workgroup (more rows in
  // more workgroups)
  bool wide = false;
  for (int64_t i = 0; i < n_calls; ++i) wide = wide || (calls[i].N > 0 && calls[i].M > 16);
  auto per_item = [&](const fn_call& c) {
    const bool sw = c.kind == FN_CALL_NORM_PROJ_SWIGLU || c.kind == FN_CALL_NORM_PROJ_SWIGLU_FP8;
    return wide ? fn::kGroupedXBlocks : fn::grouped_blocks(f8, sw);
  };
  // workgroups of a call: its column groups; in the wide tile with more than
  // one 64-row block, the groups padded to a multiple of 8 times the row
  // blocks (the kernel's XCD-aware order)
  auto call_items = [&](const fn_call& c) -> int64_t {
    const int64_t groups = ((c.N + 15) / 16 + per_item(c) - 1) / per_item(c);
    const int64_t rowblocks = (c.M + 63) / 64;
    return wide && rowblocks > 1 ? (groups + 7) / 8 * 8 * rowblocks : groups;
  };
  for (int64_t i = 0; i < n_calls; ++i) {
    const fn_call& c = calls[i];
    if (c.M == 0 || c.N == 0) continue;
    items += call_items(c);
  }
  if (outputs_overlap(spans))
    return fail(FN_ERR_ALIAS, "a grouped step runs its calls at once: no call may write a buffer another call uses");
  if (items > INT32_MAX) return fail(FN_ERR_SHAPE, "a grouped step holds at most 2^31-1 workgroups");
  const size_t rec = wide ? fn::grouped_x_call_bytes() : fn::grouped_call_bytes();
  std::vector<uint8_t> host_calls((size_t)n_calls * rec);
  std::vector<uint16_t> host_items((size_t)items);
  int64_t first = 0;
  for (int64_t i = 0; i < n_calls; ++i) {
    const fn_call& c = calls[i];
    const bool sw = c.kind == FN_CALL_NORM_PROJ_SWIGLU || c.kind == FN_CALL_NORM_PROJ_SWIGLU_FP8;
    (wide ? fn::grouped_x_call_fill : fn::grouped_call_fill)(
        host_calls.data() + (size_t)i * rec, c.x, c.w_gate, sw ? c.w_up : nullptr, f8 ? c.s_gate : nullptr,
        f8 && sw ? c.s_up : nullptr, c.y, (int)c.M, (int)c.K, (int)c.N, c.eps, (int)first);
    if (c.M == 0 || c.N == 0) continue;
    const int64_t nb = call_items(c);   // workgroups of this call
    for (int64_t b = 0; b < nb; ++b) host_items[(size_t)(first + b)] = (uint16_t)i;
    first += nb;
  }
  fn_step h = new (std::nothrow) fn_step_s;
  if (h == nullptr) return fail(FN_ERR_HIP, "step: out of host memory");
  h->grouped = true;
  h->fp8 = f8;
  h->wide = wide;
  if (items == 0) {   // every call empty: the step launches nothing
    *out = h;
    return FN_OK;
  }
  fn_status st = hip_status(hipMalloc(&h->calls, host_calls.size()), "grouped step: allocate calls");
  if (st == FN_OK) st = hip_status(hipMalloc(&h->items, host_items.size() * 2), "grouped step: allocate items");
  if (st == FN_OK)
    st = hip_status(hipMemcpy(h->calls, host_calls.data(), host_calls.size(), hipMemcpyHostToDevice),
                    "grouped step: copy calls");
  if (st == FN_OK)
    st = hip_status(hipMemcpy(h->items, host_items.data(), host_items.size() * 2, hipMemcpyHostToDevice),
                    "grouped step: copy items");
  if (st != FN_OK) {
    if (h->calls != nullptr) (void)hipFree(h->calls);
    if (h->items != nullptr) (void)hipFree(h->items);
    delete h;
    return st;
  }
  h->nitems = items;
  h->kernels = 1;
  *out = h;
  return FN_OK;
}
}  // namespace

fn_status fn_step_launch(fn_step step, hipStream_t stream) {
  g_last_error[0] = '\0';
  if (step == nullptr) return fail(FN_ERR_NULL, "step is NULL");
  if (step->grouped)
    return step->nitems == 0 ? FN_OK
           : hip_status(step->wide ? fn::launch_decode_x_grouped(step->calls, step->items, (int)step->nitems,
                                                                 step->fp8, stream)
                                   : fn::launch_decode_grouped(step->calls, step->items, (int)step->nitems,
                                                               step->fp8, stream),
                        "grouped step: launch");
  return hip_status(hipGraphLaunch(step->exec, stream), "step: launch");
}

int64_t fn_step_num_kernels(fn_step step) { return step == nullptr ? -1 : step->kernels; }

fn_status fn_step_destroy(fn_step step) {
  g_last_error[0] = '\0';
  if (step == nullptr) return FN_OK;
  fn_status st = FN_OK;
  if (step->grouped) {
    if (step->calls != nullptr) st = hip_status(hipFree(step->calls), "grouped step: free calls");
    const fn_status s2 =
        step->items == nullptr ? FN_OK : hip_status(hipFree(step->items), "grouped step: free items");
    if (st == FN_OK) st = s2;
  } else {
    st = hip_status(hipGraphExecDestroy(step->exec), "step: destroy exec");
    const fn_status s2 = hip_status(hipGraphDestroy(step->graph), "step: destroy graph");
    if (st == FN_OK) st = s2;
  }
  delete step;
  return st;
}

const char* fn_kernel_name_fp8(int64_t M, int64_t K, int64_t N, int swiglu) {
  if (K < 1 || K > kMaxK || K % 8 != 0 || M < 1 || M > kMaxM || N < 1 || N > kMaxN) return "invalid";
  if (M > 64 && !decode_rows_tiled(M, N, true))
    return fn::plan_prefill(fn::DType::BF16, M, K, N, swiglu != 0, false, false, true).name;
  if (fn::fp8_k_split(M, N, swiglu != 0) != 0) return fn::plan_fp8_ksplit(M, N, swiglu != 0).name;
  return fn::plan_fp8(M, K, N, swiglu != 0).name;
}

const char* fn_kernel_name(int64_t M, int64_t K, int64_t N, int swiglu, fn_dtype dt) {
  if (!dtype_ok(dt) || K < 1 || K > kMaxK || K % 8 != 0 || M < 1 || M > kMaxM || N < 1 || N > kMaxN)
    return "invalid";
  return fn::plan_fused(to_dt(dt), M, K, N, swiglu != 0).name;
}

const char* fn_status_string(fn_status s) {
  switch (s) {
    case FN_OK: return "ok";
    case FN_ERR_NULL: return "null pointer";
    case FN_ERR_SHAPE: return "shape out of range";
    case FN_ERR_ALIGN: return "misaligned pointer";
    case FN_ERR_DTYPE: return "unknown dtype";
    case FN_ERR_EPS: return "eps must be finite and non-negative";
    case FN_ERR_ALIAS: return "output overlaps an input";
    case FN_ERR_HIP: return "HIP launch failed";
    case FN_ERR_WORKSPACE: return "workspace missing, misaligned or too small";
  }
  return "unknown status";
}

const char* fn_last_error(void) { return g_last_error; }

}  // extern "C"
