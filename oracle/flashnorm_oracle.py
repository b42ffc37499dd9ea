"""Plain float64 CPU oracle for fused RMSNorm + projection (FlashNorm).

TEST INFRASTRUCTURE.  Only the tests, the smoke check and the benchmark's
CPU-baseline leg may import or call this module.  The product path (the HIP
library and its Python binding) never does, and shares no code with it.

What it computes, and where the pages state it
----------------------------------------------
Sources (web pages; cited by title and section):

* [FlashNorm digest] "RMS norm는 연산량 1할인데 왜 33번 호출로 속도를 갉아먹나"
  (news.juniverse.app feature, 2026-09-20), summary bullets:
  - proposal 1, weightless normalisation: the norm's gain is folded offline
    into the projection weights, leaving a single matrix;
  - proposal 2, deferred normalisation: the per-row scalar division is moved
    after the matrix product so matrix and vector units can run together;
  - proposal 3, double-norm removal: scale invariance makes the second of two
    back-to-back RMS norms redundant.
* [FlashInfer #5521] "MiniMax-H3 Fused FC1 + SwiGLU" analysis, sections
  "Segmented Chain" (norm -> GEMM -> silu_and_mul as separate steps) and
  "Design" item 2 (SwiGLU applied to the GEMM accumulators in registers).
* [FlashInfer #4040] "Fused SwiGLU 및 NVFP4 양자화", section "하드웨어 최적화"
  (fp32 -> bf16 conversion rounds to nearest, ties to even).
* [FlashInfer #5668] "Kimi-K3 TP12 LatentMoE Tail", section on K23_LADDER
  (keep fp32 through the whole sum and round to bf16 once; judge accuracy
  against a float64 reference).

The pages never write the RMSNorm formula.  Every proposal above presupposes
standard RMSNorm with a gain, so the oracle takes the plain reading

    r[m]      = sqrt( (1/K) * sum_k x[m,k]^2 + eps )
    xhat[m,k] = x[m,k] / r[m] * g[k]
    y[m,n]    = sum_k xhat[m,k] * W[k,n]

with eps inside the square root and the mean over the hidden size K.  The
SwiGLU variant computes a = xhat @ W_gate, b = xhat @ W_up and
out = a * sigmoid(a) * b (the gate is the operand inside the SiLU).  Folding
and deferral are exact in real arithmetic, so the oracle computes the
unfolded definition directly; the folded/deferred form exists only to pin
that equality.

All arithmetic is float64.  Inputs are the stored (bf16 or fp32) values,
up-cast exactly.  eps is taken as float64(float32(eps)), the exact value a
GPU kernel receives as a float argument.

The fp8-weight functions (E4M3 codes with one scale per output column) and
the fp8 output functions (E4M3 codes with one scale per 16-column row
block) and the AdaLN functions at the end follow the readings stated in
their sections.

Pins (see tests/test_oracle.py): hand-derived worked cases, brute force on
tiny inputs, torch's float64 rms_norm followed by a float64 matmul, the fold
identity, scale invariance, norm-after-weightless-norm, row permutation and
column concatenation, library round-to-nearest-even conversions (bf16, and
torch's float8_e4m3fn for the E4M3 codes), hand-evaluated E4M3 codes, the
quantisation error bound, and the exact reduction of the fp8 path to the
deferred form when the weights are E4M3-exact.  Every function here is
pinned; none is "parity unpinned".
"""
from __future__ import annotations

import numpy as np


def _f64(a) -> np.ndarray:
    return np.asarray(a, dtype=np.float64)


def eps_as_received(eps: float) -> float:
    """eps as a float32 kernel argument carries it, widened to float64."""
    return float(np.float32(eps))


def rms(x, eps: float) -> np.ndarray:
    """Per-row root mean square with eps inside the root (the plain RMSNorm
    reading of [FlashNorm digest] proposals 1-3): r[m] = sqrt(mean_k x^2 + eps)."""
    x = _f64(x)
    K = x.shape[-1]
    mean_sq = np.sum(x * x, axis=-1) / K
    return np.sqrt(mean_sq + eps_as_received(eps))


def rmsnorm(x, g, eps: float) -> np.ndarray:
    """xhat = x / r * g, row by row ([FlashNorm digest]: the norm the proposals
    act on; g is the gain that proposal 1 folds away)."""
    x = _f64(x)
    g = _f64(g)
    return x / rms(x, eps)[..., None] * g


def norm_proj(x, g, W, eps: float) -> np.ndarray:
    """Unfolded definition y = RMSNorm_g(x) @ W: the norm followed by the
    projection that [FlashNorm digest] fuses."""
    return rmsnorm(x, g, eps) @ _f64(W)


def silu(a) -> np.ndarray:
    """SiLU(a) = a * sigmoid(a) = a / (1 + exp(-a)) ([FlashInfer #5521]
    silu_and_mul step of the segmented chain)."""
    a = _f64(a)
    return a / (1.0 + np.exp(-a))


def norm_proj_swiglu(x, g, W_gate, W_up, eps: float) -> np.ndarray:
    """SwiGLU after the normalised gate and up projections:
    out = silu(xhat @ W_gate) * (xhat @ W_up) ([FlashInfer #5521], chain
    steps "GEMM" then "silu_and_mul"; the fused kernel's register epilogue
    computes the same function).  Both products see the normalised xhat, so
    the 1/r factor reaches a before the nonlinearity."""
    xhat = rmsnorm(x, g, eps)
    a = xhat @ _f64(W_gate)
    b = xhat @ _f64(W_up)
    return silu(a) * b


def fold_exact(g, W) -> np.ndarray:
    """Weightless normalisation, before storage rounding: W'[k,n] = g[k]*W[k,n]
    ([FlashNorm digest] proposal 1).  For bf16 or fp32 operands the float64
    product is exact."""
    return _f64(g)[:, None] * _f64(W)


def round_to_bf16(a) -> np.ndarray:
    """Round float64 values to the nearest bf16 value, ties to even
    ([FlashInfer #4040]: the fp32 -> bf16 conversion is round-to-nearest-even).

    bf16 keeps 8 significant bits and fp32's exponent range: the quantum of a
    value m*2^e (0.5 <= |m| < 1) is 2^(e-8), held at 2^-133 below the
    smallest normal 2^-126.  Results of magnitude 2^128 or more overflow to
    infinity.  NaN stays NaN."""
    a = _f64(a)
    with np.errstate(invalid="ignore", over="ignore"):
        _, e = np.frexp(a)
        e = np.maximum(e, -125)
        q = np.ldexp(np.rint(np.ldexp(a, 8 - e)), e - 8)   # np.rint: half to even
        q = np.where(np.abs(q) >= 2.0 ** 128, np.copysign(np.inf, a), q)
    return q


def round_to_f32(a) -> np.ndarray:
    """Round float64 values to the nearest float32 (numpy's cast is IEEE
    round-to-nearest-even)."""
    return _f64(a).astype(np.float32).astype(np.float64)


def round_to(a, dtype: str) -> np.ndarray:
    if dtype == "bf16":
        return round_to_bf16(a)
    if dtype == "f32":
        return round_to_f32(a)
    raise ValueError(f"unknown dtype {dtype!r}")


def fold_weights(g, W, dtype: str) -> np.ndarray:
    """Stored folded weights: W' = round_dtype(g[k] * W[k,n]), one rounding of
    the exact product ([FlashNorm digest] proposal 1; single rounding as in
    [FlashInfer #5668]).  Returned as float64 holding the stored values."""
    return round_to(fold_exact(g, W), dtype)


def norm_proj_folded(x, W_folded, eps: float) -> np.ndarray:
    """Deferred normalisation on folded weights: y = (x @ W') / r, the scalar
    division moved after the product ([FlashNorm digest] proposal 2).  Used
    only to pin that this equals the unfolded definition."""
    x = _f64(x)
    return (x @ _f64(W_folded)) / rms(x, eps)[:, None]


def norm_proj_swiglu_folded(x, Wg_folded, Wu_folded, eps: float) -> np.ndarray:
    """Deferred form of the SwiGLU variant: a = (x @ W'_g)/r, b = (x @ W'_u)/r,
    out = silu(a) * b.  Used only to pin equality with the unfolded form."""
    x = _f64(x)
    r = rms(x, eps)[:, None]
    a = (x @ _f64(Wg_folded)) / r
    b = (x @ _f64(Wu_folded)) / r
    return silu(a) * b


# ------------------------------------------------------------ fp8 weights --
# The pages state that folded weights stay valid for quantised models
# ([FlashNorm digest], the compatibility bullet), carry an FP8 variant of the
# fused FC1 + SwiGLU kernel ([FlashInfer #5521], "FP8 Variant" in the
# results), and dequantise low-precision weights in registers right before
# the matrix product ([Fused-kernel memory hierarchy] "Fused 커널은 왜 3~4배
# 빠른가", section "트릭 2": in-register dequantisation).  They fix no format,
# scale granularity or rounding.  The reading taken here:
#
# * format: OCP FP8 E4M3 (1 sign, 4 exponent bits with bias 7, 3 mantissa
#   bits; subnormals; no infinities; codes 0x7F/0xFF are NaN; largest finite
#   magnitude 448), the FP8 format of the target's matrix cores;
# * quantised operand: the folded, stored W' (fold first, as for bf16);
# * one fp32 scale per output column: amax[n] = max_k |W'[k,n]|,
#   r[n] = fp32(448 / amax[n]), codes q = RNE_e4m3(fp32(W'[k,n] * r[n])),
#   dequantisation scale s[n] = fp32(amax[n] / 448); an all-zero column takes
#   r = s = 1.  Every step is one IEEE fp32 operation, so the codes are a
#   deterministic function of W' that a GPU reproduces bit for bit;
# * the product: y[m,n] = s[n] * (sum_k x[m,k] * q[k,n]) / r_rms[m], i.e. the
#   deferred form with the weight decoded exactly (every E4M3 value is a bf16
#   value) and the column scale applied with 1/RMS after the sum.

E4M3_MAX = 448.0


def e4m3_decode(codes) -> np.ndarray:
    """Value of each OCP E4M3 code (uint8): (-1)^s * 2^(e-7) * (1 + m/8) for
    exponent field e > 0, (-1)^s * 2^-6 * (m/8) for e = 0; 0x7F and 0xFF are
    NaN."""
    c = np.asarray(codes, dtype=np.int64) & 0xFF
    sign = np.where(c & 0x80, -1.0, 1.0)
    e = (c >> 3) & 0xF
    m = (c & 0x7).astype(np.float64)
    val = np.where(e == 0, np.ldexp(m / 8.0, -6), np.ldexp(1.0 + m / 8.0, e - 7))
    val = np.where((c & 0x7F) == 0x7F, np.nan, val)
    return sign * val


def e4m3_encode(a) -> np.ndarray:
    """Code of the E4M3 value nearest to a, ties to even (RNE on the 3-bit
    mantissa, on the 2^-9 grid below the smallest normal 2^-6).  Magnitudes
    at or past the rounding boundary above 448 saturate to 448; NaN gives
    0x7F."""
    a = _f64(a)
    mag = np.abs(a)
    with np.errstate(invalid="ignore", over="ignore", divide="ignore"):
        _, e = np.frexp(mag)                     # mag = f * 2^e, 0.5 <= f < 1
        e = np.maximum(e, -5)                    # below 2^-6: the subnormal quantum 2^-9
        q = np.rint(np.ldexp(mag, 4 - e))        # units of the quantum 2^(e-4); half to even
        val = np.ldexp(q, e - 4)
    val = np.minimum(val, E4M3_MAX)
    # exponent field and mantissa of the rounded magnitude
    _, ev = np.frexp(np.where(val > 0, val, 1.0))
    field = np.where(val >= 2.0 ** -6, ev + 6, 0)        # 2^(ev-1) = 2^(field-7)
    mant = np.where(field > 0, np.ldexp(val, 4 - ev) - 8, np.ldexp(val, 9))
    mant = np.where(np.isnan(mant), 0.0, mant)
    code = (field.astype(np.int64) << 3) | np.rint(mant).astype(np.int64)
    code = np.where(val == 0, 0, code)
    code = code | np.where(np.signbit(a), 0x80, 0)
    code = np.where(np.isnan(a), 0x7F, code)
    return code.astype(np.uint8)


def quantize_e4m3_columns(W_folded):
    """Per-column E4M3 quantisation of stored folded weights (float values of
    bf16 or fp32 storage).  Returns (codes uint8 [K,N], s float32 [N],
    r float32 [N]) as described above."""
    Wf = np.asarray(W_folded, dtype=np.float32)
    amax = np.max(np.abs(Wf), axis=0) if Wf.shape[0] else np.zeros(Wf.shape[1], np.float32)
    zero = amax == 0
    safe = np.where(zero, np.float32(1.0), amax).astype(np.float32)
    r = np.where(zero, np.float32(1.0), np.float32(E4M3_MAX) / safe).astype(np.float32)
    s = np.where(zero, np.float32(1.0), safe / np.float32(E4M3_MAX)).astype(np.float32)
    scaled = (Wf * r[None, :]).astype(np.float32)             # one fp32 multiply
    return e4m3_encode(scaled), s, r


def fold_weights_fp8(g, W, dtype: str):
    """Fold, store in dtype, then quantise per column: (codes, s)."""
    codes, s, _ = quantize_e4m3_columns(fold_weights(g, W, dtype))
    return codes, s


def norm_proj_fp8(x, codes, s, eps: float) -> np.ndarray:
    """Deferred normalisation with E4M3 weights: y = s[n] * (x @ q) / r."""
    x = _f64(x)
    return (x @ e4m3_decode(codes)) * _f64(s)[None, :] / rms(x, eps)[:, None]


def norm_proj_swiglu_fp8(x, codes_gate, s_gate, codes_up, s_up, eps: float) -> np.ndarray:
    """SwiGLU variant with E4M3 weights: a and b as in norm_proj_fp8, then
    out = silu(a) * b."""
    a = norm_proj_fp8(x, codes_gate, s_gate, eps)
    b = norm_proj_fp8(x, codes_up, s_up, eps)
    return silu(a) * b


# ------------------------------------------ fp8 output with block scales --
# The SwiGLU result can leave the kernel already quantised for the next
# projection: [FlashInfer #4040] ("Fused SwiGLU 및 NVFP4 양자화 최적화 분석",
# sections "들어가며" and "Fused Kernel 구현") quantises the silu * up values
# in registers, one scale factor per vector of SF_VEC_SIZE consecutive
# values, instead of writing them and quantising in a second kernel.  The
# page's format is NVFP4; the reading taken here keeps the method and uses
# the fp8 format of the weight path:
#
# * format: OCP E4M3 as above;
# * blocks: 16 consecutive output columns of one row (the vector length of
#   the page's NVFP4 scale factors); the last block of a row is shorter when
#   N % 16 != 0;
# * per block, from the fp32 values v: amax = max |v|, r = fp32(448 / amax),
#   s = fp32(amax / 448) (r = s = 1 for an all-zero block) and
#   codes = RNE_e4m3(fp32(v * r)); the value a consumer reads back is
#   s * decode(code).  The same steps as the per-column weight scales, with
#   the block in place of the column.

Q8_BLOCK = 16


def quantize_e4m3_row_blocks(v, block: int = Q8_BLOCK):
    """Row-block E4M3 quantisation of v [M, N] (taken as fp32 values).
    Returns (codes uint8 [M, N], s float32 [M, ceil(N / block)])."""
    v32 = np.asarray(v, dtype=np.float32)
    M, N = v32.shape
    nb = -(-N // block)
    padded = np.zeros((M, nb * block), dtype=np.float32)   # zero padding leaves every amax unchanged
    padded[:, :N] = v32
    cols = padded.reshape(M * nb, block).T                  # one block per column
    codes, s, _ = quantize_e4m3_columns(cols)
    return np.ascontiguousarray(codes.T.reshape(M, nb * block)[:, :N]), s.reshape(M, nb)


def dequantize_row_blocks(codes, s, block: int = Q8_BLOCK) -> np.ndarray:
    """s[m, n // block] * decode(codes[m, n]) in float64."""
    codes = np.asarray(codes)
    cols = np.arange(codes.shape[1]) // block
    return e4m3_decode(codes) * _f64(s)[:, cols]


def norm_proj_swiglu_q8(x, g, W_gate, W_up, eps: float):
    """The SwiGLU output quantised in row blocks: (codes, s, v), v the
    float64 SwiGLU output it quantises (through fp32)."""
    v = norm_proj_swiglu(x, g, W_gate, W_up, eps)
    codes, s = quantize_e4m3_row_blocks(v)
    return codes, s, v


def norm_proj_swiglu_fp8_q8(x, codes_gate, s_gate, codes_up, s_up, eps: float):
    """E4M3 weights in, row-block E4M3 out: (codes, s, v)."""
    v = norm_proj_swiglu_fp8(x, codes_gate, s_gate, codes_up, s_up, eps)
    codes, s = quantize_e4m3_row_blocks(v)
    return codes, s, v


# ------------------------------------------------------ AdaLN prologue --
# [FlashInfer #5521] ("MiniMax-H3 Fused FC1 + SwiGLU", sections "Segmented
# Chain" and "Fused Kernel on SM120"): the diffusion model's FC1 step runs
# RMSNorm + AdaLN, then the projection, then silu_and_mul, and the fused
# call takes raw x, the norm weight, an AdaLN scale, an AdaLN shift and a
# per-input index into them.  The page never writes the modulation.  The
# reading taken here is the usual adaptive-norm modulation after the norm,
# with the scale and shift rows of two tables [T, K] picked per row of x by
# idx[m]:
#
#     h[m,k] = xhat[m,k] * (1 + scale[idx[m], k]) + shift[idx[m], k],
#     xhat = RMSNorm_g(x),   y = h @ W,   or   out = silu(h @ W_gate) * (h @ W_up).
#
# The modulation is chosen at run time, so it cannot be folded into the
# weights.  The gain can still be folded offline -- here into the
# modulation table instead of W: in real arithmetic
#
#     h @ W = ((x * mod[idx]) @ W) / r + bias[idx],
#     mod[t,k] = g[k] * (1 + scale[t,k]),   bias[t,:] = shift[t,:] @ W,
#
# with W the plain (unfolded) weights.  A matrix-core operand x * mod must be
# rounded to bf16 anyway; folding g into W as well would round every
# product term twice (once in W', once in the operand), so the AdaLN path
# keeps W exact and carries the gain in the table (an fp32 table, one
# rounding of the float64 product).  An index outside [0, T) selects no
# table row: that row's h is taken as 0 (mod row 0, bias row 0), so its
# output is 0.


def adaln_modulate(x, g, scale, shift, idx, eps: float) -> np.ndarray:
    """h = RMSNorm_g(x) * (1 + scale[idx]) + shift[idx], row by row
    (idx within [0, T))."""
    i = np.asarray(idx, dtype=np.int64)
    return rmsnorm(x, g, eps) * (1.0 + _f64(scale)[i]) + _f64(shift)[i]


def adaln_norm_proj(x, g, scale, shift, idx, W, eps: float) -> np.ndarray:
    """y = h @ W with h the AdaLN-modulated normalised x."""
    return adaln_modulate(x, g, scale, shift, idx, eps) @ _f64(W)


def adaln_norm_proj_swiglu(x, g, scale, shift, idx, W_gate, W_up, eps: float) -> np.ndarray:
    """out = silu(h @ W_gate) * (h @ W_up)."""
    h = adaln_modulate(x, g, scale, shift, idx, eps)
    return silu(h @ _f64(W_gate)) * (h @ _f64(W_up))


def adaln_fold_table(g, scale) -> np.ndarray:
    """The gain folded into the modulation table, as stored: mod[t,k] =
    g[k] * (1 + scale[t,k]), the sum and the product taken in float64 and
    the result rounded once to float32.  Returned as float64 holding the
    float32 values."""
    return round_to_f32(_f64(g)[None, :] * (1.0 + _f64(scale)))


def adaln_shift_bias(shift, W) -> np.ndarray:
    """Per-index bias rows shift @ W (unfolded W), [T, N]."""
    return _f64(shift) @ _f64(W)


def _rows_or_zero(table, idx) -> np.ndarray:
    """table[idx[m]] per row, all zero where idx[m] is outside the table."""
    t = _f64(table)
    i = np.asarray(idx, dtype=np.int64)
    ok = (i >= 0) & (i < t.shape[0])
    return np.where(ok[:, None], t[np.where(ok, i, 0)], 0.0)


def adaln_norm_proj_fold(x, W, mod, bias, idx, eps: float) -> np.ndarray:
    """Folded and deferred form: ((x * mod[idx]) @ W) / r + bias[idx], the
    rows of an index outside the table zero.  With mod = g * (1 + scale)
    unrounded it equals adaln_norm_proj in real arithmetic (pinned); with
    the stored (float32) table it is what the kernels compute up to the
    rounding of their bf16 operand and their fp32 sums."""
    x = _f64(x)
    return ((x * _rows_or_zero(mod, idx)) @ _f64(W)) / rms(x, eps)[:, None] + _rows_or_zero(bias, idx)


def adaln_norm_proj_swiglu_fold(x, W_gate, W_up, mod, bias_gate, bias_up, idx, eps: float) -> np.ndarray:
    """SwiGLU on the folded and deferred form: a, b as in
    adaln_norm_proj_fold, out = silu(a) * b."""
    a = adaln_norm_proj_fold(x, W_gate, mod, bias_gate, idx, eps)
    b = adaln_norm_proj_fold(x, W_up, mod, bias_up, idx, eps)
    return silu(a) * b


def adaln_norm_proj_fp8(x, codes, s, mod, bias, idx, eps: float) -> np.ndarray:
    """AdaLN with E4M3 weights (the page's AdaLN FC1 kernel takes
    pre-processed fp8 weights with their scales, [FlashInfer #5521] "Fused
    Kernel on SM120"): the folded/deferred form with the quantised plain
    weights s[n] * q in place of W; bias = shift @ W from the bf16 weights."""
    return adaln_norm_proj_fold(x, e4m3_decode(codes) * _f64(s)[None, :], mod, bias, idx, eps)


def adaln_norm_proj_swiglu_fp8(x, codes_gate, s_gate, codes_up, s_up, mod, bias_gate, bias_up, idx,
                               eps: float) -> np.ndarray:
    """SwiGLU variant: a, b as in adaln_norm_proj_fp8, out = silu(a) * b."""
    a = adaln_norm_proj_fp8(x, codes_gate, s_gate, mod, bias_gate, idx, eps)
    b = adaln_norm_proj_fp8(x, codes_up, s_up, mod, bias_up, idx, eps)
    return silu(a) * b


def adaln_norm_proj_swiglu_q8(x, g, scale, shift, idx, W_gate, W_up, eps: float):
    """AdaLN FC1 with fp8 row-block output ([FlashInfer #5521] "Segmented
    Chain": norm + AdaLN, FC1, SwiGLU, quantisation for the next projection;
    the format as read for norm_proj_swiglu_q8): the row-block quantisation
    of the SwiGLU output of the definition.  Returns (codes, s, v)."""
    v = adaln_norm_proj_swiglu(x, g, scale, shift, idx, W_gate, W_up, eps)
    codes, s = quantize_e4m3_row_blocks(v)
    return codes, s, v


def adaln_norm_proj_swiglu_fp8_q8(x, codes_gate, s_gate, codes_up, s_up, mod, bias_gate, bias_up, idx,
                                  eps: float):
    """The same with E4M3 weights: the row-block quantisation of
    adaln_norm_proj_swiglu_fp8.  Returns (codes, s, v)."""
    v = adaln_norm_proj_swiglu_fp8(x, codes_gate, s_gate, codes_up, s_up, mod, bias_gate, bias_up, idx, eps)
    codes, s = quantize_e4m3_row_blocks(v)
    return codes, s, v


def adaln_operand(x, mod, idx) -> np.ndarray:
    """The modulated matrix-core operand of the AdaLN path: x * mod[idx[m]]
    (float64-exact for bf16 x and a float32 table) rounded to float32, then
    to bf16 with ties to even ([FlashInfer #4040]: the fp32 -> bf16 step
    rounds to nearest even); a row whose index is outside [0, T) is 0.  This
    is the specification of the library's modulation pre-pass, which
    exports the operand, so it fixes bits; the projection oracles above do
    not use it."""
    return round_to_bf16(round_to_f32(_f64(x) * _rows_or_zero(mod, idx)))


__all__ = ["rms", "rmsnorm", "norm_proj", "silu", "norm_proj_swiglu", "fold_exact",
           "round_to_bf16", "round_to_f32", "round_to", "fold_weights", "norm_proj_folded",
           "norm_proj_swiglu_folded", "eps_as_received", "E4M3_MAX", "e4m3_decode", "e4m3_encode",
           "quantize_e4m3_columns", "fold_weights_fp8", "norm_proj_fp8", "norm_proj_swiglu_fp8",
           "Q8_BLOCK", "quantize_e4m3_row_blocks", "dequantize_row_blocks", "norm_proj_swiglu_q8",
           "norm_proj_swiglu_fp8_q8", "adaln_modulate", "adaln_norm_proj", "adaln_norm_proj_swiglu",
           "adaln_fold_table", "adaln_shift_bias", "adaln_norm_proj_fold", "adaln_norm_proj_swiglu_fold",
           "adaln_operand", "adaln_norm_proj_fp8", "adaln_norm_proj_swiglu_fp8", "adaln_norm_proj_swiglu_q8",
           "adaln_norm_proj_swiglu_fp8_q8"]
