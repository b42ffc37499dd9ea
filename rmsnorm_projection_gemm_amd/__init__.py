"""Python binding of libflashnorm: fused RMSNorm + projection on MI355X.

Argument marshalling only.  Every step of the computation runs in the HIP
kernels of libflashnorm.so; PyTorch provides device memory and the current
stream.  There is no CPU fallback: if the library is not built, every call
raises.

    import rmsnorm_projection_gemm_amd as fn
    Wp = fn.fold_weights(g, W)           # offline: W' = diag(g) W, packed
    y = fn.norm_proj(x, Wp, eps=1e-6)    # y = (x W') / rms(x), one launch
    out = fn.norm_proj_swiglu(x, Wg, Wu) # silu(a) * b, one launch
    P8 = fn.fold_weights_fp8(g, W)       # W' quantised to E4M3 per column
    y8 = fn.norm_proj_fp8(x, P8)         # y = s * (x q) / rms(x), one launch
    st = fn.Step(); st.norm_proj(x, Wp, y); st.record()
    st.launch()                          # every recorded call, one graph launch
"""
from __future__ import annotations

import ctypes
import dataclasses
import os
import re
from typing import Optional

PKG_DIR = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(PKG_DIR, "libflashnorm.so")
HEADER_PATH = os.path.join(os.path.dirname(PKG_DIR), "include", "flashnorm.h")

FN_F32 = 0
FN_BF16 = 1

STATUS = {0: "FN_OK", 1: "FN_ERR_NULL", 2: "FN_ERR_SHAPE", 3: "FN_ERR_ALIGN", 4: "FN_ERR_DTYPE",
          5: "FN_ERR_EPS", 6: "FN_ERR_ALIAS", 7: "FN_ERR_HIP", 8: "FN_ERR_WORKSPACE"}

_lib = None


class FlashNormError(RuntimeError):
    def __init__(self, status: int, detail: str):
        self.status = status
        super().__init__(f"{STATUS.get(status, status)}: {detail}")


def header_functions():
    """Names of the functions include/flashnorm.h declares."""
    with open(HEADER_PATH) as f:
        text = f.read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(fn_[a-z0-9_]+)\s*\(", text)))


def load():
    """Load libflashnorm.so (raises if it is missing: there is no fallback)."""
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(LIB_PATH):
        raise RuntimeError(f"{LIB_PATH} is not built; run `python -m rmsnorm_projection_gemm_amd.build`")
    lib = ctypes.CDLL(LIB_PATH)
    vp, i64, f32, i32 = ctypes.c_void_p, ctypes.c_int64, ctypes.c_float, ctypes.c_int
    sigs = {
        "fn_packed_weight_bytes": (ctypes.c_size_t, [i64, i64, i32]),
        "fn_fold_weights": (i32, [vp, vp, vp, i64, i64, i32, vp]),
        "fn_norm_proj": (i32, [vp, vp, vp, i64, i64, i64, f32, i32, vp]),
        "fn_norm_proj_swiglu": (i32, [vp, vp, vp, vp, i64, i64, i64, f32, i32, vp]),
        "fn_rmsnorm": (i32, [vp, vp, vp, i64, i64, f32, i32, vp]),
        "fn_probe_hbm_read": (i32, [vp, i64, vp, i64, vp]),
        "fn_probe_mfma_bf16": (i32, [vp, i64, i64, vp]),
        "fn_silu_mul": (i32, [vp, vp, i64, i64, i32, vp]),
        "fn_kernel_name": (ctypes.c_char_p, [i64, i64, i64, i32, i32]),
        "fn_packed_fp8_bytes": (ctypes.c_size_t, [i64, i64]),
        "fn_fold_weights_fp8": (i32, [vp, vp, vp, vp, i64, i64, i32, vp]),
        "fn_norm_proj_fp8": (i32, [vp, vp, vp, vp, i64, i64, i64, f32, vp]),
        "fn_norm_proj_swiglu_fp8": (i32, [vp, vp, vp, vp, vp, vp, i64, i64, i64, f32, vp]),
        "fn_kernel_name_fp8": (ctypes.c_char_p, [i64, i64, i64, i32]),
        "fn_norm_proj_swiglu_q8": (i32, [vp, vp, vp, vp, vp, i64, i64, i64, f32, vp]),
        "fn_norm_proj_swiglu_fp8_q8": (i32, [vp, vp, vp, vp, vp, vp, vp, i64, i64, i64, f32, vp]),
        "fn_kernel_name_q8": (ctypes.c_char_p, [i64, i64, i64, i32]),
        "fn_adaln_shift_bias": (i32, [vp, vp, vp, i64, i64, i64, i32, vp]),
        "fn_adaln_fold_table": (i32, [vp, vp, vp, i64, i64, i32, vp]),
        "fn_norm_proj_swiglu_adaln_static": (i32, [vp, vp, vp, vp, vp, vp, vp, vp, i64, i64, i64, i64, f32, vp]),
        "fn_norm_proj_swiglu_adaln_static_max_bytes": (i64, []),
        "fn_norm_proj_adaln": (i32, [vp, vp, vp, vp, vp, vp, i64, i64, i64, i64, f32, vp]),
        "fn_norm_proj_swiglu_adaln": (i32, [vp, vp, vp, vp, vp, vp, vp, vp, i64, i64, i64, i64, f32, vp]),
        "fn_kernel_name_adaln": (ctypes.c_char_p, [i64, i64, i64, i64, i32]),
        "fn_norm_proj_adaln_ws": (i32, [vp, vp, vp, vp, vp, vp, i64, i64, i64, i64, f32, vp, i64, vp]),
        "fn_norm_proj_swiglu_adaln_ws": (i32, [vp, vp, vp, vp, vp, vp, vp, vp, i64, i64, i64, i64, f32, vp, i64,
                                               vp]),
        "fn_adaln_workspace_bytes": (i64, [i64, i64]),
        "fn_kernel_name_adaln_ws": (ctypes.c_char_p, [i64, i64, i64, i64, i32]),
        "fn_adaln_modulate": (i32, [vp, vp, vp, vp, vp, i64, i64, i64, f32, vp]),
        "fn_norm_proj_adaln_fp8_ws": (i32, [vp, vp, vp, vp, vp, vp, vp, i64, i64, i64, i64, f32, vp, i64, vp]),
        "fn_norm_proj_swiglu_adaln_fp8_ws": (i32, [vp, vp, vp, vp, vp, vp, vp, vp, vp, vp, i64, i64, i64, i64, f32,
                                                   vp, i64, vp]),
        "fn_adaln_prepass_bytes": (i64, [i64, i64]),
        "fn_kernel_name_adaln_fp8": (ctypes.c_char_p, [i64, i64, i64, i64, i32]),
        "fn_norm_proj_swiglu_adaln_q8_ws": (i32, [vp, vp, vp, vp, vp, vp, vp, vp, vp, i64, i64, i64, i64, f32, vp,
                                                  i64, vp]),
        "fn_norm_proj_swiglu_adaln_fp8_q8_ws": (i32, [vp, vp, vp, vp, vp, vp, vp, vp, vp, vp, vp, i64, i64, i64, i64,
                                                      f32, vp, i64, vp]),
        "fn_kernel_name_adaln_q8": (ctypes.c_char_p, [i64, i64, i64, i64, i32]),
        "fn_step_create": (i32, [vp, i64, ctypes.POINTER(vp)]),
        "fn_step_create_grouped": (i32, [vp, i64, ctypes.POINTER(vp)]),
        "fn_step_launch": (i32, [vp, vp]),
        "fn_step_num_kernels": (i64, [vp]),
        "fn_step_destroy": (i32, [vp]),
        "fn_status_string": (ctypes.c_char_p, [i32]),
        "fn_last_error": (ctypes.c_char_p, []),
    }
    for name, (res, args) in sigs.items():
        f = getattr(lib, name)
        f.restype = res
        f.argtypes = args
    _lib = lib
    return lib


def _check(status: int):
    if status != 0:
        raise FlashNormError(status, load().fn_last_error().decode())


def _torch():
    import torch
    return torch


_DTYPES = {}


def _dt(dtype) -> int:
    if not _DTYPES:
        torch = _torch()
        _DTYPES.update({torch.bfloat16: FN_BF16, torch.float32: FN_F32})
    code = _DTYPES.get(dtype)
    if code is None:
        raise ValueError(f"dtype must be torch.bfloat16 or torch.float32, got {dtype}")
    return code


_raw_stream = None


def _stream(t) -> int:
    """The current HIP stream of t's device, as an integer handle: torch's raw
    getter when it has one (a tenth of the cost of building a Stream object
    per call, which dominates a launch-bound call), else the public API."""
    global _raw_stream
    if _raw_stream is None:
        torch = _torch()
        getter = getattr(torch._C, "_cuda_getCurrentRawStream", None)
        _raw_stream = ((lambda d: getter(d.index)) if getter is not None
                       else (lambda d: torch.cuda.current_stream(d).cuda_stream))
    return _raw_stream(t.device)


def _need_cuda(name, t):
    if not t.is_cuda:
        raise ValueError(f"{name} must be a CUDA (HIP) tensor, got device {t.device}")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")


@dataclasses.dataclass
class PackedWeights:
    """Folded weights W' = diag(g) W in libflashnorm's packed layout."""
    data: "object"      # torch.uint8 tensor on the device, packed bytes
    K: int
    N: int
    dtype: "object"     # torch.bfloat16 or torch.float32


def packed_weight_bytes(K: int, N: int, dtype) -> int:
    n = load().fn_packed_weight_bytes(K, N, _dt(dtype))
    if n == 0 and N > 0:
        raise ValueError(f"K={K} must be in [1, 2^20] and a multiple of 8; N={N} in [0, 2^24]")
    return n


def fold_weights(g, W, out: Optional[PackedWeights] = None) -> PackedWeights:
    """W'[k, n] = round(g[k] * W[k, n]) in the packed layout (g=None packs W)."""
    torch = _torch()
    _need_cuda("W", W)
    if W.dim() != 2:
        raise ValueError(f"W must be [K, N], got shape {tuple(W.shape)}")
    K, N = W.shape
    dt = _dt(W.dtype)
    if g is not None:
        _need_cuda("g", g)
        if g.dtype != W.dtype or tuple(g.shape) != (K,):
            raise ValueError(f"g must be [{K}] of dtype {W.dtype}, got {tuple(g.shape)} {g.dtype}")
    nbytes = packed_weight_bytes(K, N, W.dtype)
    if out is None:
        out = PackedWeights(torch.empty(nbytes, dtype=torch.uint8, device=W.device), K, N, W.dtype)
    elif (out.K, out.N, out.dtype) != (K, N, W.dtype) or out.data.numel() != nbytes:
        raise ValueError("out does not match W's shape and dtype")
    _check(load().fn_fold_weights(None if g is None else g.data_ptr(), W.data_ptr(), out.data.data_ptr(),
                                  K, N, dt, _stream(W)))
    return out


def _check_x(x, Wp: PackedWeights):
    _need_cuda("x", x)
    if x.dim() != 2 or x.shape[1] != Wp.K:
        raise ValueError(f"x must be [M, {Wp.K}], got {tuple(x.shape)}")
    if x.dtype != Wp.dtype:
        raise ValueError(f"x dtype {x.dtype} must match the folded weights' {Wp.dtype}")
    if x.device != Wp.data.device:
        raise ValueError("x and the folded weights must be on the same device")


def _out(out, M, N, x):
    torch = _torch()
    if out is None:
        return torch.empty((M, N), dtype=x.dtype, device=x.device)
    _need_cuda("out", out)
    if tuple(out.shape) != (M, N) or out.dtype != x.dtype:
        raise ValueError(f"out must be [{M}, {N}] of dtype {x.dtype}")
    return out


def norm_proj(x, Wp: PackedWeights, eps: float = 1e-6, out=None):
    """y = (x @ W') / sqrt(mean(x^2) + eps), one fused launch."""
    _check_x(x, Wp)
    M, N = x.shape[0], Wp.N
    y = _out(out, M, N, x)
    _check(load().fn_norm_proj(x.data_ptr(), Wp.data.data_ptr(), y.data_ptr(), M, Wp.K, N, eps,
                               _dt(x.dtype), _stream(x)))
    return y


def norm_proj_swiglu(x, Wg: PackedWeights, Wu: PackedWeights, eps: float = 1e-6, out=None):
    """out = silu(a) * b with a, b the normalised gate/up projections, one launch."""
    _check_x(x, Wg)
    if (Wu.K, Wu.N, Wu.dtype) != (Wg.K, Wg.N, Wg.dtype):
        raise ValueError("gate and up weights must have the same K, N and dtype")
    M, N = x.shape[0], Wg.N
    y = _out(out, M, N, x)
    _check(load().fn_norm_proj_swiglu(x.data_ptr(), Wg.data.data_ptr(), Wu.data.data_ptr(), y.data_ptr(),
                                      M, Wg.K, N, eps, _dt(x.dtype), _stream(x)))
    return y


def rmsnorm(x, g, eps: float = 1e-6, out=None):
    """Unfused chain step: xhat = x / rms(x) * g written to memory."""
    _need_cuda("x", x)
    _need_cuda("g", g)
    M, K = x.shape
    y = _out(out, M, K, x)
    _check(load().fn_rmsnorm(x.data_ptr(), g.data_ptr(), y.data_ptr(), M, K, eps, _dt(x.dtype), _stream(x)))
    return y


PROBE_MFMA_FLOPS_PER_WG_ITER = 524288   # 4 waves x 8 MFMAs x 16*16*32*2


def probe_hbm_read(src, workgroups: int = 2048):
    """Measurement probe: stream all of `src` (a contiguous device tensor whose
    size is a multiple of 16 bytes) once; returns the sink tensor."""
    _need_cuda("src", src)
    if not src.is_contiguous():
        raise ValueError("src must be contiguous")
    import torch
    sink = torch.empty((workgroups,), dtype=torch.int32, device=src.device)
    nbytes = src.numel() * src.element_size()
    _check(load().fn_probe_hbm_read(src.data_ptr(), nbytes, sink.data_ptr(), workgroups, _stream(src)))
    return sink


def probe_mfma_bf16(iters: int, workgroups: int = 2048, device="cuda"):
    """Measurement probe: an MFMA-only loop of workgroups * iters * 524288
    bf16 FLOPs on the current stream; returns the sink tensor."""
    import torch
    sink = torch.empty((workgroups,), dtype=torch.float32, device=device)
    _check(load().fn_probe_mfma_bf16(sink.data_ptr(), iters, workgroups, _stream(sink)))
    return sink


def silu_mul(h, out=None):
    """Unfused chain step: out = silu(h[:, :N]) * h[:, N:] for h of shape [M, 2N]."""
    _need_cuda("h", h)
    M, N2 = h.shape
    if N2 % 2:
        raise ValueError("h must have an even number of columns")
    y = _out(out, M, N2 // 2, h)
    _check(load().fn_silu_mul(h.data_ptr(), y.data_ptr(), M, N2 // 2, _dt(h.dtype), _stream(h)))
    return y


def kernel_name(M: int, K: int, N: int, swiglu: bool, dtype) -> str:
    return load().fn_kernel_name(M, K, N, int(swiglu), _dt(dtype)).decode()


# ------------------------------------------------------------ fp8 weights --
@dataclasses.dataclass
class PackedFp8:
    """Folded weights quantised to E4M3 per output column: packed codes and
    the column scales s (y = s * (x @ q) / rms(x))."""
    data: "object"      # torch.uint8 tensor on the device, packed codes
    scales: "object"    # torch.float32 tensor [N] on the device
    K: int
    N: int


def packed_fp8_bytes(K: int, N: int) -> int:
    n = load().fn_packed_fp8_bytes(K, N)
    if n == 0 and N > 0:
        raise ValueError(f"K={K} must be in [1, 2^20] and a multiple of 8; N={N} in [0, 2^24]")
    return n


def fold_weights_fp8(g, W, out: Optional[PackedFp8] = None) -> PackedFp8:
    """Fold W' = round(g[k] * W[k, n]) in W's dtype, then quantise each column
    to E4M3 with scale s[n] = max|W'[:, n]| / 448 (g=None quantises W)."""
    torch = _torch()
    _need_cuda("W", W)
    if W.dim() != 2:
        raise ValueError(f"W must be [K, N], got shape {tuple(W.shape)}")
    K, N = W.shape
    dt = _dt(W.dtype)
    if g is not None:
        _need_cuda("g", g)
        if g.dtype != W.dtype or tuple(g.shape) != (K,):
            raise ValueError(f"g must be [{K}] of dtype {W.dtype}, got {tuple(g.shape)} {g.dtype}")
    nbytes = packed_fp8_bytes(K, N)
    if out is None:
        out = PackedFp8(torch.empty(nbytes, dtype=torch.uint8, device=W.device),
                        torch.empty(N, dtype=torch.float32, device=W.device), K, N)
    elif (out.K, out.N) != (K, N) or out.data.numel() != nbytes or out.scales.numel() != N:
        raise ValueError("out does not match W's shape")
    _check(load().fn_fold_weights_fp8(None if g is None else g.data_ptr(), W.data_ptr(), out.data.data_ptr(),
                                      out.scales.data_ptr(), K, N, dt, _stream(W)))
    return out


def _check_x_fp8(x, P: PackedFp8):
    torch = _torch()
    _need_cuda("x", x)
    if x.dim() != 2 or x.shape[1] != P.K:
        raise ValueError(f"x must be [M, {P.K}], got {tuple(x.shape)}")
    if x.dtype != torch.bfloat16:
        raise ValueError(f"fp8-weight calls take bf16 activations, got {x.dtype}")
    if x.device != P.data.device:
        raise ValueError("x and the fp8 weights must be on the same device")


def norm_proj_fp8(x, P: PackedFp8, eps: float = 1e-6, out=None):
    """y = s * (x @ q) / sqrt(mean(x^2) + eps) with E4M3 weights, one launch."""
    _check_x_fp8(x, P)
    M, N = x.shape[0], P.N
    y = _out(out, M, N, x)
    _check(load().fn_norm_proj_fp8(x.data_ptr(), P.data.data_ptr(), P.scales.data_ptr(), y.data_ptr(), M, P.K, N,
                                   eps, _stream(x)))
    return y


def norm_proj_swiglu_fp8(x, Pg: PackedFp8, Pu: PackedFp8, eps: float = 1e-6, out=None):
    """out = silu(a) * b with E4M3 gate/up weights, one launch."""
    _check_x_fp8(x, Pg)
    if (Pu.K, Pu.N) != (Pg.K, Pg.N):
        raise ValueError("gate and up weights must have the same K and N")
    M, N = x.shape[0], Pg.N
    y = _out(out, M, N, x)
    _check(load().fn_norm_proj_swiglu_fp8(x.data_ptr(), Pg.data.data_ptr(), Pg.scales.data_ptr(), Pu.data.data_ptr(),
                                          Pu.scales.data_ptr(), y.data_ptr(), M, Pg.K, N, eps, _stream(x)))
    return y


def kernel_name_fp8(M: int, K: int, N: int, swiglu: bool) -> str:
    return load().fn_kernel_name_fp8(M, K, N, int(swiglu)).decode()


# ------------------------------------------- SwiGLU with fp8 output (q8) --
Q8_BLOCK = 16


def _q8_out(out, M, N, x):
    """(codes uint8 [M, N], scales float32 [M, ceil(N/16)]) on x's device."""
    torch = _torch()
    nb = -(-N // Q8_BLOCK)
    if out is None:
        return (torch.empty((M, N), dtype=torch.uint8, device=x.device),
                torch.empty((M, nb), dtype=torch.float32, device=x.device))
    codes, scales = out
    _need_cuda("codes", codes)
    _need_cuda("scales", scales)
    if tuple(codes.shape) != (M, N) or codes.dtype != torch.uint8:
        raise ValueError(f"codes must be [{M}, {N}] uint8")
    if tuple(scales.shape) != (M, nb) or scales.dtype != torch.float32:
        raise ValueError(f"scales must be [{M}, {nb}] float32")
    return codes, scales


def norm_proj_swiglu_q8(x, Wg: PackedWeights, Wu: PackedWeights, eps: float = 1e-6, out=None):
    """silu(a) * b quantised to E4M3 with one scale per 16-column row block:
    returns (codes, scales); the values are scales[m, n // 16] * decode(codes[m, n])."""
    torch = _torch()
    _check_x(x, Wg)
    if x.dtype != torch.bfloat16:
        raise ValueError("fp8 output takes bf16 activations and weights")
    if (Wu.K, Wu.N, Wu.dtype) != (Wg.K, Wg.N, Wg.dtype):
        raise ValueError("gate and up weights must have the same K, N and dtype")
    M, N = x.shape[0], Wg.N
    codes, scales = _q8_out(out, M, N, x)
    _check(load().fn_norm_proj_swiglu_q8(x.data_ptr(), Wg.data.data_ptr(), Wu.data.data_ptr(), codes.data_ptr(),
                                         scales.data_ptr(), M, Wg.K, N, eps, _stream(x)))
    return codes, scales


def norm_proj_swiglu_fp8_q8(x, Pg: PackedFp8, Pu: PackedFp8, eps: float = 1e-6, out=None):
    """E4M3 weights in, E4M3 row-block output out: (codes, scales)."""
    _check_x_fp8(x, Pg)
    if (Pu.K, Pu.N) != (Pg.K, Pg.N):
        raise ValueError("gate and up weights must have the same K and N")
    M, N = x.shape[0], Pg.N
    codes, scales = _q8_out(out, M, N, x)
    _check(load().fn_norm_proj_swiglu_fp8_q8(x.data_ptr(), Pg.data.data_ptr(), Pg.scales.data_ptr(),
                                             Pu.data.data_ptr(), Pu.scales.data_ptr(), codes.data_ptr(),
                                             scales.data_ptr(), M, Pg.K, N, eps, _stream(x)))
    return codes, scales


def kernel_name_q8(M: int, K: int, N: int, fp8_weights: bool) -> str:
    return load().fn_kernel_name_q8(M, K, N, int(fp8_weights)).decode()


# ------------------------------------------------------- AdaLN prologue --
def adaln_shift_bias(shift, W, out=None):
    """bias[t] = shift[t] @ W (unfolded W, fp32 sums): [T, N] float32."""
    torch = _torch()
    _need_cuda("shift", shift)
    _need_cuda("W", W)
    if shift.dim() != 2 or W.dim() != 2 or shift.shape[1] != W.shape[0] or shift.dtype != W.dtype:
        raise ValueError(f"shift must be [T, {W.shape[0]}] of W's dtype, got {tuple(shift.shape)} {shift.dtype}")
    T, K = shift.shape
    N = W.shape[1]
    bias = torch.empty((T, N), dtype=torch.float32, device=W.device) if out is None else out
    _check(load().fn_adaln_shift_bias(shift.data_ptr(), W.data_ptr(), bias.data_ptr(), T, K, N, _dt(W.dtype),
                                      _stream(W)))
    return bias


def adaln_fold_table(g, scale, out=None):
    """mod[t] = g * (1 + scale[t]) in float32 (float64 arithmetic, one
    rounding): the gain folded into the AdaLN modulation table, [T, K]."""
    torch = _torch()
    _need_cuda("g", g)
    _need_cuda("scale", scale)
    if scale.dim() != 2 or g.dim() != 1 or scale.shape[1] != g.shape[0] or scale.dtype != g.dtype:
        raise ValueError(f"scale must be [T, {g.shape[0]}] of g's dtype, got {tuple(scale.shape)} {scale.dtype}")
    T, K = scale.shape
    mod = torch.empty((T, K), dtype=torch.float32, device=g.device) if out is None else out
    _check(load().fn_adaln_fold_table(g.data_ptr(), scale.data_ptr(), mod.data_ptr(), T, K, _dt(g.dtype), _stream(g)))
    return mod


def _check_mod(mod, K):
    torch = _torch()
    _need_cuda("mod", mod)
    if mod.dim() != 2 or mod.shape[1] != K or mod.dtype != torch.float32 or not mod.is_contiguous():
        raise ValueError(f"mod must be a contiguous [T, {K}] float32 tensor (adaln_fold_table)")


def _check_adaln(x, mod, idx, Wp: PackedWeights, bias):
    torch = _torch()
    _check_x(x, Wp)
    if x.dtype != torch.bfloat16:
        raise ValueError("AdaLN calls take bf16 activations and weights")
    for name, t in (("idx", idx), ("bias", bias)):
        _need_cuda(name, t)
    _check_mod(mod, Wp.K)
    if idx.dtype != torch.int32 or tuple(idx.shape) != (x.shape[0],):
        raise ValueError(f"idx must be [{x.shape[0]}] int32")
    if tuple(bias.shape) != (mod.shape[0], Wp.N) or bias.dtype != torch.float32:
        raise ValueError(f"bias must be [{mod.shape[0]}, {Wp.N}] float32")


def norm_proj_adaln(x, mod, idx, Wp: PackedWeights, bias, eps: float = 1e-6, out=None):
    """y = (RMSNorm_g(x) * (1 + scale[idx]) + shift[idx]) @ W, one launch, up
    to 16 rows (mod = adaln_fold_table(g, scale), Wp = fold_weights(None, W),
    bias = adaln_shift_bias(shift, W))."""
    _check_adaln(x, mod, idx, Wp, bias)
    M, N = x.shape[0], Wp.N
    y = _out(out, M, N, x)
    _check(load().fn_norm_proj_adaln(x.data_ptr(), mod.data_ptr(), idx.data_ptr(), Wp.data.data_ptr(),
                                     bias.data_ptr(), y.data_ptr(), M, Wp.K, N, mod.shape[0], eps, _stream(x)))
    return y


def norm_proj_swiglu_adaln(x, mod, idx, Wg: PackedWeights, bias_g, Wu: PackedWeights, bias_u, eps: float = 1e-6,
                           out=None):
    """out = silu(h @ W_gate) * (h @ W_up) with h the AdaLN-modulated norm, one
    launch, up to 16 rows."""
    _check_adaln(x, mod, idx, Wg, bias_g)
    _check_adaln(x, mod, idx, Wu, bias_u)
    M, N = x.shape[0], Wg.N
    y = _out(out, M, N, x)
    _check(load().fn_norm_proj_swiglu_adaln(x.data_ptr(), mod.data_ptr(), idx.data_ptr(), Wg.data.data_ptr(),
                                            bias_g.data_ptr(), Wu.data.data_ptr(), bias_u.data_ptr(), y.data_ptr(),
                                            M, Wg.K, N, mod.shape[0], eps, _stream(x)))
    return y


def kernel_name_adaln(M: int, K: int, N: int, T: int, swiglu: bool) -> str:
    return load().fn_kernel_name_adaln(M, K, N, T, int(swiglu)).decode()


def adaln_workspace_bytes(M: int, K: int) -> int:
    """Workspace bytes of the two-launch AdaLN calls (0: one launch)."""
    return int(load().fn_adaln_workspace_bytes(M, K))


def _workspace(workspace, M: int, K: int, like):
    """(pointer, bytes) of the caller's workspace, or of a new one from
    torch's caching allocator when none is given and the call needs it."""
    need = adaln_workspace_bytes(M, K)
    if workspace is None:
        if need == 0:
            return None, 0
        workspace = _torch().empty((need,), dtype=_torch().uint8, device=like.device)
    _need_cuda("workspace", workspace)
    return workspace, workspace.numel() * workspace.element_size()


def norm_proj_adaln_ws(x, mod, idx, Wp: PackedWeights, bias, eps: float = 1e-6, out=None, workspace=None):
    """norm_proj_adaln for any M: above 16 rows in two launches, the AdaLN
    pre-pass into a workspace (allocated here when not given), then the
    projection kernel of the row count on the modulated operand."""
    _check_adaln(x, mod, idx, Wp, bias)
    M, N = x.shape[0], Wp.N
    y = _out(out, M, N, x)
    ws, nbytes = _workspace(workspace, M, Wp.K, x)
    _check(load().fn_norm_proj_adaln_ws(x.data_ptr(), mod.data_ptr(), idx.data_ptr(), Wp.data.data_ptr(),
                                        bias.data_ptr(), y.data_ptr(), M, Wp.K, N, mod.shape[0], eps,
                                        None if ws is None else ws.data_ptr(), nbytes, _stream(x)))
    return y


def norm_proj_swiglu_adaln_ws(x, mod, idx, Wg: PackedWeights, bias_g, Wu: PackedWeights, bias_u,
                              eps: float = 1e-6, out=None, workspace=None):
    """norm_proj_swiglu_adaln for any M (see norm_proj_adaln_ws)."""
    _check_adaln(x, mod, idx, Wg, bias_g)
    _check_adaln(x, mod, idx, Wu, bias_u)
    M, N = x.shape[0], Wg.N
    y = _out(out, M, N, x)
    ws, nbytes = _workspace(workspace, M, Wg.K, x)
    _check(load().fn_norm_proj_swiglu_adaln_ws(x.data_ptr(), mod.data_ptr(), idx.data_ptr(), Wg.data.data_ptr(),
                                               bias_g.data_ptr(), Wu.data.data_ptr(), bias_u.data_ptr(),
                                               y.data_ptr(), M, Wg.K, N, mod.shape[0], eps,
                                               None if ws is None else ws.data_ptr(), nbytes, _stream(x)))
    return y


def norm_proj_swiglu_adaln_static(x, mod, idx, Wg: PackedWeights, bias_g, Wu: PackedWeights, bias_u,
                                  eps: float = 1e-6, out=None):
    """norm_proj_swiglu_adaln_ws with the library's own device scratch as the
    workspace (the entry point allocates nothing; pass `out` to allocate
    nothing here either).  Calls that overlap on one GPU race."""
    _check_adaln(x, mod, idx, Wg, bias_g)
    _check_adaln(x, mod, idx, Wu, bias_u)
    M, N = x.shape[0], Wg.N
    y = _out(out, M, N, x)
    _check(load().fn_norm_proj_swiglu_adaln_static(x.data_ptr(), mod.data_ptr(), idx.data_ptr(), Wg.data.data_ptr(),
                                                   bias_g.data_ptr(), Wu.data.data_ptr(), bias_u.data_ptr(),
                                                   y.data_ptr(), M, Wg.K, N, mod.shape[0], eps, _stream(x)))
    return y


def adaln_static_max_bytes() -> int:
    """Bytes of the device scratch norm_proj_swiglu_adaln_static uses."""
    return int(load().fn_norm_proj_swiglu_adaln_static_max_bytes())


def kernel_name_adaln_ws(M: int, K: int, N: int, T: int, swiglu: bool) -> str:
    return load().fn_kernel_name_adaln_ws(M, K, N, T, int(swiglu)).decode()


def adaln_prepass_bytes(M: int, K: int) -> int:
    """Workspace bytes of the fp8-weight AdaLN calls (needed for every M)."""
    return int(load().fn_adaln_prepass_bytes(M, K))


def _check_adaln_fp8(x, mod, idx, P: PackedFp8, bias):
    torch = _torch()
    _check_x_fp8(x, P)
    for name, t in (("idx", idx), ("bias", bias)):
        _need_cuda(name, t)
    _check_mod(mod, P.K)
    if idx.dtype != torch.int32 or tuple(idx.shape) != (x.shape[0],):
        raise ValueError(f"idx must be [{x.shape[0]}] int32")
    if tuple(bias.shape) != (mod.shape[0], P.N) or bias.dtype != torch.float32:
        raise ValueError(f"bias must be [{mod.shape[0]}, {P.N}] float32")


def _workspace_fp8(workspace, M: int, K: int, like):
    if workspace is None:
        n = adaln_prepass_bytes(M, K)
        if n == 0:
            return None, 0
        workspace = _torch().empty((n,), dtype=_torch().uint8, device=like.device)
    _need_cuda("workspace", workspace)
    return workspace, workspace.numel() * workspace.element_size()


def norm_proj_adaln_fp8_ws(x, mod, idx, P: PackedFp8, bias, eps: float = 1e-6, out=None, workspace=None):
    """AdaLN with E4M3 weights, two launches (the pre-pass into a workspace,
    allocated here when not given, then the fp8 kernel)."""
    _check_adaln_fp8(x, mod, idx, P, bias)
    M, N = x.shape[0], P.N
    y = _out(out, M, N, x)
    ws, nbytes = _workspace_fp8(workspace, M, P.K, x)
    _check(load().fn_norm_proj_adaln_fp8_ws(x.data_ptr(), mod.data_ptr(), idx.data_ptr(), P.data.data_ptr(),
                                            P.scales.data_ptr(), bias.data_ptr(), y.data_ptr(), M, P.K, N,
                                            mod.shape[0], eps, None if ws is None else ws.data_ptr(), nbytes,
                                            _stream(x)))
    return y


def norm_proj_swiglu_adaln_fp8_ws(x, mod, idx, Pg: PackedFp8, bias_g, Pu: PackedFp8, bias_u, eps: float = 1e-6,
                                  out=None, workspace=None):
    """SwiGLU AdaLN with E4M3 gate/up weights, two launches."""
    _check_adaln_fp8(x, mod, idx, Pg, bias_g)
    _check_adaln_fp8(x, mod, idx, Pu, bias_u)
    M, N = x.shape[0], Pg.N
    y = _out(out, M, N, x)
    ws, nbytes = _workspace_fp8(workspace, M, Pg.K, x)
    _check(load().fn_norm_proj_swiglu_adaln_fp8_ws(x.data_ptr(), mod.data_ptr(), idx.data_ptr(), Pg.data.data_ptr(),
                                                   Pg.scales.data_ptr(), bias_g.data_ptr(), Pu.data.data_ptr(),
                                                   Pu.scales.data_ptr(), bias_u.data_ptr(), y.data_ptr(), M, Pg.K, N,
                                                   mod.shape[0], eps, None if ws is None else ws.data_ptr(),
                                                   nbytes, _stream(x)))
    return y


def kernel_name_adaln_fp8(M: int, K: int, N: int, T: int, swiglu: bool) -> str:
    return load().fn_kernel_name_adaln_fp8(M, K, N, T, int(swiglu)).decode()


def norm_proj_swiglu_adaln_q8_ws(x, mod, idx, Wg: PackedWeights, bias_g, Wu: PackedWeights, bias_u,
                                 eps: float = 1e-6, out=None, workspace=None):
    """AdaLN FC1 + SwiGLU with E4M3 row-block output, two launches:
    (codes, scales)."""
    _check_adaln(x, mod, idx, Wg, bias_g)
    _check_adaln(x, mod, idx, Wu, bias_u)
    M, N = x.shape[0], Wg.N
    codes, scales = _q8_out(out, M, N, x)
    ws, nbytes = _workspace_fp8(workspace, M, Wg.K, x)
    _check(load().fn_norm_proj_swiglu_adaln_q8_ws(x.data_ptr(), mod.data_ptr(), idx.data_ptr(), Wg.data.data_ptr(),
                                                  bias_g.data_ptr(), Wu.data.data_ptr(), bias_u.data_ptr(),
                                                  codes.data_ptr(), scales.data_ptr(), M, Wg.K, N, mod.shape[0], eps,
                                                  None if ws is None else ws.data_ptr(), nbytes, _stream(x)))
    return codes, scales


def norm_proj_swiglu_adaln_fp8_q8_ws(x, mod, idx, Pg: PackedFp8, bias_g, Pu: PackedFp8, bias_u,
                                     eps: float = 1e-6, out=None, workspace=None):
    """The same with E4M3 gate/up weights: (codes, scales)."""
    _check_adaln_fp8(x, mod, idx, Pg, bias_g)
    _check_adaln_fp8(x, mod, idx, Pu, bias_u)
    M, N = x.shape[0], Pg.N
    codes, scales = _q8_out(out, M, N, x)
    ws, nbytes = _workspace_fp8(workspace, M, Pg.K, x)
    _check(load().fn_norm_proj_swiglu_adaln_fp8_q8_ws(x.data_ptr(), mod.data_ptr(), idx.data_ptr(),
                                                      Pg.data.data_ptr(), Pg.scales.data_ptr(), bias_g.data_ptr(),
                                                      Pu.data.data_ptr(), Pu.scales.data_ptr(), bias_u.data_ptr(),
                                                      codes.data_ptr(), scales.data_ptr(), M, Pg.K, N, mod.shape[0],
                                                      eps, None if ws is None else ws.data_ptr(), nbytes, _stream(x)))
    return codes, scales


def kernel_name_adaln_q8(M: int, K: int, N: int, T: int, fp8_weights: bool) -> str:
    return load().fn_kernel_name_adaln_q8(M, K, N, T, int(fp8_weights)).decode()


def adaln_modulate(x, mod, idx, eps: float = 1e-6, u=None, rs=None):
    """The AdaLN pre-pass alone: (u, rs) with u = bf16(fp32(x * mod[idx]))
    [M, K] and rs = 1/RMS(x) [M] float32."""
    torch = _torch()
    for name, t in (("x", x), ("idx", idx)):
        _need_cuda(name, t)
    if x.dim() != 2 or x.dtype != torch.bfloat16 or not x.is_contiguous():
        raise ValueError("x must be a contiguous [M, K] bf16 tensor")
    M, K = x.shape
    _check_mod(mod, K)
    if idx.dtype != torch.int32 or tuple(idx.shape) != (M,):
        raise ValueError(f"idx must be [{M}] int32")
    u = torch.empty((M, K), dtype=torch.bfloat16, device=x.device) if u is None else u
    rs = torch.empty((M,), dtype=torch.float32, device=x.device) if rs is None else rs
    _check(load().fn_adaln_modulate(x.data_ptr(), mod.data_ptr(), idx.data_ptr(), u.data_ptr(), rs.data_ptr(), M, K,
                                    mod.shape[0], eps, _stream(x)))
    return u, rs


# ------------------------------------------------------- recorded steps --
FN_CALL_NORM_PROJ, FN_CALL_NORM_PROJ_SWIGLU, FN_CALL_NORM_PROJ_FP8, FN_CALL_NORM_PROJ_SWIGLU_FP8 = 0, 1, 2, 3
FN_CALL_NORM_PROJ_SWIGLU_Q8, FN_CALL_NORM_PROJ_SWIGLU_FP8_Q8 = 4, 5


class FnCall(ctypes.Structure):
    """struct fn_call of include/flashnorm.h."""
    _fields_ = [("kind", ctypes.c_int), ("x", ctypes.c_void_p), ("w_gate", ctypes.c_void_p),
                ("w_up", ctypes.c_void_p), ("s_gate", ctypes.c_void_p), ("s_up", ctypes.c_void_p),
                ("y", ctypes.c_void_p), ("M", ctypes.c_int64), ("K", ctypes.c_int64), ("N", ctypes.c_int64),
                ("eps", ctypes.c_float), ("dt", ctypes.c_int), ("y_scales", ctypes.c_void_p)]


class Step:
    """A sequence of fused calls recorded once into a HIP graph and replayed
    with one launch (fn_step_create / fn_step_launch).  Every call names its
    output buffer; pointers are fixed at record() time, so refresh inputs in
    place between replays.  The tensors stay referenced by the Step."""

    def __init__(self):
        self._calls = []
        self._keep = []
        self._handle = None

    def _add(self, kind, x, wg, wu, sg, su, out, M, K, N, eps, dt, keep, out_scales=None):
        if self._handle is not None:
            raise RuntimeError("the step is already recorded")
        self._calls.append(FnCall(kind, x.data_ptr(), wg, wu, sg, su, out.data_ptr(), M, K, N, eps, dt,
                                  None if out_scales is None else out_scales.data_ptr()))
        self._keep.extend(keep)

    def norm_proj(self, x, Wp: PackedWeights, out, eps: float = 1e-6):
        _check_x(x, Wp)
        _out(out, x.shape[0], Wp.N, x)
        self._add(FN_CALL_NORM_PROJ, x, Wp.data.data_ptr(), None, None, None, out, x.shape[0], Wp.K, Wp.N, eps,
                  _dt(x.dtype), (x, Wp.data, out))

    def norm_proj_swiglu(self, x, Wg: PackedWeights, Wu: PackedWeights, out, eps: float = 1e-6):
        _check_x(x, Wg)
        if (Wu.K, Wu.N, Wu.dtype) != (Wg.K, Wg.N, Wg.dtype):
            raise ValueError("gate and up weights must have the same K, N and dtype")
        _out(out, x.shape[0], Wg.N, x)
        self._add(FN_CALL_NORM_PROJ_SWIGLU, x, Wg.data.data_ptr(), Wu.data.data_ptr(), None, None, out,
                  x.shape[0], Wg.K, Wg.N, eps, _dt(x.dtype), (x, Wg.data, Wu.data, out))

    def norm_proj_fp8(self, x, P: PackedFp8, out, eps: float = 1e-6):
        _check_x_fp8(x, P)
        _out(out, x.shape[0], P.N, x)
        self._add(FN_CALL_NORM_PROJ_FP8, x, P.data.data_ptr(), None, P.scales.data_ptr(), None, out,
                  x.shape[0], P.K, P.N, eps, FN_BF16, (x, P.data, P.scales, out))

    def norm_proj_swiglu_fp8(self, x, Pg: PackedFp8, Pu: PackedFp8, out, eps: float = 1e-6):
        _check_x_fp8(x, Pg)
        if (Pu.K, Pu.N) != (Pg.K, Pg.N):
            raise ValueError("gate and up weights must have the same K and N")
        _out(out, x.shape[0], Pg.N, x)
        self._add(FN_CALL_NORM_PROJ_SWIGLU_FP8, x, Pg.data.data_ptr(), Pu.data.data_ptr(), Pg.scales.data_ptr(),
                  Pu.scales.data_ptr(), out, x.shape[0], Pg.K, Pg.N, eps, FN_BF16,
                  (x, Pg.data, Pg.scales, Pu.data, Pu.scales, out))

    def norm_proj_swiglu_q8(self, x, Wg: PackedWeights, Wu: PackedWeights, codes, scales, eps: float = 1e-6):
        _check_x(x, Wg)
        if (Wu.K, Wu.N, Wu.dtype) != (Wg.K, Wg.N, Wg.dtype):
            raise ValueError("gate and up weights must have the same K, N and dtype")
        _q8_out((codes, scales), x.shape[0], Wg.N, x)
        self._add(FN_CALL_NORM_PROJ_SWIGLU_Q8, x, Wg.data.data_ptr(), Wu.data.data_ptr(), None, None, codes,
                  x.shape[0], Wg.K, Wg.N, eps, FN_BF16, (x, Wg.data, Wu.data, codes, scales), scales)

    def norm_proj_swiglu_fp8_q8(self, x, Pg: PackedFp8, Pu: PackedFp8, codes, scales, eps: float = 1e-6):
        _check_x_fp8(x, Pg)
        if (Pu.K, Pu.N) != (Pg.K, Pg.N):
            raise ValueError("gate and up weights must have the same K and N")
        _q8_out((codes, scales), x.shape[0], Pg.N, x)
        self._add(FN_CALL_NORM_PROJ_SWIGLU_FP8_Q8, x, Pg.data.data_ptr(), Pu.data.data_ptr(), Pg.scales.data_ptr(),
                  Pu.scales.data_ptr(), codes, x.shape[0], Pg.K, Pg.N, eps, FN_BF16,
                  (x, Pg.data, Pg.scales, Pu.data, Pu.scales, codes, scales), scales)

    def record(self, grouped: bool = False):
        """Validate and record the calls: into a HIP graph (fn_step_create),
        or, grouped=True, as one launch of independent calls
        (fn_step_create_grouped)."""
        if self._handle is not None:
            raise RuntimeError("the step is already recorded")
        arr = (FnCall * len(self._calls))(*self._calls)
        h = ctypes.c_void_p()
        create = load().fn_step_create_grouped if grouped else load().fn_step_create
        _check(create(arr, len(self._calls), ctypes.byref(h)))
        self._handle = h
        return self

    @property
    def num_kernels(self) -> int:
        return load().fn_step_num_kernels(self._handle)

    def launch(self, stream=None):
        """Replay every recorded call with one graph launch (one kernel
        launch for a grouped step) on `stream` (default: the current stream
        of the first call's device)."""
        if self._handle is None:
            raise RuntimeError("record() the step first")
        if stream is None:
            stream = _stream(self._keep[0])
        _check(load().fn_step_launch(self._handle, stream))

    def close(self):
        """Release the graph (or the grouped step's call table); the caller
        makes sure no replay is running."""
        if self._handle is not None:
            _check(load().fn_step_destroy(self._handle))
            self._handle = None


__all__ = ["load", "fold_weights", "norm_proj", "norm_proj_swiglu", "rmsnorm", "silu_mul",
           "packed_weight_bytes", "kernel_name", "PackedWeights", "FlashNormError", "header_functions",
           "LIB_PATH", "FN_F32", "FN_BF16", "PackedFp8", "packed_fp8_bytes", "fold_weights_fp8",
           "norm_proj_fp8", "norm_proj_swiglu_fp8", "kernel_name_fp8", "Step", "FnCall", "FN_CALL_NORM_PROJ",
           "FN_CALL_NORM_PROJ_SWIGLU", "FN_CALL_NORM_PROJ_FP8", "FN_CALL_NORM_PROJ_SWIGLU_FP8",
           "FN_CALL_NORM_PROJ_SWIGLU_Q8", "FN_CALL_NORM_PROJ_SWIGLU_FP8_Q8", "Q8_BLOCK", "norm_proj_swiglu_q8",
           "norm_proj_swiglu_fp8_q8", "kernel_name_q8", "adaln_shift_bias", "adaln_fold_table", "norm_proj_adaln",
           "norm_proj_swiglu_adaln", "kernel_name_adaln", "adaln_workspace_bytes", "norm_proj_adaln_ws",
           "norm_proj_swiglu_adaln_ws", "norm_proj_swiglu_adaln_static", "adaln_static_max_bytes", "kernel_name_adaln_ws", "adaln_modulate", "adaln_prepass_bytes",
           "norm_proj_adaln_fp8_ws", "norm_proj_swiglu_adaln_fp8_ws", "kernel_name_adaln_fp8",
           "norm_proj_swiglu_adaln_q8_ws", "norm_proj_swiglu_adaln_fp8_q8_ws", "kernel_name_adaln_q8"]
