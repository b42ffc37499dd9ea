"""GPU parity at the size limits the C ABI accepts, with the other
dimensions kept small: K at its maximum (2^20, the longest k loops and the
largest in-buffer offsets of every kernel family), very wide N (4097
column blocks) and many rows (65539: thousands of row tiles and pre-pass
workgroups), each against the float64 oracle."""
import numpy as np
import pytest

import oracle
import workloads as W
from tests.gpu_helpers import assert_close, to_dev, to_f64

pytestmark = pytest.mark.gpu

K_MAX = 1 << 20


def _plain(fn, M, K, N, dtype, swiglu, seed):
    inp = W.random_inputs(M, K, N, dtype, seed=seed, swiglu=swiglu)
    x, g = to_dev(inp.x, dtype), to_dev(inp.g, dtype)
    Pg = fn.fold_weights(g, to_dev(inp.W, dtype))
    if swiglu:
        Pu = fn.fold_weights(g, to_dev(inp.W_up, dtype))
        y = fn.norm_proj_swiglu(x, Pg, Pu, inp.call.eps)
        ref = oracle.norm_proj_swiglu(inp.x, inp.g, inp.W, inp.W_up, inp.call.eps)
    else:
        y = fn.norm_proj(x, Pg, inp.call.eps)
        ref = oracle.norm_proj(inp.x, inp.g, inp.W, inp.call.eps)
    return to_f64(y), ref


def _fp8(fn, M, K, N, swiglu, seed):
    inp = W.random_inputs(M, K, N, "bf16", seed=seed, swiglu=swiglu)
    x, g = to_dev(inp.x, "bf16"), to_dev(inp.g, "bf16")
    Pg = fn.fold_weights_fp8(g, to_dev(inp.W, "bf16"))
    cg, sg = oracle.fold_weights_fp8(inp.g, inp.W, "bf16")
    if swiglu:
        Pu = fn.fold_weights_fp8(g, to_dev(inp.W_up, "bf16"))
        cu, su = oracle.fold_weights_fp8(inp.g, inp.W_up, "bf16")
        y = fn.norm_proj_swiglu_fp8(x, Pg, Pu, inp.call.eps)
        ref = oracle.norm_proj_swiglu_fp8(inp.x, cg, sg, cu, su, inp.call.eps)
    else:
        y = fn.norm_proj_fp8(x, Pg, inp.call.eps)
        ref = oracle.norm_proj_fp8(inp.x, cg, sg, inp.call.eps)
    return to_f64(y), ref


@pytest.mark.parametrize("M,swiglu,dtype", [(1, False, "bf16"), (16, True, "bf16"), (33, False, "bf16"),
                                            (64, True, "bf16"), (65, False, "bf16"), (4, False, "f32"),
                                            (16, True, "f32"), (70, False, "f32")])
def test_max_k(gpu_lib, M, swiglu, dtype):
    """The tolerance rule of the dtype (fp32: 1e-5 (|ref| + 1)) at the
    largest K the library accepts."""
    y, ref = _plain(gpu_lib, M, K_MAX, 24, dtype, swiglu, seed=M + 1)
    err = assert_close(y, ref, dtype, f"K=2^20 M={M} {dtype} swiglu={swiglu}")
    print(f"K=2^20 M={M} {dtype} swiglu={swiglu}: max |err|/(|ref|+1) = {err:.2e}")


@pytest.mark.parametrize("M,swiglu", [(16, False), (64, True), (65, False), (130, True)])
def test_max_k_fp8(gpu_lib, M, swiglu):
    y, ref = _fp8(gpu_lib, M, K_MAX, 24, swiglu, seed=M + 2)
    assert_close(y, ref, "bf16", f"fp8 K=2^20 M={M} swiglu={swiglu}")


@pytest.mark.parametrize("M,swiglu", [(16, False), (64, True), (300, False)])
def test_wide_n(gpu_lib, M, swiglu):
    y, ref = _plain(gpu_lib, M, 72, 65552, "bf16", swiglu, seed=M + 3)
    assert_close(y, ref, "bf16", f"N=65552 M={M} swiglu={swiglu}")


@pytest.mark.parametrize("kind", ["bf16", "bf16_swiglu", "fp8"])
def test_many_rows(gpu_lib, kind):
    M = 65539
    if kind == "fp8":
        y, ref = _fp8(gpu_lib, M, 64, 48, False, seed=5)
    else:
        y, ref = _plain(gpu_lib, M, 64, 48, "bf16", kind.endswith("swiglu"), seed=6)
    assert_close(y, ref, "bf16", f"M={M} {kind}")


@pytest.mark.parametrize("M,K,N,T,swiglu", [(65, K_MAX, 24, 3, False), (40, K_MAX, 24, 2, True),
                                            (65539, 64, 48, 5, True)])
def test_adaln_two_launch_limits(gpu_lib, M, K, N, T, swiglu):
    """The AdaLN pre-pass and the projection on the modulated operand (split
    for SwiGLU) at the longest rows (K = 2^20: 2048 chunks per lane) and the
    most rows."""
    from tests.gpu_helpers import AdalnCase, assert_adaln_close
    c = AdalnCase(gpu_lib, M, K, N, T, swiglu, seed=M + K + T)
    f = gpu_lib.norm_proj_swiglu_adaln_ws if swiglu else gpu_lib.norm_proj_adaln_ws
    y = to_f64(f(c.x, *c.args(), c.eps))
    assert_adaln_close(y, c.reference(), c.value_error_bound(), f"adaln two-launch M={M} K={K}")
