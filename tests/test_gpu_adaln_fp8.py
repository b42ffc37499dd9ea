"""GPU parity of AdaLN with fp8 weights (E4M3 codes, one scale per output
column; two launches: the modulation pre-pass, then the fp8-weight decode
kernel on the modulated operand) against the float64 oracle, within a bound
derived from the arithmetic."""
import numpy as np
import pytest

import oracle
import workloads as W
from tests.gpu_helpers import assert_close, to_dev, to_f64

pytestmark = pytest.mark.gpu


def _idx_dev(idx):
    import torch
    return torch.from_numpy(np.ascontiguousarray(idx, dtype=np.int32)).cuda()


def _err(x, scale0, idx0, codes, s, shift0, Wm, eps):
    """Bound on |a_gpu - a_oracle| for one projection: the bf16 operand
    x + x*scale is within 2^-9 of its exact value and the decoded weights are
    exact, so the product is off by at most 2^-9 * sum_k |x(1+s)| |s q|
    (over r), plus fp32 accumulation (1e-5 of the same sum) and the fp32 bias
    rows against float64 (1e-5 of sum_k |shift| |W|)."""
    xm = np.abs(np.asarray(x, np.float64) * (1.0 + np.asarray(scale0, np.float64)[idx0]))
    r = oracle.rms(x, eps)[:, None]
    Wq = np.abs(oracle.e4m3_decode(codes) * np.asarray(s, np.float64)[None, :])
    prod = (xm @ Wq) / r
    return (2.0 ** -9 + 1e-5) * prod + 1e-5 * (np.abs(np.asarray(shift0, np.float64)) @ np.abs(Wm))[idx0] + 1e-6


def _run(fn, M, K, N, T, swiglu, seed, bad_idx=True):
    inp = W.random_inputs(M, K, N, "bf16", seed=seed, swiglu=swiglu)
    scale, shift, idx = W.adaln_tables(T, K, M, seed=seed + 1)
    if bad_idx and M >= 3:
        idx[0], idx[-1] = -1, T
    scale0 = np.vstack([scale, np.zeros((1, K), np.float32)])
    shift0 = np.vstack([shift, np.zeros((1, K), np.float32)])
    idx0 = np.where((idx < 0) | (idx >= T), T, idx)
    x, g = to_dev(inp.x, "bf16"), to_dev(inp.g, "bf16")
    sc, sh = to_dev(scale, "bf16"), to_dev(shift, "bf16")
    Wg = to_dev(inp.W, "bf16")
    Pg, bg = fn.fold_weights_fp8(g, Wg), fn.adaln_shift_bias(sh, Wg)
    cg, sg = oracle.fold_weights_fp8(inp.g, inp.W, "bf16")
    bias_g = oracle.adaln_shift_bias(shift0, inp.W)
    eps = inp.call.eps
    Ea = _err(inp.x, scale0, idx0, cg, sg, shift0, np.asarray(inp.W, np.float64), eps)
    if not swiglu:
        y = fn.norm_proj_adaln_fp8_ws(x, sc, _idx_dev(idx), Pg, bg, eps)
        ref = oracle.adaln_norm_proj_fp8(inp.x, cg, sg, scale0, bias_g, idx0, eps)
        return to_f64(y), ref, Ea + 2.0 ** -8 * np.abs(ref)
    Wu = to_dev(inp.W_up, "bf16")
    Pu, bu = fn.fold_weights_fp8(g, Wu), fn.adaln_shift_bias(sh, Wu)
    cu, su = oracle.fold_weights_fp8(inp.g, inp.W_up, "bf16")
    bias_u = oracle.adaln_shift_bias(shift0, inp.W_up)
    y = fn.norm_proj_swiglu_adaln_fp8_ws(x, sc, _idx_dev(idx), Pg, bg, Pu, bu, eps)
    ref = oracle.adaln_norm_proj_swiglu_fp8(inp.x, cg, sg, cu, su, scale0, bias_g, bias_u, idx0, eps)
    a = oracle.adaln_norm_proj_fp8(inp.x, cg, sg, scale0, bias_g, idx0, eps)
    b = oracle.adaln_norm_proj_fp8(inp.x, cu, su, scale0, bias_u, idx0, eps)
    Eb = _err(inp.x, scale0, idx0, cu, su, shift0, np.asarray(inp.W_up, np.float64), eps)
    sig = 1.0 / (1.0 + np.exp(-a))
    dsilu = sig * (1.0 + a * (1.0 - sig))
    bound = np.abs(dsilu) * np.abs(b) * Ea + np.abs(a * sig) * Eb + Ea * Eb + 2.0 ** -8 * np.abs(ref) + 1e-6
    return to_f64(y), ref, bound


def _check(y, ref, bound, what):
    assert y.shape == ref.shape and np.all(np.isfinite(y)), what
    bad = np.abs(y - ref) > bound
    assert not bad.any(), (f"{what}: {bad.sum()} outputs outside the derived bound, worst "
                           f"{np.max(np.abs(y - ref) / bound):.2f}x")
    assert_close(y, ref, "bf16", what)


@pytest.mark.parametrize("swiglu", [False, True])
@pytest.mark.parametrize("M,K,N,T", [(1, 8, 16, 1), (5, 264, 100, 3), (16, 1032, 270, 5), (17, 4104, 530, 100),
                                     (33, 264, 1100, 2), (64, 1032, 48, 7), (65, 520, 33, 3), (200, 264, 160, 30)])
def test_adaln_fp8_parity(gpu_lib, swiglu, M, K, N, T):
    y, ref, bound = _run(gpu_lib, M, K, N, T, swiglu, seed=M * 11 + K + N + T)
    _check(y, ref, bound, f"{'swiglu' if swiglu else 'proj'} adaln fp8 {M}x{K}x{N} T={T}")


@pytest.mark.parametrize("M,N,swiglu", [(16, 12288, False), (64, 11008, True)])
def test_adaln_fp8_decode_shapes(gpu_lib, M, N, swiglu):
    """The QKV and FFN decode shapes (K = 4096) with four table rows."""
    y, ref, bound = _run(gpu_lib, M, 4096, N, 4, swiglu, seed=M + N, bad_idx=False)
    _check(y, ref, bound, f"adaln fp8 decode {M}x4096x{N}")


def test_adaln_fp8_zero_tables_match_the_plain_fp8_path(gpu_lib):
    """Zero tables and zero bias rows: the operand is x itself, so the
    output equals the one-launch fp8 call's within the fp32 sum order (the
    two kernels take the sums of squares differently)."""
    import torch
    fn = gpu_lib
    M, K, N = 64, 1032, 530
    inp = W.random_inputs(M, K, N, "bf16", seed=4, swiglu=True)
    x, g = to_dev(inp.x, "bf16"), to_dev(inp.g, "bf16")
    Pg, Pu = fn.fold_weights_fp8(g, to_dev(inp.W, "bf16")), fn.fold_weights_fp8(g, to_dev(inp.W_up, "bf16"))
    sc = torch.zeros((3, K), dtype=torch.bfloat16, device="cuda")
    b = torch.zeros((3, N), dtype=torch.float32, device="cuda")
    idx = torch.zeros((M,), dtype=torch.int32, device="cuda")
    y = to_f64(fn.norm_proj_swiglu_adaln_fp8_ws(x, sc, idx, Pg, b, Pu, b, 1e-6))
    want = to_f64(fn.norm_proj_swiglu_fp8(x, Pg, Pu, 1e-6))
    assert np.all(np.abs(y - want) <= 2.0 ** -7 * np.abs(want) + 1e-6)
