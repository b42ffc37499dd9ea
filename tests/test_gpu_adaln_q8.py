"""GPU parity of AdaLN + SwiGLU with fp8 row-block output (E4M3 codes, one
scale per 16-column row block; two launches: the modulation pre-pass, then
the q8 kernel of the row count on the modulated operand) against the float64
oracle.  The codes are decisions, so the oracle forms the values it
quantises on the same bf16 operand the kernels use (adaln_operand, pinned
bit for bit) and the folded weights the GPU reads; codes must then match
except at rounding midpoints."""
import numpy as np
import pytest

import oracle
import workloads as W
from tests.gpu_helpers import assert_q8_close, to_dev

pytestmark = pytest.mark.gpu


def _idx_dev(idx):
    import torch
    return torch.from_numpy(np.ascontiguousarray(idx, dtype=np.int32)).cuda()


def _run(fn, M, K, N, T, weights, seed, bad_idx=True, rows=None):
    inp = W.random_inputs(M, K, N, "bf16", seed=seed, swiglu=True)
    scale, shift, idx = W.adaln_tables(T, K, M, seed=seed + 1)
    if bad_idx and M >= 3:
        idx[0], idx[-1] = -1, T
    x, g = to_dev(inp.x, "bf16"), to_dev(inp.g, "bf16")
    sc, sh = to_dev(scale, "bf16"), to_dev(shift, "bf16")
    Wg, Wu = to_dev(inp.W, "bf16"), to_dev(inp.W_up, "bf16")
    bg, bu = fn.adaln_shift_bias(sh, Wg), fn.adaln_shift_bias(sh, Wu)
    rbg, rbu = oracle.adaln_shift_bias(shift, inp.W), oracle.adaln_shift_bias(shift, inp.W_up)
    pick = slice(None) if rows is None else rows
    if weights == "bf16":
        Pg, Pu = fn.fold_weights(g, Wg), fn.fold_weights(g, Wu)
        codes, scales = fn.norm_proj_swiglu_adaln_q8_ws(x, sc, _idx_dev(idx), Pg, bg, Pu, bu, inp.call.eps)
        Wgf = oracle.fold_weights(inp.g, inp.W, "bf16")
        Wuf = oracle.fold_weights(inp.g, inp.W_up, "bf16")
        _, _, v = oracle.adaln_norm_proj_swiglu_q8(inp.x[pick], scale, idx[pick], Wgf, Wuf, rbg, rbu, inp.call.eps)
    else:
        Pg, Pu = fn.fold_weights_fp8(g, Wg), fn.fold_weights_fp8(g, Wu)
        codes, scales = fn.norm_proj_swiglu_adaln_fp8_q8_ws(x, sc, _idx_dev(idx), Pg, bg, Pu, bu, inp.call.eps)
        cg, sg = oracle.fold_weights_fp8(inp.g, inp.W, "bf16")
        cu, su = oracle.fold_weights_fp8(inp.g, inp.W_up, "bf16")
        _, _, v = oracle.adaln_norm_proj_swiglu_fp8_q8(inp.x[pick], scale, idx[pick], cg, sg, cu, su, rbg, rbu,
                                                       inp.call.eps)
    return codes.cpu().numpy()[pick], scales.cpu().numpy()[pick], v


@pytest.mark.parametrize("weights", ["bf16", "fp8"])
@pytest.mark.parametrize("M,K,N,T", [(1, 8, 16, 1), (5, 264, 100, 3), (16, 1032, 270, 5), (17, 256, 48, 100),
                                     (40, 1032, 270, 4), (64, 264, 1100, 2), (65, 256, 160, 3), (130, 520, 33, 30),
                                     (300, 136, 530, 7)])
def test_adaln_q8_parity(gpu_lib, weights, M, K, N, T):
    codes, scales, v = _run(gpu_lib, M, K, N, T, weights, seed=M * 13 + K + N + T)
    assert_q8_close(codes, scales, v, f"adaln q8 {weights} {M}x{K}x{N} T={T}")


@pytest.mark.parametrize("weights", ["bf16", "fp8"])
def test_adaln_q8_ffn_decode_shape(gpu_lib, weights):
    """The FFN decode shape (64 x 4096 -> 2 x 11008), four table rows."""
    codes, scales, v = _run(gpu_lib, 64, 4096, 11008, 4, weights, seed=12, bad_idx=False)
    flips = assert_q8_close(codes, scales, v, f"adaln q8 {weights} FFN decode")
    print(f"midpoint flips: {flips} of {codes.size}")


def test_adaln_q8_prefill_sampled_rows(gpu_lib):
    """4096 rows through the prefill kernel's fp8 epilogue on the modulated
    operand; the oracle on a seeded sample of rows."""
    M, K, N = 4096, 1024, 2048
    assert gpu_lib.kernel_name_adaln_q8(M, K, N, 8, False).startswith("prefill_swiglu_bf16_q8_premod")
    rows = W.sample_indices(M, 48, seed=6)
    codes, scales, v = _run(gpu_lib, M, K, N, 8, "bf16", seed=78, rows=rows)
    assert_q8_close(codes, scales, v, "adaln q8 prefill rows")
