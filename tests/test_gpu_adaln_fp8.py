"""GPU parity of AdaLN with fp8 weights (E4M3 codes of the plain W, one
scale per output column; two launches: the modulation pre-pass, then the
fp8-weight kernel of the row count on the modulated operand) against the
float64 oracle on the same codes, every output held to the tolerance rule
and to the bound derived from the arithmetic (the operand rounded once for
the projection, split exactly in two parts for SwiGLU; the codes decode
exactly)."""
import numpy as np
import pytest

from tests.gpu_helpers import AdalnCase, assert_adaln_close, to_f64

pytestmark = pytest.mark.gpu


def _run(fn, M, K, N, T, swiglu, seed, bad_idx=True):
    c = AdalnCase(fn, M, K, N, T, swiglu, seed=seed, bad_idx=bad_idx, weights="fp8")
    f = fn.norm_proj_swiglu_adaln_fp8_ws if swiglu else fn.norm_proj_adaln_fp8_ws
    return to_f64(f(c.x, *c.args(), c.eps)), c


@pytest.mark.parametrize("swiglu", [False, True])
@pytest.mark.parametrize("M,K,N,T", [(1, 8, 16, 1), (5, 264, 100, 3), (16, 1032, 270, 5), (17, 4104, 530, 100),
                                     (33, 264, 1100, 2), (64, 1032, 48, 7), (65, 520, 33, 3), (200, 264, 160, 30)])
def test_adaln_fp8_parity(gpu_lib, swiglu, M, K, N, T):
    y, c = _run(gpu_lib, M, K, N, T, swiglu, seed=M * 11 + K + N + T)
    assert_adaln_close(y, c.reference(), c.value_error_bound(),
                       f"{'swiglu' if swiglu else 'proj'} adaln fp8 {M}x{K}x{N} T={T}")


@pytest.mark.parametrize("M,K,N,T,swiglu", [(100, 264, 8200, 5, False), (256, 136, 8192, 3, False),
                                             (65, 264, 8208, 7, True), (128, 72, 8200, 30, True),
                                             (150, 8, 8192, 2, False), (70, 8, 8200, 2, True)])
def test_adaln_fp8_rows_tiled_parity(gpu_lib, M, K, N, T, swiglu):
    """Past 64 rows of projections with at least 512 column blocks (up to
    256 rows, 128 for the SwiGLU pair) the 64-row decode tiles repeat over
    the rows on the modulated operand: every output."""
    assert gpu_lib.kernel_name_adaln_fp8(M, K, N, T, swiglu).startswith(("decode_fp8", "decode_swiglu_fp8"))
    y, c = _run(gpu_lib, M, K, N, T, swiglu, seed=M * 3 + K + N + T)
    assert_adaln_close(y, c.reference(), c.value_error_bound(),
                       f"{'swiglu' if swiglu else 'proj'} adaln fp8 rows tiled {M}x{K}x{N} T={T}")


@pytest.mark.parametrize("M,N,swiglu", [(16, 12288, False), (64, 11008, True), (4096, 11008, True)])
def test_adaln_fp8_decode_and_prefill_shapes(gpu_lib, M, N, swiglu):
    """The QKV and FFN decode shapes and the FFN prefill shape (K = 4096)
    with four table rows, every output."""
    y, c = _run(gpu_lib, M, 4096, N, 4, swiglu, seed=M + N, bad_idx=False)
    err = assert_adaln_close(y, c.reference(), c.value_error_bound(), f"adaln fp8 {M}x4096x{N}")
    print(f"adaln fp8 {M}x4096x{N}: max |err|/(|ref|+1) = {err:.2e}")


def test_adaln_fp8_identity_modulation_matches_the_plain_fp8_path(gpu_lib):
    """g = 1, scale 0 and zero bias rows: the operand is x itself, so the
    output equals the plain fp8 call's within the fp32 sum order (the two
    kernels take the sums of squares differently)."""
    import torch
    import workloads as W
    from tests.gpu_helpers import to_dev
    fn = gpu_lib
    M, K, N = 64, 1032, 530
    inp = W.random_inputs(M, K, N, "bf16", seed=4, swiglu=True)
    x = to_dev(inp.x, "bf16")
    Pg, Pu = fn.fold_weights_fp8(None, to_dev(inp.W, "bf16")), fn.fold_weights_fp8(None, to_dev(inp.W_up, "bf16"))
    ones = torch.ones((K,), dtype=torch.bfloat16, device="cuda")
    mod = fn.adaln_fold_table(ones, torch.zeros((3, K), dtype=torch.bfloat16, device="cuda"))
    b = torch.zeros((3, N), dtype=torch.float32, device="cuda")
    idx = torch.zeros((M,), dtype=torch.int32, device="cuda")
    y = to_f64(fn.norm_proj_swiglu_adaln_fp8_ws(x, mod, idx, Pg, b, Pu, b, 1e-6))
    want = to_f64(fn.norm_proj_swiglu_fp8(x, Pg, Pu, 1e-6))
    assert np.all(np.abs(y - want) <= 2.0 ** -7 * np.abs(want) + 1e-6)
