"""GPU parity of AdaLN + SwiGLU with fp8 row-block output (E4M3 codes, one
scale per 16-column row block; two launches: the modulation pre-pass, then
the q8 kernel of the row count on the operand rounded once) against the
float64 oracle: the row-block quantisation of the definition's SwiGLU values
(bf16 weights) or of the fp8 AdaLN form's (E4M3 weights).  The codes are
decisions on values the kernel knows only to its arithmetic's error (the
bf16 operand, fp32 sums), so a code may take its neighbour where the
reference lies within that derived error of a rounding midpoint, and
nowhere else; the scales agree to the same error."""
import pytest

from tests.gpu_helpers import AdalnCase, assert_q8_close

pytestmark = pytest.mark.gpu


def _run(fn, M, K, N, T, weights, seed, bad_idx=True, rows=None):
    c = AdalnCase(fn, M, K, N, T, True, seed=seed, bad_idx=bad_idx, weights=weights)
    f = fn.norm_proj_swiglu_adaln_q8_ws if weights == "bf16" else fn.norm_proj_swiglu_adaln_fp8_q8_ws
    codes, scales = f(c.x, *c.args(), c.eps)
    pick = slice(None) if rows is None else rows
    v = c.reference(rows)
    err = c.value_error_bound(rows, split=False)
    return codes.cpu().numpy()[pick], scales.cpu().numpy()[pick], v, err


@pytest.mark.parametrize("weights", ["bf16", "fp8"])
@pytest.mark.parametrize("M,K,N,T", [(1, 8, 16, 1), (5, 264, 100, 3), (16, 1032, 270, 5), (17, 256, 48, 100),
                                     (40, 1032, 270, 4), (64, 264, 1100, 2), (65, 256, 160, 3), (130, 520, 33, 30),
                                     (300, 136, 530, 7)])
def test_adaln_q8_parity(gpu_lib, weights, M, K, N, T):
    codes, scales, v, err = _run(gpu_lib, M, K, N, T, weights, seed=M * 13 + K + N + T)
    assert_q8_close(codes, scales, v, f"adaln q8 {weights} {M}x{K}x{N} T={T}", v_err=err)


@pytest.mark.parametrize("weights,M,K,N,T", [("bf16", 96, 264, 8200, 4), ("bf16", 128, 72, 8192, 2),
                                             ("fp8", 200, 136, 8208, 9), ("fp8", 256, 72, 8200, 3),
                                             ("bf16", 77, 8, 8192, 2), ("fp8", 129, 8, 8200, 2)])
def test_adaln_q8_rows_tiled_parity(gpu_lib, weights, M, K, N, T):
    """Past 64 rows of projections with at least 512 column blocks (up to
    128 rows with bf16 weights, 256 with fp8) the 64-row decode tiles repeat
    over the rows on the modulated operand: every output."""
    assert gpu_lib.kernel_name_adaln_q8(M, K, N, T, weights == "fp8").startswith("decode_swiglu")
    codes, scales, v, err = _run(gpu_lib, M, K, N, T, weights, seed=M * 7 + K + N + T)
    assert_q8_close(codes, scales, v, f"adaln q8 rows tiled {weights} {M}x{K}x{N} T={T}", v_err=err)


def test_adaln_q8_prefill_128_row_tiles_parity(gpu_lib):
    """129..256 rows of a wide projection with bf16 weights: the prefill
    kernel's 128-row tiles on the modulated operand, every output."""
    M, K, N, T = 256, 136, 8208, 6
    assert "128x128" in gpu_lib.kernel_name_adaln_q8(M, K, N, T, False)
    codes, scales, v, err = _run(gpu_lib, M, K, N, T, "bf16", seed=91)
    assert_q8_close(codes, scales, v, f"adaln q8 128-row tiles {M}x{K}x{N}", v_err=err)


@pytest.mark.parametrize("weights", ["bf16", "fp8"])
def test_adaln_q8_ffn_decode_shape(gpu_lib, weights):
    """The FFN decode shape (64 x 4096 -> 2 x 11008), four table rows."""
    codes, scales, v, err = _run(gpu_lib, 64, 4096, 11008, 4, weights, seed=12, bad_idx=False)
    flips = assert_q8_close(codes, scales, v, f"adaln q8 {weights} FFN decode", v_err=err)
    print(f"neighbour codes within the derived error of a midpoint: {flips} of {codes.size}")


def test_adaln_q8_prefill_full(gpu_lib):
    """4096 rows through the prefill kernel's fp8 epilogue on the modulated
    operand, every output."""
    M, K, N = 4096, 1024, 2048
    assert gpu_lib.kernel_name_adaln_q8(M, K, N, 8, False).startswith("prefill_swiglu_bf16_q8_premod")
    codes, scales, v, err = _run(gpu_lib, M, K, N, 8, "bf16", seed=78)
    assert_q8_close(codes, scales, v, "adaln q8 prefill", v_err=err)
