"""GPU parity of SwiGLU with fp8 output (E4M3 codes, one scale per 16-column
row block) against the float64 oracle, for bf16 weights (LDS-shared-x decode
kernel up to 64 rows, prefill kernel above) and fp8 weights (any M).  The
reference is taken on the folded weights the GPU reads (bf16 W', or the
E4M3 codes and column scales), so fp32-vs-float64 arithmetic is the only
difference and codes must match except at rounding midpoints."""
import numpy as np
import pytest

import oracle
import workloads as W
from tests.gpu_helpers import assert_q8_close, to_dev

pytestmark = pytest.mark.gpu

SHAPES = [(1, 8, 16), (3, 40, 37), (9, 4104, 530), (16, 1032, 270), (17, 256, 48), (33, 96, 100),
          (40, 1032, 270), (61, 4104, 530), (64, 264, 1100), (65, 256, 160), (130, 520, 33), (300, 136, 530)]


def _bf16_case(fn, inp):
    x = to_dev(inp.x, "bf16")
    Pg = fn.fold_weights(to_dev(inp.g, "bf16"), to_dev(inp.W, "bf16"))
    Pu = fn.fold_weights(to_dev(inp.g, "bf16"), to_dev(inp.W_up, "bf16"))
    codes, scales = fn.norm_proj_swiglu_q8(x, Pg, Pu, inp.call.eps)
    Wg = oracle.fold_weights(inp.g, inp.W, "bf16")
    Wu = oracle.fold_weights(inp.g, inp.W_up, "bf16")
    v = oracle.norm_proj_swiglu_folded(inp.x, Wg, Wu, inp.call.eps)
    return codes.cpu().numpy(), scales.cpu().numpy(), v


def _fp8_case(fn, inp):
    x = to_dev(inp.x, "bf16")
    Pg = fn.fold_weights_fp8(to_dev(inp.g, "bf16"), to_dev(inp.W, "bf16"))
    Pu = fn.fold_weights_fp8(to_dev(inp.g, "bf16"), to_dev(inp.W_up, "bf16"))
    codes, scales = fn.norm_proj_swiglu_fp8_q8(x, Pg, Pu, inp.call.eps)
    cg, sg = oracle.fold_weights_fp8(inp.g, inp.W, "bf16")
    cu, su = oracle.fold_weights_fp8(inp.g, inp.W_up, "bf16")
    v = oracle.norm_proj_swiglu_fp8(inp.x, cg, sg, cu, su, inp.call.eps)
    return codes.cpu().numpy(), scales.cpu().numpy(), v


@pytest.mark.parametrize("weights", ["bf16", "fp8"])
@pytest.mark.parametrize("M,K,N", SHAPES)
def test_q8_parity(gpu_lib, weights, M, K, N):
    inp = W.random_inputs(M, K, N, "bf16", seed=M * 5 + K * 7 + N, swiglu=True)
    codes, scales, v = (_bf16_case if weights == "bf16" else _fp8_case)(gpu_lib, inp)
    assert_q8_close(codes, scales, v, f"q8 {weights} {M}x{K}x{N}")


@pytest.mark.parametrize("weights,M,K,N", [("bf16", 65, 264, 8200), ("bf16", 128, 136, 8192), ("bf16", 97, 8, 8192),
                                           ("fp8", 100, 264, 8200), ("fp8", 256, 72, 8208), ("fp8", 200, 8, 8192)])
def test_q8_rows_tiled_parity(gpu_lib, weights, M, K, N):
    """Past 64 rows of projections with at least 512 column blocks (up to
    128 rows with bf16 weights, 256 with fp8) the 64-row decode tiles repeat
    over the rows (ragged rows, K and N): every output against the oracle."""
    assert gpu_lib.kernel_name_q8(M, K, N, weights == "fp8").startswith("decode_swiglu")
    inp = W.random_inputs(M, K, N, "bf16", seed=M * 3 + K + N, swiglu=True)
    codes, scales, v = (_bf16_case if weights == "bf16" else _fp8_case)(gpu_lib, inp)
    assert_q8_close(codes, scales, v, f"q8 rows tiled {weights} {M}x{K}x{N}")


@pytest.mark.parametrize("M,K,N", [(129, 72, 8192), (200, 264, 8200)])
def test_q8_prefill_128_row_tiles_parity(gpu_lib, M, K, N):
    """129..256 rows of a wide projection with bf16 weights: the prefill
    kernel's 128-row tiles with the fp8 epilogue, every output."""
    assert "128x128" in gpu_lib.kernel_name_q8(M, K, N, False)
    inp = W.random_inputs(M, K, N, "bf16", seed=M + K * 3 + N, swiglu=True)
    codes, scales, v = _bf16_case(gpu_lib, inp)
    assert_q8_close(codes, scales, v, f"q8 128-row tiles {M}x{K}x{N}")


@pytest.mark.parametrize("weights", ["bf16", "fp8"])
def test_q8_ffn_decode_full(gpu_lib, weights):
    inp = W.make_inputs(W.FFN_DECODE)
    codes, scales, v = (_bf16_case if weights == "bf16" else _fp8_case)(gpu_lib, inp)
    flips = assert_q8_close(codes, scales, v, f"q8 {weights} FFN decode")
    print(f"midpoint flips: {flips} of {codes.size}")


def test_q8_prefill_full(gpu_lib):
    """4096 rows through the prefill kernel's fp8 epilogue, every output."""
    import torch
    M, K, N = 4096, 1024, 2048
    inp = W.random_inputs(M, K, N, "bf16", seed=77, swiglu=True)
    x = to_dev(inp.x, "bf16")
    Pg = gpu_lib.fold_weights(to_dev(inp.g, "bf16"), to_dev(inp.W, "bf16"))
    Pu = gpu_lib.fold_weights(to_dev(inp.g, "bf16"), to_dev(inp.W_up, "bf16"))
    assert gpu_lib.kernel_name_q8(M, K, N, False).startswith("prefill_swiglu_bf16_q8")
    c, s = gpu_lib.norm_proj_swiglu_q8(x, Pg, Pu, 1e-6)
    torch.cuda.synchronize()
    Wg = oracle.fold_weights(inp.g, inp.W, "bf16")
    Wu = oracle.fold_weights(inp.g, inp.W_up, "bf16")
    v = oracle.norm_proj_swiglu_folded(inp.x, Wg, Wu, 1e-6)
    assert_q8_close(c.cpu().numpy(), s.cpu().numpy(), v, "q8 prefill")


def test_q8_nan_row_and_zero_blocks(gpu_lib):
    """A NaN in x row 2 makes that row's codes NaN (0x7F) and scales NaN and
    touches no other row; all-zero weight columns give all-zero blocks
    (scale 1, code 0)."""
    M, K, N = 5, 64, 40
    inp = W.random_inputs(M, K, N, "bf16", seed=9, swiglu=True)
    inp.x[2, 7] = np.nan
    inp.W[:, 16:32] = 0.0
    codes, scales, v = _bf16_case(gpu_lib, inp)
    assert np.all(codes[2] == 0x7F) and np.all(np.isnan(scales[2]))
    assert np.all(scales[[0, 1, 3, 4], 1] == 1.0) and np.all(codes[[0, 1, 3, 4], 16:32] & 0x7F == 0)
    keep = [0, 1, 3, 4]
    assert_q8_close(codes[keep], scales[keep], v[keep], "q8 rows next to a NaN row")


def test_q8_in_a_recorded_step(gpu_lib):
    """q8 calls recorded into a step replay bit for bit like the eager calls."""
    import torch
    fn = gpu_lib
    st = fn.Step()
    items = []
    for i, (M, K, N, f8) in enumerate([(8, 1032, 270, False), (40, 256, 100, True), (100, 264, 48, False)]):
        inp = W.random_inputs(M, K, N, "bf16", seed=300 + i, swiglu=True)
        x = to_dev(inp.x, "bf16")
        fold = fn.fold_weights_fp8 if f8 else fn.fold_weights
        Pg = fold(to_dev(inp.g, "bf16"), to_dev(inp.W, "bf16"))
        Pu = fold(to_dev(inp.g, "bf16"), to_dev(inp.W_up, "bf16"))
        c = torch.empty((M, N), dtype=torch.uint8, device="cuda")
        s = torch.empty((M, -(-N // 16)), dtype=torch.float32, device="cuda")
        (st.norm_proj_swiglu_fp8_q8 if f8 else st.norm_proj_swiglu_q8)(x, Pg, Pu, c, s, 1e-6)
        items.append((x, Pg, Pu, c, s, f8))
    st.record()
    for replay in range(3):
        for *_r, c, s, _f in items:
            c.fill_(0xAB)
            s.fill_(float("nan"))
        st.launch()
        torch.cuda.synchronize()
        for x, Pg, Pu, c, s, f8 in items:
            wc, ws = (fn.norm_proj_swiglu_fp8_q8 if f8 else fn.norm_proj_swiglu_q8)(x, Pg, Pu, 1e-6)
            torch.cuda.synchronize()
            assert torch.equal(c, wc) and torch.equal(s.view(torch.int32), ws.view(torch.int32)), f"replay {replay}"
    st.close()


def test_q8_binding_rejects(gpu_lib):
    import torch
    fn = gpu_lib
    P = fn.fold_weights(None, torch.zeros((64, 32), dtype=torch.bfloat16, device="cuda"))
    with pytest.raises(ValueError):
        fn.norm_proj_swiglu_q8(torch.zeros((2, 64), dtype=torch.bfloat16, device="cuda"), P, P,
                               out=(torch.empty((2, 32), dtype=torch.uint8, device="cuda"),
                                    torch.empty((2, 1), dtype=torch.float32, device="cuda")))
    c, s = fn.norm_proj_swiglu_q8(torch.zeros((0, 64), dtype=torch.bfloat16, device="cuda"), P, P)
    assert tuple(c.shape) == (0, 32) and tuple(s.shape) == (0, 2)
