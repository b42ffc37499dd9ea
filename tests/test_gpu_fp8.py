"""GPU parity of the fp8-weight path (E4M3 codes, one scale per output
column) against the float64 oracle: the fold and quantisation bit for bit
(codes and scales), the fused calls within the bf16 tolerance."""
import numpy as np
import pytest

import oracle
import workloads as W
from tests.gpu_helpers import assert_close, pack_fp8_host, to_dev, to_f64

pytestmark = pytest.mark.gpu


def _fold8(fn, g, Wm, dtype):
    return fn.fold_weights_fp8(None if g is None else to_dev(g, dtype), to_dev(Wm, dtype))


@pytest.mark.parametrize("dtype", ["bf16", "f32"])
@pytest.mark.parametrize("K,N", [(8, 1), (40, 37), (72, 17), (256, 768), (4104, 100)])
def test_fold_fp8_bit_exact(gpu_lib, dtype, K, N):
    inp = W.random_inputs(2, K, N, dtype, seed=K * 13 + N)
    Wm = inp.W.copy()
    Wm[:, N // 2] = 0.0                     # an all-zero column takes s = 1
    P = _fold8(gpu_lib, inp.g, Wm, dtype)
    codes, s = oracle.fold_weights_fp8(inp.g, Wm, dtype)
    got = P.data.cpu().numpy()
    want = pack_fp8_host(codes)
    assert got.shape == want.shape
    bad = np.nonzero(got != want)[0]
    assert bad.size == 0, f"{bad.size} code bytes differ, first at {bad[:5]}: {got[bad[:5]]} vs {want[bad[:5]]}"
    assert np.array_equal(P.scales.cpu().numpy(), s), "column scales"
    Pn = _fold8(gpu_lib, None, Wm, dtype)   # g = None quantises W as stored
    codes_n, s_n, _ = oracle.quantize_e4m3_columns(Wm)
    assert np.array_equal(Pn.data.cpu().numpy(), pack_fp8_host(codes_n))
    assert np.array_equal(Pn.scales.cpu().numpy(), s_n)


def test_every_code_decodes_exactly(gpu_lib):
    """Columns holding every finite E4M3 value (largest 448, so r = s = 1 and
    the codes are the values' own): the fold reproduces each code and the
    fused product decodes each one exactly."""
    codes = np.arange(256, dtype=np.uint8)
    vals = oracle.e4m3_decode(codes)
    vals[np.isnan(vals)] = 0.0
    Wm = np.stack([np.roll(vals, 7 * n) for n in range(16)], axis=1).astype(np.float32)
    P = _fold8(gpu_lib, None, Wm, "bf16")
    want_codes, s, _ = oracle.quantize_e4m3_columns(Wm)
    assert np.all(s == 1.0)
    assert np.array_equal(P.data.cpu().numpy(), pack_fp8_host(want_codes))
    x = W.make_x(5, 256, "bf16", seed=3)
    y = to_f64(gpu_lib.norm_proj_fp8(to_dev(x, "bf16"), P, 1e-6))
    assert_close(y, oracle.norm_proj_fp8(x, want_codes, s, 1e-6), "bf16", "every code")


def _run(fn, inp, swiglu):
    c = inp.call
    x = to_dev(inp.x, "bf16")
    Pg = _fold8(fn, inp.g, inp.W, "bf16")
    cg, sg = oracle.fold_weights_fp8(inp.g, inp.W, "bf16")
    if swiglu:
        Pu = _fold8(fn, inp.g, inp.W_up, "bf16")
        cu, su = oracle.fold_weights_fp8(inp.g, inp.W_up, "bf16")
        y = fn.norm_proj_swiglu_fp8(x, Pg, Pu, c.eps)
        ref = oracle.norm_proj_swiglu_fp8(inp.x, cg, sg, cu, su, c.eps)
    else:
        y = fn.norm_proj_fp8(x, Pg, c.eps)
        ref = oracle.norm_proj_fp8(inp.x, cg, sg, c.eps)
    return to_f64(y), ref


@pytest.mark.parametrize("swiglu", [False, True])
@pytest.mark.parametrize("M,K,N", [(1, 8, 16), (3, 40, 37), (4, 256, 768), (9, 4104, 530), (16, 1032, 270),
                                   (17, 256, 48), (24, 8, 1), (32, 4104, 100), (33, 96, 100), (48, 8, 1),
                                   (63, 128, 17), (65, 256, 160), (130, 520, 33), (300, 136, 530)])
def test_fp8_parity(gpu_lib, swiglu, M, K, N):
    inp = W.random_inputs(M, K, N, "bf16", seed=M * 7 + K * 3 + N, swiglu=swiglu)
    y, ref = _run(gpu_lib, inp, swiglu)
    assert_close(y, ref, "bf16", f"fp8 {M}x{K}x{N} swiglu={swiglu}")


@pytest.mark.parametrize("M,K,N,swiglu", [(65, 264, 8200, False), (130, 1032, 8192, True), (256, 136, 8200, False),
                                          (200, 4104, 8200, True), (128, 4096, 12288, False)])
def test_fp8_rows_tiled_decode_parity(gpu_lib, M, K, N, swiglu):
    """65..256 rows of a wide projection with fp8 weights run the decode
    kernel's 64-row (projection) or 128-row (SwiGLU) blocks tiled over the
    rows (a ragged last block): every output against the oracle."""
    assert gpu_lib.kernel_name_fp8(M, K, N, swiglu).startswith("decode")
    inp = W.random_inputs(M, K, N, "bf16", seed=M * 5 + K + N, swiglu=swiglu)
    y, ref = _run(gpu_lib, inp, swiglu)
    assert_close(y, ref, "bf16", f"fp8 rows tiled {M}x{K}x{N} swiglu={swiglu}")


@pytest.mark.parametrize("M,K,N,swiglu", [(1, 8, 16, False), (16, 72, 1540, False), (9, 264, 4096, True),
                                          (16, 4104, 1380, True), (5, 1032, 100, False), (12, 4096, 4000, False)])
def test_fp8_narrow_ksplit_parity(gpu_lib, M, K, N, swiglu):
    """Up to 16 rows of at most 256 column blocks with fp8 weights: the
    register-x tile with k split over four waves (uneven and empty k ranges,
    ragged K and N): every output against the oracle."""
    assert "_k4_" in gpu_lib.kernel_name_fp8(M, K, N, swiglu)
    inp = W.random_inputs(M, K, N, "bf16", seed=M * 11 + K + N, swiglu=swiglu)
    y, ref = _run(gpu_lib, inp, swiglu)
    assert_close(y, ref, "bf16", f"fp8 k-split {M}x{K}x{N} swiglu={swiglu}")


@pytest.mark.parametrize("M,K,N,swiglu", [(1024, 72, 1380, True), (700, 136, 3000, False), (400, 136, 6000, False),
                                          (256, 72, 8100, False), (333, 264, 5500, True)])
def test_fp8_narrow_rows_tiled_parity(gpu_lib, M, K, N, swiglu):
    """Narrow projections with fp8 weights keep the decode kernel's row
    blocks tiled over the rows further: to 1024 rows at 192 column blocks or
    fewer, 512 to 384 blocks, 256 above (ragged rows, K and N): every
    output against the oracle."""
    assert gpu_lib.kernel_name_fp8(M, K, N, swiglu).startswith("decode")
    inp = W.random_inputs(M, K, N, "bf16", seed=M * 3 + K + N, swiglu=swiglu)
    y, ref = _run(gpu_lib, inp, swiglu)
    assert_close(y, ref, "bf16", f"fp8 narrow rows tiled {M}x{K}x{N} swiglu={swiglu}")


def test_fp8_qkv_decode_full(gpu_lib):
    inp = W.make_inputs(W.QKV_DECODE)
    y, ref = _run(gpu_lib, inp, False)
    assert_close(y, ref, "bf16", "fp8 QKV decode")


def test_fp8_ffn_decode_full(gpu_lib):
    inp = W.make_inputs(W.FFN_DECODE)
    y, ref = _run(gpu_lib, inp, True)
    assert_close(y, ref, "bf16", "fp8 FFN decode")


@pytest.mark.parametrize("idx", [0, 1, 64])
def test_fp8_decode_step_calls_full(gpu_lib, idx):
    """The M=8 calls of the decode step (QKV, gate/up SwiGLU, LM head) at full size."""
    c = W.decode_step_calls()[idx]
    inp = W.make_inputs(c)
    y, ref = _run(gpu_lib, inp, c.swiglu)
    assert_close(y, ref, "bf16", f"fp8 {c.name}")


def test_fp8_binding_rejects(gpu_lib):
    import torch
    P = gpu_lib.fold_weights_fp8(None, torch.zeros((64, 32), dtype=torch.bfloat16, device="cuda"))
    with pytest.raises(ValueError):
        gpu_lib.norm_proj_fp8(torch.zeros((2, 64), dtype=torch.float32, device="cuda"), P)
    with pytest.raises(ValueError):
        gpu_lib.norm_proj_fp8(torch.zeros((2, 48), dtype=torch.bfloat16, device="cuda"), P)
    y = gpu_lib.norm_proj_fp8(torch.zeros((0, 64), dtype=torch.bfloat16, device="cuda"), P)
    assert tuple(y.shape) == (0, 32)


@pytest.mark.parametrize("N,swiglu", [(12288, False), (11008, True)])
def test_fp8_prefill_full(gpu_lib, N, swiglu):
    """4096 rows x 4096 through the prefill kernel with fp8 weights (the
    QKV projection and the FFN gate/up pair), every output against the
    oracle with the same codes and scales."""
    import torch
    fn = gpu_lib
    M, K = 4096, 4096
    assert fn.kernel_name_fp8(M, K, N, swiglu).startswith("prefill_")
    inp = W.random_inputs(M, K, N, "bf16", seed=91, swiglu=swiglu)
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
    torch.cuda.synchronize()
    err = assert_close(to_f64(y), ref, "bf16", f"fp8 prefill {M}x{K}x{N} swiglu={swiglu}")
    print(f"fp8 prefill {M}x{K}x{N} swiglu={swiglu}: max |err|/(|ref|+1) = {err:.2e}")


@pytest.mark.parametrize("M,K,N", [(65, 64, 16), (97, 8, 1), (256, 200, 300), (257, 4104, 33), (1000, 1032, 1100),
                                   (2048, 264, 768)])
def test_fp8_prefill_ragged(gpu_lib, M, K, N):
    """Ragged rows, columns and k (a half pair at the end) through the fp8
    prefill instances, projection and SwiGLU."""
    for swiglu in (False, True):
        inp = W.random_inputs(M, K, N, "bf16", seed=M + K + N + int(swiglu), swiglu=swiglu)
        y, ref = _run(gpu_lib, inp, swiglu)
        assert_close(y, ref, "bf16", f"fp8 prefill {M}x{K}x{N} swiglu={swiglu}")
