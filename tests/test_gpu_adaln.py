"""GPU parity of the AdaLN prologue (h = RMSNorm_g(x) * (1 + scale[idx]) +
shift[idx] before the projection / SwiGLU) against the float64 oracle of
the unfolded definition, every output held to the tolerance rule
2e-2 (|ref| + 1) and to a tighter bound derived from the arithmetic: the
bf16 operand x * mod is rounded once (the projection) or split exactly in
two parts (SwiGLU), the plain weights are exact, sums are fp32.  Also the
offline forms (the gain-folded table, the bias rows) and the pre-pass
operand bit for bit."""
import numpy as np
import pytest

import oracle
import workloads as W
from tests.gpu_helpers import (AdalnCase, assert_adaln_close, idx_dev, storage_bits, to_dev, to_f64)

pytestmark = pytest.mark.gpu


@pytest.mark.parametrize("dtype", ["bf16", "f32"])
@pytest.mark.parametrize("T,K,N", [(1, 8, 16), (3, 264, 530), (5, 4104, 33)])
def test_adaln_shift_bias(gpu_lib, dtype, T, K, N):
    inp = W.random_inputs(2, K, N, dtype, seed=T * 31 + K + N)
    _, shift, _ = W.adaln_tables(T, K, 2, seed=K + N, dtype=dtype)
    got = to_f64(gpu_lib.adaln_shift_bias(to_dev(shift, dtype), to_dev(inp.W, dtype)))
    ref = oracle.adaln_shift_bias(shift, inp.W)
    # fp32 sum of K products against float64
    bound = 1e-5 * (np.abs(shift.astype(np.float64)) @ np.abs(inp.W.astype(np.float64))) + 1e-6
    assert np.all(np.abs(got - ref) <= bound)


@pytest.mark.parametrize("dtype", ["bf16", "f32"])
@pytest.mark.parametrize("T,K", [(1, 8), (7, 1032), (300, 4096)])
def test_adaln_fold_table_bit_exact(gpu_lib, dtype, T, K):
    """mod = fp32(g * (1 + scale)) from float64 arithmetic: bit for bit."""
    inp = W.random_inputs(1, K, 16, dtype, seed=T + K)
    scale, _, _ = W.adaln_tables(T, K, 1, seed=T * K, dtype=dtype)
    scale[0, :4] = [0.0, -1.0, 2.0 ** -24, 3.0]          # exact cases and a float64-then-float32 rounding
    got = gpu_lib.adaln_fold_table(to_dev(inp.g, dtype), to_dev(scale, dtype)).cpu().numpy()
    want = oracle.adaln_fold_table(inp.g, scale).astype(np.float32)
    assert np.array_equal(got.view(np.uint32), want.view(np.uint32))


# one launch: up to 16 rows
@pytest.mark.parametrize("swiglu", [False, True])
@pytest.mark.parametrize("M,K,N,T", [(1, 8, 16, 1), (3, 40, 37, 2), (9, 4104, 530, 3), (16, 1032, 270, 5),
                                     (16, 264, 100, 24), (5, 264, 1100, 500), (16, 4096, 12288, 4)])
def test_adaln_one_launch_parity(gpu_lib, swiglu, M, K, N, T):
    c = AdalnCase(gpu_lib, M, K, N, T, swiglu, seed=M * 3 + K + N + T, bad_idx=True)
    f = gpu_lib.norm_proj_swiglu_adaln if swiglu else gpu_lib.norm_proj_adaln
    y = to_f64(f(c.x, *c.args(), c.eps))
    assert_adaln_close(y, c.reference(), c.value_error_bound(),
                       f"{'swiglu' if swiglu else 'proj'} adaln one launch {M}x{K}x{N} T={T}")


def test_adaln_one_launch_takes_at_most_16_rows(gpu_lib):
    c = AdalnCase(gpu_lib, 17, 264, 100, 3, False, seed=1)
    with pytest.raises(gpu_lib.FlashNormError, match="at most 16 rows"):
        gpu_lib.norm_proj_adaln(c.x, *c.args(), c.eps)
    assert gpu_lib.kernel_name_adaln(17, 264, 100, 3, False) == "invalid"


# two launches: the pre-pass, then the projection kernel of the row count
@pytest.mark.parametrize("swiglu", [False, True])
@pytest.mark.parametrize("M,K,N,T", [
    # 17..64 rows: the LDS-shared-x decode kernel on the pre-modulated operand
    (17, 1032, 270, 23), (33, 4104, 530, 100), (40, 1032, 270, 4), (40, 1032, 270, 30), (64, 264, 1100, 3),
    (64, 4104, 530, 40),
    # above: the same kernel's 64-row blocks tiled over the rows (narrow
    # projections up to 512 rows here; not the split SwiGLU operand), else
    # the prefill kernel
    (65, 256, 160, 2), (130, 520, 33, 3), (300, 1032, 530, 5), (257, 264, 1100, 64), (520, 4104, 270, 63),
    (200, 1032, 300, 500), (777, 264, 48, 1)])
def test_adaln_ws_parity(gpu_lib, swiglu, M, K, N, T):
    """Ragged row, column and k tails through the pre-pass and both
    projection kernels, any table size, indices outside the table."""
    c = AdalnCase(gpu_lib, M, K, N, T, swiglu, seed=M * 5 + K + N + T, bad_idx=True)
    f = gpu_lib.norm_proj_swiglu_adaln_ws if swiglu else gpu_lib.norm_proj_adaln_ws
    y = to_f64(f(c.x, *c.args(), c.eps))
    assert_adaln_close(y, c.reference(), c.value_error_bound(),
                       f"{'swiglu' if swiglu else 'proj'} adaln two launches {M}x{K}x{N} T={T}")


@pytest.mark.parametrize("M,K,N,T", [(65, 264, 8200, 3), (128, 136, 8192, 40), (100, 4104, 8208, 5), (90, 8, 8192, 2)])
def test_adaln_ws_rows_tiled_parity(gpu_lib, M, K, N, T):
    """65..128 rows of a projection with at least 512 column blocks: the
    64-row decode tiles repeat over the rows on the modulated operand (the
    SwiGLU pair, whose operand is split in two, stays on the prefill
    kernel): every output."""
    assert gpu_lib.kernel_name_adaln_ws(M, K, N, T, False).startswith("decode_premod_bf16_m64")
    assert gpu_lib.kernel_name_adaln_ws(M, K, N, T, True).startswith("prefill_swiglu_premod_split")
    c = AdalnCase(gpu_lib, M, K, N, T, False, seed=M * 3 + K + N + T, bad_idx=True)
    y = to_f64(gpu_lib.norm_proj_adaln_ws(c.x, *c.args(), c.eps))
    assert_adaln_close(y, c.reference(), c.value_error_bound(), f"proj adaln rows tiled {M}x{K}x{N} T={T}")


@pytest.mark.parametrize("M,K,N,T", [(129, 72, 8192, 2), (160, 264, 8200, 9)])
def test_adaln_ws_prefill_128_row_tiles_parity(gpu_lib, M, K, N, T):
    """129..256 rows of a wide projection: the prefill kernel's 128-row
    tiles on the modulated operand, every output."""
    assert gpu_lib.kernel_name_adaln_ws(M, K, N, T, False) == "prefill_premod_bf16_128x128_w4x2"
    c = AdalnCase(gpu_lib, M, K, N, T, False, seed=M + K + N + T, bad_idx=True)
    y = to_f64(gpu_lib.norm_proj_adaln_ws(c.x, *c.args(), c.eps))
    assert_adaln_close(y, c.reference(), c.value_error_bound(), f"proj adaln 128-row tiles {M}x{K}x{N} T={T}")


@pytest.mark.parametrize("M,N,swiglu", [(16, 12288, False), (64, 11008, True), (64, 12288, False)])
def test_adaln_decode_shapes(gpu_lib, M, N, swiglu):
    """The QKV and FFN decode shapes (K = 4096) with four table rows, every
    output."""
    c = AdalnCase(gpu_lib, M, 4096, N, 4, swiglu, seed=11 + M + N)
    f = gpu_lib.norm_proj_swiglu_adaln_ws if swiglu else gpu_lib.norm_proj_adaln_ws
    y = to_f64(f(c.x, *c.args(), c.eps))
    err = assert_adaln_close(y, c.reference(), c.value_error_bound(), f"adaln decode {M}x4096x{N}")
    print(f"adaln decode {M}x4096x{N}: max |err|/(|ref|+1) = {err:.2e}")


@pytest.mark.parametrize("N,T,swiglu", [(12288, 8, False), (11008, 16, True)])
def test_adaln_prefill_full(gpu_lib, N, T, swiglu):
    """4096 rows x 4096 through the two-launch prefill path (the QKV
    projection with 8 table rows; the FFN gate/up SwiGLU 2 x 11008 with 16),
    every output against the oracle."""
    import torch
    c = AdalnCase(gpu_lib, 4096, 4096, N, T, swiglu, seed=43 + N)
    f = gpu_lib.norm_proj_swiglu_adaln_ws if swiglu else gpu_lib.norm_proj_adaln_ws
    y = f(c.x, *c.args(), c.eps)
    torch.cuda.synchronize()
    err = assert_adaln_close(to_f64(y), c.reference(), c.value_error_bound(), f"adaln prefill 4096x4096x{N}")
    print(f"adaln prefill 4096x4096x{N}: max |err|/(|ref|+1) = {err:.2e}")


def test_adaln_identity_modulation_matches_plain(gpu_lib):
    """g = 1, scale 0, shift 0: the modulated operand is x itself and W' = W,
    so the AdaLN calls and the plain fused calls compute the same products
    (their sums of squares differ only in fp32 order)."""
    import torch
    fn = gpu_lib
    for M, swiglu in ((16, True), (64, True), (300, False), (300, True)):
        K, N, T = 1032, 530, 2
        inp = W.random_inputs(M, K, N, "bf16", seed=M, swiglu=swiglu)
        x = to_dev(inp.x, "bf16")
        ones = torch.ones((K,), dtype=torch.bfloat16, device="cuda")
        mod = fn.adaln_fold_table(ones, torch.zeros((T, K), dtype=torch.bfloat16, device="cuda"))
        b = torch.zeros((T, N), dtype=torch.float32, device="cuda")
        idx = torch.zeros((M,), dtype=torch.int32, device="cuda")
        Pg = fn.fold_weights(None, to_dev(inp.W, "bf16"))
        if swiglu:
            Pu = fn.fold_weights(None, to_dev(inp.W_up, "bf16"))
            y = to_f64(fn.norm_proj_swiglu_adaln_ws(x, mod, idx, Pg, b, Pu, b, 1e-6))
            want = to_f64(fn.norm_proj_swiglu(x, Pg, Pu, 1e-6))
        else:
            y = to_f64(fn.norm_proj_adaln_ws(x, mod, idx, Pg, b, 1e-6))
            want = to_f64(fn.norm_proj(x, Pg, 1e-6))
        assert np.all(np.abs(y - want) <= 2.0 ** -7 * np.abs(want) + 1e-5), (M, swiglu)


def test_adaln_kernel_choice(gpu_lib):
    """One launch up to 16 rows; two launches: the decode kernel up to 64
    rows, the prefill kernel above; SwiGLU on the split operand."""
    fn = gpu_lib
    assert fn.kernel_name_adaln(16, 4096, 11008, 4, True).startswith("decode_swiglu_adaln_split")
    assert fn.kernel_name_adaln_ws(64, 4096, 11008, 4, True).startswith("decode_swiglu_premod_split")
    assert fn.kernel_name_adaln_ws(64, 4096, 12288, 4, False).startswith("decode_premod_bf16_m64")
    assert fn.kernel_name_adaln_ws(65, 4096, 11008, 63, True).startswith("prefill_swiglu_premod_split")
    assert fn.kernel_name_adaln_ws(4096, 4096, 12288, 64, False).startswith("prefill_premod_bf16")


def _bf16_bits(t):
    import torch
    return t.view(torch.int16).cpu().numpy().view(np.uint16)


@pytest.mark.parametrize("M,K,T", [(1, 8, 1), (5, 264, 3), (70, 1032, 5), (301, 4104, 100), (4096, 4096, 4)])
def test_adaln_modulate_matches_oracle(gpu_lib, M, K, T):
    """The pre-pass operand bit for bit (a rounding decides every bit: the
    oracle takes it in the same two steps, fp32 then bf16; a zero row for an
    index outside the table), and 1/RMS of the raw rows within the fp32
    bound of its sum."""
    fn = gpu_lib
    seed = M + K + T
    inp = W.random_inputs(M, K, 16, "bf16", seed=seed)
    scale, _, idx = W.adaln_tables(T, K, M, seed=seed + 1)
    if M >= 3:
        idx[0], idx[-1] = -1, T           # outside the table
    mod = fn.adaln_fold_table(to_dev(inp.g, "bf16"), to_dev(scale, "bf16"))
    u, rs = fn.adaln_modulate(to_dev(inp.x, "bf16"), mod, idx_dev(idx), 1e-6)
    want = oracle.adaln_operand(inp.x, oracle.adaln_fold_table(inp.g, scale), idx)
    got = _bf16_bits(u)
    bad = got != storage_bits(want, "bf16")
    assert not bad.any(), f"{bad.sum()} operand values differ, first at {np.argwhere(bad)[:3].tolist()}"
    ref = 1.0 / oracle.rms(inp.x, 1e-6)
    # each lane sums K/64 squares in order, then six pairwise steps; sqrt and division add a few ulps
    rel = (K / 64 + 16) * 2.0 ** -24 + 4 * 2.0 ** -24
    err = np.abs(to_f64(rs) - ref) / ref
    assert np.all(err <= rel), f"1/RMS off by {err.max():.2e} > {rel:.2e}"


def test_adaln_ws_workspace_reuse(gpu_lib):
    """One workspace for two calls in a row, the second with fewer rows
    (its contents from the first call are overwritten, not trusted)."""
    import torch
    fn = gpu_lib
    ws = torch.empty((fn.adaln_workspace_bytes(300, 1032),), dtype=torch.uint8, device="cuda")
    for M in (300, 97):
        c = AdalnCase(fn, M, 1032, 270, 7, True, seed=M)
        y = to_f64(fn.norm_proj_swiglu_adaln_ws(c.x, *c.args(), c.eps, workspace=ws))
        assert_adaln_close(y, c.reference(), c.value_error_bound(), f"shared workspace, M={M}")


def test_adaln_ws_up_to_16_rows_is_the_one_launch_call(gpu_lib):
    """Up to 16 rows the two-launch entry runs the one-launch kernel: the
    same bits, with no workspace."""
    import torch
    fn = gpu_lib
    c = AdalnCase(fn, 16, 1032, 530, 5, True, seed=8)
    assert fn.adaln_workspace_bytes(16, 1032) == 0
    a = fn.norm_proj_swiglu_adaln_ws(c.x, *c.args(), 1e-6)
    b = fn.norm_proj_swiglu_adaln(c.x, *c.args(), 1e-6)
    assert torch.equal(a.view(torch.int16), b.view(torch.int16))
