"""GPU parity of the AdaLN prologue (h = RMSNorm_g(x) * (1 + scale[idx]) +
shift[idx] before the projection / SwiGLU) against the float64 oracle of
the unfolded definition, and of the bias rows shift @ W.  The modulated
activation is a bf16 MFMA operand, one rounding more than the plain path,
so every output is checked against an error bound derived from that
arithmetic (and projections also against the plain bf16 rule)."""
import numpy as np
import pytest

import oracle
import workloads as W
from tests.gpu_helpers import assert_close, to_dev, to_f64

pytestmark = pytest.mark.gpu


def _idx_dev(idx):
    import torch
    return torch.from_numpy(np.ascontiguousarray(idx, dtype=np.int32)).cuda()


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


def _bound(inp, scale0, shift0, idx0, swiglu, ref):
    """Per-element error bound derived from the arithmetic: every product
    x~[k] * W'[k, n] carries two bf16 roundings (the modulated operand
    x~ = x * (1 + scale) and the folded weight), each at most 2^-9 relative,
    so a = h @ W is off by at most 2^-8 * sum_k |(h - shift)[k] W[k, n]|,
    plus fp32 accumulation (1e-5 of sum_k |h[k] W[k, n]|); the bf16 output
    adds 2^-8 |ref|.  Through SwiGLU the bound on a and b propagates by
    |silu'(a)| |b| E_a + |silu(a)| E_b + E_a E_b."""
    h = oracle.adaln_modulate(inp.x, inp.g, scale0, shift0, idx0, inp.call.eps)
    hx = np.abs(h - np.asarray(shift0, np.float64)[idx0])
    def err(Wm):
        Wa = np.abs(np.asarray(Wm, np.float64))
        return 2.0 ** -8 * (hx @ Wa) + 1e-5 * (np.abs(h) @ Wa)
    if not swiglu:
        return err(inp.W) + 2.0 ** -8 * np.abs(ref) + 1e-6
    a = h @ np.asarray(inp.W, np.float64)
    b = h @ np.asarray(inp.W_up, np.float64)
    sig = 1.0 / (1.0 + np.exp(-a))
    dsilu = sig * (1.0 + a * (1.0 - sig))
    Ea, Eb = err(inp.W), err(inp.W_up)
    return np.abs(dsilu) * np.abs(b) * Ea + np.abs(a * sig) * Eb + Ea * Eb + 2.0 ** -8 * np.abs(ref) + 1e-6


def _check(y, ref, bound, what):
    assert y.shape == ref.shape and np.all(np.isfinite(y)), what
    bad = np.abs(y - ref) > bound
    assert not bad.any(), (f"{what}: {bad.sum()} outputs outside the derived bound, worst "
                           f"{np.max(np.abs(y - ref) / bound):.2f}x")
    assert_close(y, ref, "bf16", what) if not what.startswith("sw") else None


def _run(fn, M, K, N, T, swiglu, seed, bad_idx=False):
    inp = W.random_inputs(M, K, N, "bf16", seed=seed, swiglu=swiglu)
    scale, shift, idx = W.adaln_tables(T, K, M, seed=seed + 1)
    if bad_idx and M >= 3:
        idx[0], idx[-1] = -1, T          # outside [0, T): scale 0, shift 0
    x = to_dev(inp.x, "bf16")
    g = to_dev(inp.g, "bf16")
    sc, sh = to_dev(scale, "bf16"), to_dev(shift, "bf16")
    idx_d = _idx_dev(idx)
    Wg = to_dev(inp.W, "bf16")
    Pg, bg = fn.fold_weights(g, Wg), fn.adaln_shift_bias(sh, Wg)
    # the oracle sees an extra all-zero table row for the out-of-range indices
    scale0 = np.vstack([scale, np.zeros((1, K), np.float32)])
    shift0 = np.vstack([shift, np.zeros((1, K), np.float32)])
    idx0 = np.where((idx < 0) | (idx >= T), T, idx)
    if swiglu:
        Wu = to_dev(inp.W_up, "bf16")
        Pu, bu = fn.fold_weights(g, Wu), fn.adaln_shift_bias(sh, Wu)
        y = fn.norm_proj_swiglu_adaln(x, sc, idx_d, Pg, bg, Pu, bu, inp.call.eps)
        ref = oracle.adaln_norm_proj_swiglu(inp.x, inp.g, scale0, shift0, idx0, inp.W, inp.W_up, inp.call.eps)
    else:
        y = fn.norm_proj_adaln(x, sc, idx_d, Pg, bg, inp.call.eps)
        ref = oracle.adaln_norm_proj(inp.x, inp.g, scale0, shift0, idx0, inp.W, inp.call.eps)
    return to_f64(y), ref, _bound(inp, scale0, shift0, idx0, swiglu, ref)


@pytest.mark.parametrize("swiglu", [False, True])
@pytest.mark.parametrize("M,K,N,T", [(1, 8, 16, 1), (3, 40, 37, 2), (9, 4104, 530, 3), (16, 1032, 270, 5),
                                     (17, 256, 48, 2), (40, 1032, 270, 4), (64, 264, 1100, 3), (65, 256, 160, 2),
                                     (130, 520, 33, 3), (300, 1032, 530, 5), (520, 4104, 270, 63),
                                     (257, 264, 1100, 64),
                                     # decode with the largest staged table slice, and tables past it
                                     (33, 1032, 270, 23), (16, 264, 100, 24), (40, 1032, 270, 30), (64, 4104, 530, 40)])
def test_adaln_parity(gpu_lib, swiglu, M, K, N, T):
    y, ref, bound = _run(gpu_lib, M, K, N, T, swiglu, seed=M * 3 + K + N + T)
    _check(y, ref, bound, f"{'swiglu' if swiglu else 'proj'} adaln {M}x{K}x{N} T={T}")


@pytest.mark.parametrize("M", [20, 300])
@pytest.mark.parametrize("swiglu", [False, True])
def test_adaln_out_of_range_index(gpu_lib, swiglu, M):
    y, ref, bound = _run(gpu_lib, M, 264, 100, 3, swiglu, seed=5, bad_idx=True)
    _check(y, ref, bound, f"{'swiglu' if swiglu else 'proj'} adaln with indices outside the table")


def test_adaln_ffn_decode_shape(gpu_lib):
    """The FFN decode shape (64 x 4096 -> 2 x 11008) with four table rows."""
    y, ref, bound = _run(gpu_lib, 64, 4096, 11008, 4, True, seed=11)
    _check(y, ref, bound, "swiglu adaln FFN decode shape")


def test_adaln_zero_tables_match_the_plain_path(gpu_lib):
    """With zero tables the modulated operand is x itself and the bias is 0:
    the AdaLN kernel then gives the plain fused call's output bit for bit
    when both use the same kernel shape (64 rows, LDS-shared x: wide enough,
    257 column blocks, that the plain call takes that kernel too)."""
    import torch
    fn = gpu_lib
    M, K, N = 64, 1032, 4112
    inp = W.random_inputs(M, K, N, "bf16", seed=3, swiglu=True)
    x = to_dev(inp.x, "bf16")
    g = to_dev(inp.g, "bf16")
    Pg = fn.fold_weights(g, to_dev(inp.W, "bf16"))
    Pu = fn.fold_weights(g, to_dev(inp.W_up, "bf16"))
    sc = torch.zeros((2, K), dtype=torch.bfloat16, device="cuda")
    b = torch.zeros((2, N), dtype=torch.float32, device="cuda")
    idx = torch.zeros((M,), dtype=torch.int32, device="cuda")
    y = fn.norm_proj_swiglu_adaln(x, sc, idx, Pg, b, Pu, b, 1e-6)
    want = fn.norm_proj_swiglu(x, Pg, Pu, 1e-6)
    assert fn.kernel_name(M, K, N, True, torch.bfloat16).endswith("m64_xlds_w3_u2")
    assert torch.equal(y.view(torch.int16), want.view(torch.int16))


def test_adaln_kernel_choice(gpu_lib):
    """Up to 64 rows the decode kernel; above, the prefill kernel while the
    table fits its staging (T <= 63), else the decode kernel tiled over rows."""
    fn = gpu_lib
    assert fn.kernel_name_adaln(64, 4096, 11008, 4, True).startswith("decode_swiglu_adaln")
    assert fn.kernel_name_adaln(64, 4096, 11008, 23, True).endswith("_tab")
    assert not fn.kernel_name_adaln(64, 4096, 11008, 24, True).endswith("_tab")
    assert fn.kernel_name_adaln(65, 4096, 11008, 63, True).startswith("prefill_swiglu_adaln")
    assert fn.kernel_name_adaln(4096, 4096, 11008, 64, False).startswith("decode_adaln")


@pytest.mark.parametrize("N,T,swiglu,rows", [(2048, 16, True, 96), (12288, 8, False, 128)])
def test_adaln_prefill_sampled_rows(gpu_lib, N, T, swiglu, rows):
    """4096 rows x 4096 through the prefill kernel (SwiGLU 2 x 2048 columns
    with 16 table rows; the 12288-column QKV projection with 8); the oracle
    on a seeded sample of rows."""
    import torch
    fn = gpu_lib
    M, K = 4096, 4096
    inp = W.random_inputs(M, K, N, "bf16", seed=41, swiglu=swiglu)
    scale, shift, idx = W.adaln_tables(T, K, M, seed=42)
    x, g = to_dev(inp.x, "bf16"), to_dev(inp.g, "bf16")
    sc, sh = to_dev(scale, "bf16"), to_dev(shift, "bf16")
    Wg = to_dev(inp.W, "bf16")
    if swiglu:
        Wu = to_dev(inp.W_up, "bf16")
        y = fn.norm_proj_swiglu_adaln(x, sc, _idx_dev(idx), fn.fold_weights(g, Wg), fn.adaln_shift_bias(sh, Wg),
                                      fn.fold_weights(g, Wu), fn.adaln_shift_bias(sh, Wu), 1e-6)
    else:
        y = fn.norm_proj_adaln(x, sc, _idx_dev(idx), fn.fold_weights(g, Wg), fn.adaln_shift_bias(sh, Wg), 1e-6)
    torch.cuda.synchronize()
    pick = W.sample_indices(M, rows, seed=7)
    sub = W.random_inputs(1, K, N, "bf16", seed=41, swiglu=swiglu)
    sub.x, sub.g, sub.W, sub.W_up = inp.x[pick], inp.g, inp.W, inp.W_up
    if swiglu:
        ref = oracle.adaln_norm_proj_swiglu(sub.x, sub.g, scale, shift, idx[pick], sub.W, sub.W_up, 1e-6)
    else:
        ref = oracle.adaln_norm_proj(sub.x, sub.g, scale, shift, idx[pick], sub.W, 1e-6)
    bound = _bound(sub, scale, shift, idx[pick], swiglu, ref)
    _check(to_f64(y)[pick], ref, bound, f"{'swiglu' if swiglu else 'proj'} adaln prefill rows")


# ---------------------------------------------------------------------------
# Two-launch form: the pre-pass (fn_adaln_modulate) into a caller workspace,
# then the prefill kernel on the modulated operand
# ---------------------------------------------------------------------------
def _bf16_bits(t):
    import torch
    return t.view(torch.int16).cpu().numpy().view(np.uint16)


@pytest.mark.parametrize("M,K,T", [(1, 8, 1), (5, 264, 3), (70, 1032, 5), (301, 4104, 100), (4096, 4096, 4)])
def test_adaln_modulate_matches_oracle(gpu_lib, M, K, T):
    """The pre-pass operand bit for bit (a rounding decides every bit: the
    oracle takes it in the same two steps, fp32 then bf16), and 1/RMS of the
    raw rows within the fp32 bound of its sum."""
    from tests.gpu_helpers import storage_bits
    fn = gpu_lib
    seed = M + K + T
    inp = W.random_inputs(M, K, 16, "bf16", seed=seed)
    scale, _, idx = W.adaln_tables(T, K, M, seed=seed + 1)
    if M >= 3:
        idx[0], idx[-1] = -1, T           # outside the table: scale 0
    u, rs = fn.adaln_modulate(to_dev(inp.x, "bf16"), to_dev(scale, "bf16"), _idx_dev(idx), 1e-6)
    want = oracle.adaln_operand(inp.x, scale, idx)
    got = _bf16_bits(u)
    bad = got != storage_bits(want, "bf16")
    assert not bad.any(), f"{bad.sum()} operand values differ, first at {np.argwhere(bad)[:3].tolist()}"
    ref = 1.0 / oracle.rms(inp.x, 1e-6)
    # each lane sums K/64 squares in order, then six pairwise steps; sqrt and division add a few ulps
    rel = (K / 64 + 16) * 2.0 ** -24 + 4 * 2.0 ** -24
    err = np.abs(to_f64(rs) - ref) / ref
    assert np.all(err <= rel), f"1/RMS off by {err.max():.2e} > {rel:.2e}"


def _run_ws(fn, M, K, N, T, swiglu, seed, bad_idx=False, workspace=None):
    inp = W.random_inputs(M, K, N, "bf16", seed=seed, swiglu=swiglu)
    scale, shift, idx = W.adaln_tables(T, K, M, seed=seed + 1)
    if bad_idx and M >= 3:
        idx[0], idx[-1] = -1, T
    x, g = to_dev(inp.x, "bf16"), to_dev(inp.g, "bf16")
    sc, sh = to_dev(scale, "bf16"), to_dev(shift, "bf16")
    idx_d = _idx_dev(idx)
    Wg = to_dev(inp.W, "bf16")
    Pg, bg = fn.fold_weights(g, Wg), fn.adaln_shift_bias(sh, Wg)
    scale0 = np.vstack([scale, np.zeros((1, K), np.float32)])
    shift0 = np.vstack([shift, np.zeros((1, K), np.float32)])
    idx0 = np.where((idx < 0) | (idx >= T), T, idx)
    if swiglu:
        Wu = to_dev(inp.W_up, "bf16")
        Pu, bu = fn.fold_weights(g, Wu), fn.adaln_shift_bias(sh, Wu)
        y = fn.norm_proj_swiglu_adaln_ws(x, sc, idx_d, Pg, bg, Pu, bu, inp.call.eps, workspace=workspace)
        ref = oracle.adaln_norm_proj_swiglu(inp.x, inp.g, scale0, shift0, idx0, inp.W, inp.W_up, inp.call.eps)
    else:
        y = fn.norm_proj_adaln_ws(x, sc, idx_d, Pg, bg, inp.call.eps, workspace=workspace)
        ref = oracle.adaln_norm_proj(inp.x, inp.g, scale0, shift0, idx0, inp.W, inp.call.eps)
    return to_f64(y), ref, _bound(inp, scale0, shift0, idx0, swiglu, ref)


@pytest.mark.parametrize("swiglu", [False, True])
@pytest.mark.parametrize("M,K,N,T", [
    # 17..64 rows: the decode kernel on the pre-modulated operand
    (17, 1032, 270, 23), (33, 4104, 530, 100), (40, 1032, 270, 4), (64, 264, 1100, 3), (64, 4096, 11008, 4),
    # above: the prefill kernel
    (65, 256, 160, 2), (130, 520, 33, 3), (300, 1032, 530, 5), (257, 264, 1100, 64),
    (520, 4104, 270, 63), (200, 1032, 300, 500), (777, 264, 48, 1)])
def test_adaln_ws_parity(gpu_lib, swiglu, M, K, N, T):
    """Ragged row, column and k tails through the pre-pass and both
    projection kernels, any table size."""
    y, ref, bound = _run_ws(gpu_lib, M, K, N, T, swiglu, seed=M * 5 + K + N + T, bad_idx=True)
    _check(y, ref, bound, f"{'swiglu' if swiglu else 'proj'} adaln two-launch {M}x{K}x{N} T={T}")


def test_adaln_ws_workspace_reuse(gpu_lib):
    """One workspace for two calls in a row, the second with fewer rows
    (its contents from the first call are overwritten, not trusted)."""
    import torch
    fn = gpu_lib
    ws = torch.empty((fn.adaln_workspace_bytes(300, 1032),), dtype=torch.uint8, device="cuda")
    for M in (300, 97):
        y, ref, bound = _run_ws(fn, M, 1032, 270, 7, True, seed=M, workspace=ws)
        _check(y, ref, bound, f"swiglu adaln two-launch, shared workspace, M={M}")


def test_adaln_ws_up_to_16_rows_is_the_one_launch_call(gpu_lib):
    """Up to 16 rows the two-launch entry runs the one-launch kernel: the
    same bits, with no workspace."""
    import torch
    fn = gpu_lib
    M, K, N, T = 16, 1032, 530, 5
    inp = W.random_inputs(M, K, N, "bf16", seed=8, swiglu=True)
    scale, shift, idx = W.adaln_tables(T, K, M, seed=9)
    x, g = to_dev(inp.x, "bf16"), to_dev(inp.g, "bf16")
    sc, sh = to_dev(scale, "bf16"), to_dev(shift, "bf16")
    Wg, Wu = to_dev(inp.W, "bf16"), to_dev(inp.W_up, "bf16")
    Pg, Pu = fn.fold_weights(g, Wg), fn.fold_weights(g, Wu)
    bg, bu = fn.adaln_shift_bias(sh, Wg), fn.adaln_shift_bias(sh, Wu)
    assert fn.adaln_workspace_bytes(M, K) == 0
    a = fn.norm_proj_swiglu_adaln_ws(x, sc, _idx_dev(idx), Pg, bg, Pu, bu, 1e-6)
    b = fn.norm_proj_swiglu_adaln(x, sc, _idx_dev(idx), Pg, bg, Pu, bu, 1e-6)
    assert torch.equal(a.view(torch.int16), b.view(torch.int16))


@pytest.mark.parametrize("N,T,swiglu,rows", [(11008, 16, True, 64), (12288, 4, False, 96)])
def test_adaln_ws_prefill_sampled_rows(gpu_lib, N, T, swiglu, rows):
    """The full prefill shapes through the two-launch form (FFN 4096 x 4096
    -> 2 x 11008 with 16 table rows; QKV 4096 x 4096 -> 12288 with 4), the
    oracle on a seeded sample of rows."""
    import torch
    fn = gpu_lib
    M, K = 4096, 4096
    inp = W.random_inputs(M, K, N, "bf16", seed=43, swiglu=swiglu)
    scale, shift, idx = W.adaln_tables(T, K, M, seed=44)
    x, g = to_dev(inp.x, "bf16"), to_dev(inp.g, "bf16")
    sc, sh = to_dev(scale, "bf16"), to_dev(shift, "bf16")
    Wg = to_dev(inp.W, "bf16")
    if swiglu:
        Wu = to_dev(inp.W_up, "bf16")
        y = fn.norm_proj_swiglu_adaln_ws(x, sc, _idx_dev(idx), fn.fold_weights(g, Wg), fn.adaln_shift_bias(sh, Wg),
                                         fn.fold_weights(g, Wu), fn.adaln_shift_bias(sh, Wu), 1e-6)
    else:
        y = fn.norm_proj_adaln_ws(x, sc, _idx_dev(idx), fn.fold_weights(g, Wg), fn.adaln_shift_bias(sh, Wg), 1e-6)
    torch.cuda.synchronize()
    pick = W.sample_indices(M, rows, seed=8)
    sub = W.random_inputs(1, K, N, "bf16", seed=43, swiglu=swiglu)
    sub.x, sub.g, sub.W, sub.W_up = inp.x[pick], inp.g, inp.W, inp.W_up
    if swiglu:
        ref = oracle.adaln_norm_proj_swiglu(sub.x, sub.g, scale, shift, idx[pick], sub.W, sub.W_up, 1e-6)
    else:
        ref = oracle.adaln_norm_proj(sub.x, sub.g, scale, shift, idx[pick], sub.W, 1e-6)
    bound = _bound(sub, scale, shift, idx[pick], swiglu, ref)
    _check(to_f64(y)[pick], ref, bound, f"{'swiglu' if swiglu else 'proj'} adaln two-launch prefill rows")
