"""GPU parity: the HIP path (through the C ABI) against the float64 oracle on
the same seeded inputs.  Tolerance per element: |gpu - oracle| <=
2e-2 * (|oracle| + 1) for bf16 storage with fp32 accumulation, 1e-5 * (|oracle| + 1)
for fp32; bit-exact for the fold and for invariants that the kernel's fixed
accumulation order preserves exactly."""
import numpy as np
import pytest

import oracle
import workloads as W
from tests import oracle_pins
from tests.gpu_helpers import TOL, assert_close, pack_host, stale_failures, to_dev, to_f64, tdtype

pytestmark = pytest.mark.gpu


def fused(fn, inp: W.Inputs, eps=None):
    """Fold on the device, then one fused call; returns (y float64, gpu tensors)."""
    c = inp.call
    eps = c.eps if eps is None else eps
    x = to_dev(inp.x, c.dtype)
    g = to_dev(inp.g, c.dtype)
    Wg = fn.fold_weights(g, to_dev(inp.W, c.dtype))
    if c.swiglu:
        Wu = fn.fold_weights(g, to_dev(inp.W_up, c.dtype))
        y = fn.norm_proj_swiglu(x, Wg, Wu, eps)
    else:
        y = fn.norm_proj(x, Wg, eps)
    return to_f64(y)


def reference(inp: W.Inputs, rows=None, cols=None, eps=None):
    c = inp.call
    eps = c.eps if eps is None else eps
    x = inp.x if rows is None else inp.x[rows]
    Wm = inp.W if cols is None else inp.W[:, cols]
    if c.swiglu:
        Wu = inp.W_up if cols is None else inp.W_up[:, cols]
        return oracle.norm_proj_swiglu(x, inp.g, Wm, Wu, eps)
    return oracle.norm_proj(x, inp.g, Wm, eps)


# ---------------------------------------------------------------- fold ----
@pytest.mark.parametrize("dtype", ["bf16", "f32"])
@pytest.mark.parametrize("K,N", [(8, 1), (40, 37), (256, 768), (4096, 1000)])
def test_fold_bit_exact(gpu_lib, dtype, K, N):
    inp = W.random_inputs(1, K, N, dtype, seed=100 + K + N)
    ref = oracle.fold_weights(inp.g, inp.W, dtype)
    Wp = gpu_lib.fold_weights(to_dev(inp.g, dtype), to_dev(inp.W, dtype))
    got = Wp.data.cpu().numpy()
    want = pack_host(ref, dtype)
    assert got.shape == want.shape
    assert np.array_equal(got, want), f"fold differs in {np.count_nonzero(got != want)} bytes"
    # g omitted: the weights are packed unchanged
    Wp1 = gpu_lib.fold_weights(None, to_dev(inp.W, dtype))
    assert np.array_equal(Wp1.data.cpu().numpy(), pack_host(inp.W, dtype))


# ----------------------------- rows just past decode, wide projections ----
@pytest.mark.parametrize("M,K,N,swiglu", [(65, 264, 8200, False), (100, 1032, 8192, True), (128, 136, 8208, False),
                                          (97, 4104, 8200, True), (128, 4096, 12288, False)])
def test_rows_tiled_decode_parity(gpu_lib, M, K, N, swiglu):
    """65..128 rows of a projection with at least 512 column blocks run the
    128-row rung of the LDS-shared-x decode kernel (ragged rows, K and N):
    every output against the oracle."""
    inp = W.random_inputs(M, K, N, "bf16", seed=M + K + N + swiglu, swiglu=swiglu)
    import torch
    assert gpu_lib.kernel_name(M, K, N, swiglu, torch.bfloat16).startswith("decode")
    assert_close(fused(gpu_lib, inp), reference(inp), "bf16", f"rows tiled {M}x{K}x{N} swiglu={swiglu}")


@pytest.mark.parametrize("M,K,N,swiglu", [(96, 264, 1540, False), (300, 136, 3000, False), (200, 72, 8000, False),
                                          (128, 264, 1380, True), (129, 136, 1380, True), (512, 72, 2750, True)])
def test_narrow_rows_tiled_parity(gpu_lib, M, K, N, swiglu):
    """Past 64 rows of a narrow projection (fewer than 512 column blocks: one
    GPU's share under tensor parallelism) the decode kernels' 64-row blocks
    repeat over the rows -- the LDS-shared-x kernel, or for a SwiGLU pair
    whose row blocks give at most 256 workgroups the register-x kernel with
    a k-split (ragged rows, K and N): every output against the oracle."""
    import torch
    assert gpu_lib.kernel_name(M, K, N, swiglu, torch.bfloat16).startswith("decode")
    inp = W.random_inputs(M, K, N, "bf16", seed=7 * M + K + N + swiglu, swiglu=swiglu)
    assert_close(fused(gpu_lib, inp), reference(inp), "bf16", f"narrow rows tiled {M}x{K}x{N} swiglu={swiglu}")


@pytest.mark.parametrize("M,K,N,swiglu", [(16, 136, 24587, False), (1, 264, 32000, False), (11, 136, 24600, True),
                                          (16, 72, 25000, True)])
def test_two_block_decode_parity(gpu_lib, M, K, N, swiglu):
    """Up to 16 rows of a projection with at least 1536 column blocks run
    the register-x decode kernel with two column blocks per wave (an odd
    block count leaves the last wave one block; ragged K and N): every
    output against the oracle."""
    import torch
    assert "_n32_" in gpu_lib.kernel_name(M, K, N, swiglu, torch.bfloat16)
    inp = W.random_inputs(M, K, N, "bf16", seed=5 * M + K + N + swiglu, swiglu=swiglu)
    assert_close(fused(gpu_lib, inp), reference(inp), "bf16", f"two-block decode {M}x{K}x{N} swiglu={swiglu}")


@pytest.mark.parametrize("M,K,N,swiglu", [(129, 264, 8200, False), (200, 1032, 8192, True), (256, 4096, 12288, False),
                                          (161, 136, 8208, True)])
def test_prefill_128_row_tiles_parity(gpu_lib, M, K, N, swiglu):
    """129..256 rows of a wide projection take the prefill kernel's 128-row
    tiles (ragged rows, K and N): every output against the oracle."""
    import torch
    assert "128x128" in gpu_lib.kernel_name(M, K, N, swiglu, torch.bfloat16)
    inp = W.random_inputs(M, K, N, "bf16", seed=3 * M + K + N + swiglu, swiglu=swiglu)
    assert_close(fused(gpu_lib, inp), reference(inp), "bf16", f"128-row tiles {M}x{K}x{N} swiglu={swiglu}")


# ------------------------------------------------------ hand-derived case --
@pytest.mark.parametrize("dtype", ["bf16", "f32"])
def test_hand_case_exact(gpu_lib, dtype):
    case = [c for c in oracle_pins.load_golden()["cases"] if c["name"] == "bf16_exact_k8"][0]
    x = np.asarray(case["x"], np.float32)
    g = np.asarray(case["g"], np.float32)
    Wm = oracle_pins._case_W(case).astype(np.float32)
    Wp = gpu_lib.fold_weights(to_dev(g, dtype), to_dev(Wm, dtype))
    y = to_f64(gpu_lib.norm_proj(to_dev(x, dtype), Wp, 0.0))
    assert np.array_equal(y, np.asarray(case["y"], np.float64))


# ------------------------------------------------------ workload configs --
def test_tiny_f32(gpu_lib):
    inp = W.make_inputs(W.TINY)
    assert_close(fused(gpu_lib, inp), reference(inp), "f32", "tiny")


def test_qkv_decode_full(gpu_lib):
    inp = W.make_inputs(W.QKV_DECODE)
    assert_close(fused(gpu_lib, inp), reference(inp), "bf16", "qkv decode")


def test_ffn_decode_swiglu_full(gpu_lib):
    inp = W.make_inputs(W.FFN_DECODE)
    assert_close(fused(gpu_lib, inp), reference(inp), "bf16", "ffn swiglu decode")


def test_prefill_qkv_full(gpu_lib):
    """The prefill QKV workload (4096 x 4096 -> 12288), every output."""
    inp = W.make_inputs(W.PREFILL_QKV)
    err = assert_close(fused(gpu_lib, inp), reference(inp), "bf16", "prefill qkv")
    print(f"prefill qkv: max |err|/(|ref|+1) = {err:.2e}")


def test_prefill_ffn_swiglu_full(gpu_lib):
    """The FFN gate/up SwiGLU prefill (4096 x 4096 -> 2 x 11008), every
    output."""
    inp = W.random_inputs(4096, 4096, 11008, "bf16", seed=5, swiglu=True)
    err = assert_close(fused(gpu_lib, inp), reference(inp), "bf16", "prefill ffn swiglu")
    print(f"prefill ffn swiglu: max |err|/(|ref|+1) = {err:.2e}")


@pytest.mark.parametrize("index", [0, 1, 30, 31, 62, 63, 64])
def test_decode_step_calls(gpu_lib, index):
    call = W.decode_step_calls()[index]
    inp = W.make_inputs(call)
    assert_close(fused(gpu_lib, inp), reference(inp), "bf16", call.name)


# ---------------------------------------------------- ragged and edges ---
RAGGED = [(1, 8, 16), (3, 40, 37), (17, 256, 48), (16, 64, 200), (24, 8, 1), (32, 1032, 270),
          (33, 96, 100), (40, 1032, 270), (48, 520, 33), (61, 4104, 530), (63, 128, 17),
          (64, 72, 64), (65, 256, 160), (100, 40, 33), (130, 512, 260), (257, 64, 31),
          (300, 136, 530), (513, 1032, 270), (777, 264, 1100)]


@pytest.mark.parametrize("dtype", ["bf16", "f32"])
@pytest.mark.parametrize("swiglu", [False, True])
@pytest.mark.parametrize("M,K,N", RAGGED)
def test_ragged(gpu_lib, dtype, swiglu, M, K, N):
    inp = W.random_inputs(M, K, N, dtype, seed=M * 7 + K * 3 + N + int(swiglu), swiglu=swiglu)
    assert_close(fused(gpu_lib, inp), reference(inp), dtype, f"ragged {M}x{K}x{N}")


@pytest.mark.parametrize("eps", [0.0, 1e-6, 0.5])
def test_eps_values(gpu_lib, eps):
    inp = W.random_inputs(5, 64, 48, "f32", seed=7)
    assert_close(fused(gpu_lib, inp, eps), reference(inp, eps=eps), "f32", f"eps={eps}")


def test_empty_calls(gpu_lib):
    import torch
    Wp = gpu_lib.fold_weights(None, torch.zeros((64, 32), dtype=torch.bfloat16, device="cuda"))
    y = gpu_lib.norm_proj(torch.zeros((0, 64), dtype=torch.bfloat16, device="cuda"), Wp)
    assert tuple(y.shape) == (0, 32)
    Wz = gpu_lib.fold_weights(None, torch.zeros((64, 0), dtype=torch.bfloat16, device="cuda"))
    y = gpu_lib.norm_proj(torch.ones((3, 64), dtype=torch.bfloat16, device="cuda"), Wz)
    assert tuple(y.shape) == (3, 0)


def test_zero_row_with_eps(gpu_lib):
    inp = W.random_inputs(4, 64, 32, "bf16", seed=9)
    inp.x[2] = 0.0
    y = fused(gpu_lib, inp, 1e-6)
    assert np.all(y[2] == 0.0)
    assert_close(y, reference(inp, eps=1e-6), "bf16", "zero row")


def test_nan_row_isolated(gpu_lib):
    inp = W.random_inputs(20, 128, 64, "bf16", seed=10)
    inp.x[5, 17] = np.nan
    c = inp.call
    x = to_dev(inp.x, c.dtype)
    Wp = gpu_lib.fold_weights(to_dev(inp.g, c.dtype), to_dev(inp.W, c.dtype))
    y = to_f64(gpu_lib.norm_proj(x, Wp, c.eps))
    assert np.all(np.isnan(y[5]))
    ref = reference(inp)
    keep = [i for i in range(20) if i != 5]
    assert_close(y[keep], ref[keep], "bf16", "rows beside a NaN row")


@pytest.mark.parametrize("dtype,M,swiglu", [("bf16", 3, False), ("bf16", 40, True), ("bf16", 100, False),
                                             ("bf16", 130, True), ("f32", 6, True)])
def test_zero_row_eps0_and_inf_row_follow_the_formula(gpu_lib, dtype, M, swiglu):
    """eps = 0 on an all-zero row: 1/RMS is 1/0 and the row's products are 0,
    so every output of the row is NaN, as the formula (0/0) gives; an Inf in a
    row makes that row's sum of squares Inf and its outputs NaN (Inf/Inf).
    Every other row matches the oracle -- in each kernel family (register-x
    decode, LDS-shared-x decode, prefill; SwiGLU and plain)."""
    inp = W.random_inputs(M, 264, 70, dtype, seed=M + 31, swiglu=swiglu)
    inp.x[1] = 0.0
    inp.x[M - 1, 13] = np.inf
    with np.errstate(invalid="ignore", divide="ignore"):
        ref = reference(inp, eps=0.0)
    assert np.all(np.isnan(ref[1])) and np.all(np.isnan(ref[M - 1]))
    y = fused(gpu_lib, inp, 0.0)
    assert np.all(np.isnan(y[1])), "zero row at eps = 0"
    assert np.all(np.isnan(y[M - 1])), "row holding an Inf"
    keep = [i for i in range(M) if i not in (1, M - 1)]
    assert_close(y[keep], ref[keep], dtype, f"rows beside them, {dtype} M={M}")


# ----------------------------------------------------------- invariants --
def _fold_and_run(fn, x_np, g_np, W_np, dtype, eps):
    Wp = fn.fold_weights(to_dev(g_np, dtype), to_dev(W_np, dtype))
    return to_f64(fn.norm_proj(to_dev(x_np, dtype), Wp, eps))


@pytest.mark.parametrize("p", [-3, 5])
def test_scale_invariance_bit_exact(gpu_lib, p):
    """RMSNorm(2^p x) = RMSNorm(x) at eps=0: the kernel scales every partial
    sum by a power of two, so the outputs agree bit for bit."""
    inp = W.random_inputs(16, 512, 96, "bf16", seed=12)
    base = _fold_and_run(gpu_lib, inp.x, inp.g, inp.W, "bf16", 0.0)
    scaled = _fold_and_run(gpu_lib, inp.x * np.float32(2.0 ** p), inp.g, inp.W, "bf16", 0.0)
    assert np.array_equal(base, scaled)


def test_row_permutation_bit_exact(gpu_lib):
    inp = W.random_inputs(48, 256, 80, "bf16", seed=13)
    perm = np.random.default_rng(1).permutation(48)
    base = _fold_and_run(gpu_lib, inp.x, inp.g, inp.W, "bf16", 1e-6)
    permd = _fold_and_run(gpu_lib, inp.x[perm], inp.g, inp.W, "bf16", 1e-6)
    assert np.array_equal(permd, base[perm])


def test_column_concatenation_bit_exact(gpu_lib):
    """Columns are independent: splitting W' by columns splits y, bit for bit
    (the split sits at 1536 columns, a multiple of every workgroup width, and
    all three widths take the same k-split: at most 256 column blocks)."""
    inp = W.random_inputs(8, 256, 1632, "bf16", seed=14)
    full = _fold_and_run(gpu_lib, inp.x, inp.g, inp.W, "bf16", 1e-6)
    left = _fold_and_run(gpu_lib, inp.x, inp.g, np.ascontiguousarray(inp.W[:, :1536]), "bf16", 1e-6)
    right = _fold_and_run(gpu_lib, inp.x, inp.g, np.ascontiguousarray(inp.W[:, 1536:]), "bf16", 1e-6)
    assert np.array_equal(full, np.concatenate([left, right], axis=1))
    assert_close(full, oracle.norm_proj(inp.x, inp.g, inp.W, 1e-6), "bf16", "concat")


def test_rne_store(gpu_lib):
    """Outputs that are exact fp32 ties round to even in bf16: x = ones(8)
    gives r = 1 and y[n] = sum_k W[k, n] exactly in fp32."""
    K = 8
    cols = [[1.0, 2.0 ** -8], [1.0, 2.0 ** -7, 2.0 ** -8], [-1.0, -2.0 ** -8],
            [255.0, 0.5], [1.0, 2.0 ** -8, 2.0 ** -20], [3.0, 2.0 ** -7]]
    Wm = np.zeros((K, 16), np.float32)
    for n, vals in enumerate(cols):
        Wm[:len(vals), n] = vals
    x = np.ones((1, K), np.float32)
    y = _fold_and_run(gpu_lib, x, np.ones(K, np.float32), Wm, "bf16", 0.0)
    want = oracle.round_to_bf16(Wm.astype(np.float64).sum(axis=0))
    assert np.array_equal(y[0], want)


# ------------------------------------------------------ staleness (T5) --
def test_back_to_back_calls_not_stale(gpu_lib):
    """256 consecutive calls with distinct x into one reused, NaN-poisoned y:
    every output must match its own input's oracle and not the previous
    call's."""
    import torch
    M, K, N, T = 16, 1024, 512, 256
    base = W.random_inputs(M, K, N, "bf16", seed=15)
    Wp = gpu_lib.fold_weights(to_dev(base.g, "bf16"), to_dev(base.W, "bf16"))
    y = torch.full((M, N), float("nan"), dtype=torch.bfloat16, device="cuda")
    xs = [W.make_x(M, K, "bf16", seed=1000 + t) for t in range(T)]
    xd = [to_dev(x, "bf16") for x in xs]
    outs = []
    for t in range(T):
        gpu_lib.norm_proj(xd[t], Wp, 1e-6, out=y)
        outs.append(y.clone())
    torch.cuda.synchronize()
    refs = [oracle.norm_proj(xs[t], base.g, base.W, 1e-6) for t in range(T)]
    bad = stale_failures([to_f64(o) for o in outs], refs)
    assert not bad, bad[:5]


def test_two_stream_chain_with_its_event_join_passes_the_check(gpu_lib):
    """The pages' two-stream form of the deferred norm ([FlashNorm digest],
    the bug / cause / fix bullets) in plain torch -- the product x @ W' on one
    stream behind unrelated work, the sums of squares and the post-scale on
    another that waits on the product's event (the fix) -- passes the
    staleness check.  That the check flags the unjoined form's one-step-stale
    outputs is shown on the CPU (tests/test_staleness_check.py): whether
    two streams actually overlap depends on how they map to hardware queues,
    so a GPU race is no dependable negative control."""
    import torch
    M, K, N, T = 16, 1024, 512, 8
    base = W.random_inputs(M, K, N, "bf16", seed=15)
    Wf = torch.from_numpy(oracle.fold_weights(base.g, base.W, "bf16").astype(np.float32)).cuda()
    xs = [W.make_x(M, K, "bf16", seed=2000 + t) for t in range(T)]
    xd = [torch.from_numpy(x).cuda() for x in xs]
    s_mm, s_post = torch.cuda.Stream(), torch.cuda.Stream()
    busy_a = torch.randn((2048, 2048), device="cuda")
    h = torch.full((M, N), float("nan"), device="cuda")
    outs = []
    torch.cuda.synchronize()
    for t in range(T):
        done = torch.cuda.Event()
        with torch.cuda.stream(s_mm):
            for _ in range(20):                  # unrelated work ahead of the product
                busy_a = busy_a @ busy_a * 1e-3
            torch.matmul(xd[t], Wf, out=h)
            done.record()
        with torch.cuda.stream(s_post):
            inv = torch.rsqrt(xd[t].pow(2).mean(dim=1, keepdim=True) + 1e-6)
            s_post.wait_event(done)
            y = (h * inv).to(torch.bfloat16)
        torch.cuda.synchronize()
        outs.append(y.to(torch.float64).cpu().numpy())
    refs = [oracle.norm_proj(xs[t], base.g, base.W, 1e-6) for t in range(T)]
    bad = stale_failures(outs, refs)
    assert not bad, bad[:5]


# ------------------------------------------------------ unfused chain ---
@pytest.mark.parametrize("dtype", ["bf16", "f32"])
def test_chain_rmsnorm(gpu_lib, dtype):
    inp = W.random_inputs(9, 264, 8, dtype, seed=16)
    xhat = to_f64(gpu_lib.rmsnorm(to_dev(inp.x, dtype), to_dev(inp.g, dtype), 1e-6))
    assert_close(xhat, oracle.rmsnorm(inp.x, inp.g, 1e-6), dtype, "rmsnorm")


@pytest.mark.parametrize("dtype", ["bf16", "f32"])
def test_chain_silu_mul(gpu_lib, dtype):
    rng = np.random.default_rng(17)
    h = rng.standard_normal((7, 2 * 45)).astype(np.float32)
    hd = to_dev(h, dtype)
    hs = to_f64(hd)
    out = to_f64(gpu_lib.silu_mul(hd))
    assert_close(out, oracle.silu(hs[:, :45]) * hs[:, 45:], dtype, "silu_mul")


def test_python_binding_rejects_bad_arguments(gpu_lib):
    import torch
    Wp = gpu_lib.fold_weights(None, torch.zeros((64, 32), dtype=torch.bfloat16, device="cuda"))
    with pytest.raises(ValueError):
        gpu_lib.norm_proj(torch.zeros((4, 32), dtype=torch.bfloat16, device="cuda"), Wp)
    with pytest.raises(ValueError):
        gpu_lib.norm_proj(torch.zeros((4, 64), dtype=torch.float32, device="cuda"), Wp)
    with pytest.raises(gpu_lib.FlashNormError):
        gpu_lib.norm_proj(torch.zeros((4, 64), dtype=torch.bfloat16, device="cuda"), Wp, eps=-1.0)
    assert tdtype("bf16") == torch.bfloat16


@pytest.mark.parametrize("M,K,N,swiglu", [(2048, 264, 768, False), (1792, 136, 1024, True), (1024, 72, 1024, False),
                                          (4096, 40, 500, True)])
def test_prefill_tile_order(gpu_lib, M, K, N, swiglu):
    """Tile counts that divide by 8 take the XCD-grouped tile order (groups of
    6 row tiles, here with a partial last group): every output against the
    oracle, so a tile computed twice or not at all would show.  The oracle
    takes the folded bf16 weights the kernel reads (the fold's rounding is
    not what this checks; the unfolded comparison is the other tests')."""
    import torch
    assert gpu_lib.kernel_name(M, K, N, swiglu, torch.bfloat16).startswith("prefill")
    inp = W.random_inputs(M, K, N, "bf16", seed=M + K + N, swiglu=swiglu)
    y = fused(gpu_lib, inp)
    assert np.all(np.isfinite(y))
    Wg = oracle.fold_weights(inp.g, inp.W, "bf16")
    if swiglu:
        ref = oracle.norm_proj_swiglu_folded(inp.x, Wg, oracle.fold_weights(inp.g, inp.W_up, "bf16"), inp.call.eps)
    else:
        ref = oracle.norm_proj_folded(inp.x, Wg, inp.call.eps)
    assert_close(y, ref, "bf16", f"prefill tile order {M}x{K}x{N} swiglu={swiglu}")


@pytest.mark.parametrize("M,K,N,swiglu", [(4000, 4104, 4100, False), (4100, 4104, 4200, False),
                                          (2560, 4104, 6600, False)])
def test_prefill_w_direct_ragged(gpu_lib, M, K, N, swiglu):
    """Plain projections over at least 256 tiles with K >= 4096 take the
    instance that loads W' fragments straight into registers (rotated
    row-fragment order per wave): ragged
    rows, columns and k (a partial k-block, a k-block count that is not a
    multiple of the unroll), tile counts with and without the XCD-grouped
    order; every output against the oracle on the folded weights."""
    import torch
    assert gpu_lib.kernel_name(M, K, N, swiglu, torch.bfloat16).endswith("_wd")
    inp = W.random_inputs(M, K, N, "bf16", seed=7 * M + K + N, swiglu=swiglu)
    y = fused(gpu_lib, inp)
    assert np.all(np.isfinite(y))
    Wg = oracle.fold_weights(inp.g, inp.W, "bf16")
    if swiglu:
        ref = oracle.norm_proj_swiglu_folded(inp.x, Wg, oracle.fold_weights(inp.g, inp.W_up, "bf16"), inp.call.eps)
    else:
        ref = oracle.norm_proj_folded(inp.x, Wg, inp.call.eps)
    assert_close(y, ref, "bf16", f"prefill W' direct {M}x{K}x{N} swiglu={swiglu}")
