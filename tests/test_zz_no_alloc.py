"""The SwiGLU AdaLN entry point that allocates nothing
(fn_norm_proj_swiglu_adaln_static: the library's own device scratch as the
workspace) against the workspace entry point it varies
(fn_norm_proj_swiglu_adaln_ws), through the C ABI: two calls in a row, the
second with fewer rows, bit for bit; and a size past the scratch rejected
before any HIP call."""
import pytest

from tests.gpu_helpers import AdalnCase

pytestmark = pytest.mark.gpu


def _bits(t):
    import torch
    return t.view(torch.int16)


def test_static_scratch_matches_the_workspace_call(gpu_lib):
    import torch
    fn = gpu_lib
    for M, K, N, T in ((300, 1032, 530, 7), (97, 1032, 270, 3), (64, 4096, 11008, 4), (20, 264, 100, 2)):
        c = AdalnCase(fn, M, K, N, T, True, seed=M + K, bad_idx=True)
        want = fn.norm_proj_swiglu_adaln_ws(c.x, *c.args(), c.eps)
        out = torch.full((M, N), float("nan"), dtype=torch.bfloat16, device="cuda")
        got = fn.norm_proj_swiglu_adaln_static(c.x, *c.args(), c.eps, out=out)
        torch.cuda.synchronize()
        assert got.data_ptr() == out.data_ptr()
        assert torch.equal(_bits(got), _bits(want)), f"M={M}: {int((_bits(got) != _bits(want)).sum())} differ"


def test_static_scratch_rejects_sizes_past_it(gpu_lib):
    import torch
    fn = gpu_lib
    cap = fn.adaln_static_max_bytes()
    assert cap == (64 << 20) + (64 << 10)
    M, K, N, T = 4200, 4096, 16, 1          # 2 * M * K * 2 bytes > 64 MiB + 64 KiB
    assert fn.adaln_workspace_bytes(M, K) > cap
    x = torch.zeros((M, K), dtype=torch.bfloat16, device="cuda")
    mod = torch.zeros((T, K), dtype=torch.float32, device="cuda")
    idx = torch.zeros((M,), dtype=torch.int32, device="cuda")
    W = fn.fold_weights(None, torch.zeros((K, N), dtype=torch.bfloat16, device="cuda"))
    b = torch.zeros((T, N), dtype=torch.float32, device="cuda")
    with pytest.raises(fn.FlashNormError, match="static scratch"):
        fn.norm_proj_swiglu_adaln_static(x, mod, idx, W, b, W, b, 1e-6)
    # the largest square size that fits still runs
    M = 4096
    assert fn.adaln_workspace_bytes(M, K) <= cap
