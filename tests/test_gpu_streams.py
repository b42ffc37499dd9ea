"""Stream and graph behaviour of the two-launch AdaLN calls: calls on two
streams at once, each with its own workspace, and the calls captured into a
HIP graph (preallocated output and workspace: nothing is allocated inside a
call) replayed several times with unrelated eager work in between.  Every
result must equal the eager single-stream result bit for bit."""
import pytest

pytestmark = pytest.mark.gpu


def _case(fn, M, K, N, T, seed):
    import torch
    gen = torch.Generator(device="cuda")
    gen.manual_seed(seed)
    x = torch.randn((M, K), generator=gen, device="cuda").to(torch.bfloat16)
    g = (torch.rand((K,), generator=gen, device="cuda") + 0.5).to(torch.bfloat16)
    W = (torch.randn((K, N), generator=gen, device="cuda") / 64).to(torch.bfloat16)
    sc = (torch.randn((T, K), generator=gen, device="cuda") * 0.3).to(torch.bfloat16)
    sh = (torch.randn((T, K), generator=gen, device="cuda") * 0.3).to(torch.bfloat16)
    idx = torch.randint(0, T, (M,), generator=gen, device="cuda", dtype=torch.int32)
    return x, fn.adaln_fold_table(g, sc), idx, fn.fold_weights(None, W), fn.adaln_shift_bias(sh, W)


def test_two_streams_separate_workspaces(gpu_lib):
    import torch
    fn = gpu_lib
    cases = [_case(fn, 300, 1032, 2048, 5, 1), _case(fn, 4096, 1024, 1024, 3, 2)]
    want = [fn.norm_proj_adaln_ws(*c, 1e-6) for c in cases]
    torch.cuda.synchronize()
    streams = [torch.cuda.Stream(), torch.cuda.Stream()]
    outs = [torch.empty_like(w) for w in want]
    wss = [torch.empty((fn.adaln_workspace_bytes(c[0].shape[0], c[0].shape[1]),), dtype=torch.uint8, device="cuda")
           for c in cases]
    torch.cuda.synchronize()
    for rep in range(3):
        for s, c, o, ws in zip(streams, cases, outs, wss):
            with torch.cuda.stream(s):
                fn.norm_proj_adaln_ws(*c, 1e-6, out=o, workspace=ws)
        torch.cuda.synchronize()
        for o, w in zip(outs, want):
            assert torch.equal(o.view(torch.int16), w.view(torch.int16)), f"repeat {rep}"


@pytest.mark.parametrize("M", [48, 1000])
def test_graph_capture_and_replay(gpu_lib, M):
    import torch
    fn = gpu_lib
    x, sc, idx, Pw, bias = _case(fn, M, 1032, 1100, 4, 3)
    want = fn.norm_proj_adaln_ws(x, sc, idx, Pw, bias, 1e-6)
    out = torch.empty_like(want)
    ws = torch.empty((fn.adaln_workspace_bytes(M, 1032),), dtype=torch.uint8, device="cuda")
    torch.cuda.synchronize()
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        fn.norm_proj_adaln_ws(x, sc, idx, Pw, bias, 1e-6, out=out, workspace=ws)
    busy = torch.empty((1 << 20,), device="cuda")
    for rep in range(4):
        out.fill_(float("nan"))
        busy.normal_()                          # unrelated eager work between replays
        graph.replay()
        torch.cuda.synchronize()
        assert torch.equal(out.view(torch.int16), want.view(torch.int16)), f"replay {rep}"
