"""Recorded steps (fn_step_create / fn_step_launch): a sequence of fused
calls replayed with one HIP graph launch gives bit for bit what the same
calls give launched one by one, on every replay, with inputs refreshed in
place between replays; calls run in order, so a later call reads an earlier
call's output; and the replay agrees with the float64 oracle."""
import numpy as np
import pytest

import oracle
import workloads as W
from tests.gpu_helpers import assert_close, to_dev, to_f64

pytestmark = pytest.mark.gpu


def _mixed(fn, torch):
    """Calls of every kind, ragged shapes, an empty call and a chained pair."""
    specs = []
    dev = "cuda"

    def bf16(M, K, N, seed, swiglu=False, dtype="bf16"):
        inp = W.random_inputs(M, K, N, dtype, seed=seed, swiglu=swiglu)
        x = to_dev(inp.x, dtype)
        Pg = fn.fold_weights(to_dev(inp.g, dtype), to_dev(inp.W, dtype))
        Pu = fn.fold_weights(to_dev(inp.g, dtype), to_dev(inp.W_up, dtype)) if swiglu else None
        return inp, x, Pg, Pu

    def fp8(M, K, N, seed, swiglu=False):
        inp = W.random_inputs(M, K, N, "bf16", seed=seed, swiglu=swiglu)
        x = to_dev(inp.x, "bf16")
        Pg = fn.fold_weights_fp8(to_dev(inp.g, "bf16"), to_dev(inp.W, "bf16"))
        Pu = fn.fold_weights_fp8(to_dev(inp.g, "bf16"), to_dev(inp.W_up, "bf16")) if swiglu else None
        return inp, x, Pg, Pu

    inp, x, Pg, _ = bf16(8, 256, 520, 11)
    specs.append(("proj", x, Pg, None, torch.empty((8, 520), dtype=torch.bfloat16, device=dev)))
    chained_in = specs[-1][4]                       # [8, 520] bf16 feeds the next call as x
    _, _, Pc, _ = bf16(8, 520, 136, 12)
    specs.append(("proj", chained_in, Pc, None, torch.empty((8, 136), dtype=torch.bfloat16, device=dev)))
    inp, x, Pg, Pu = bf16(40, 1032, 270, 13, swiglu=True)
    specs.append(("swiglu", x, Pg, Pu, torch.empty((40, 270), dtype=torch.bfloat16, device=dev)))
    inp, x, Pg, _ = bf16(4, 256, 768, 14, dtype="f32")
    specs.append(("proj", x, Pg, None, torch.empty((4, 768), dtype=torch.float32, device=dev)))
    inp, x, Pg, _ = bf16(0, 64, 32, 15)
    specs.append(("proj", x, Pg, None, torch.empty((0, 32), dtype=torch.bfloat16, device=dev)))
    inp, x, Pg, _ = fp8(13, 1032, 270, 16)
    specs.append(("proj8", x, Pg, None, torch.empty((13, 270), dtype=torch.bfloat16, device=dev)))
    inp, x, Pg, Pu = fp8(64, 4104, 530, 17, swiglu=True)
    specs.append(("swiglu8", x, Pg, Pu, torch.empty((64, 530), dtype=torch.bfloat16, device=dev)))
    inp, x, Pg, _ = bf16(130, 520, 33, 18)
    specs.append(("proj", x, Pg, None, torch.empty((130, 33), dtype=torch.bfloat16, device=dev)))
    return specs


def _eager(fn, kind, x, Pg, Pu, eps=1e-6):
    return {"proj": lambda: fn.norm_proj(x, Pg, eps), "swiglu": lambda: fn.norm_proj_swiglu(x, Pg, Pu, eps),
            "proj8": lambda: fn.norm_proj_fp8(x, Pg, eps),
            "swiglu8": lambda: fn.norm_proj_swiglu_fp8(x, Pg, Pu, eps)}[kind]()


def _record(fn, specs, eps=1e-6):
    st = fn.Step()
    for kind, x, Pg, Pu, out in specs:
        {"proj": lambda: st.norm_proj(x, Pg, out, eps), "swiglu": lambda: st.norm_proj_swiglu(x, Pg, Pu, out, eps),
         "proj8": lambda: st.norm_proj_fp8(x, Pg, out, eps),
         "swiglu8": lambda: st.norm_proj_swiglu_fp8(x, Pg, Pu, out, eps)}[kind]()
    return st.record()


def test_step_replays_match_eager_bit_for_bit(gpu_lib):
    import torch
    fn = gpu_lib
    specs = _mixed(fn, torch)
    st = _record(fn, specs)
    assert st.num_kernels == len(specs) - 1          # the empty call records nothing
    gen = torch.Generator(device="cuda")
    for replay in range(4):
        if replay:
            gen.manual_seed(100 + replay)             # refresh every x in place (the chained one is an output)
            for i, (kind, x, *_rest) in enumerate(specs):
                if i != 1 and x.numel():
                    x.copy_(torch.randn(x.shape, generator=gen, device="cuda").to(x.dtype))
        for _, _, _, _, out in specs:
            out.fill_(float("nan"))
        torch.cuda.synchronize()
        st.launch()
        torch.cuda.synchronize()
        # eager work between replays: the same calls one by one
        for i, (kind, x, Pg, Pu, out) in enumerate(specs):
            want = _eager(fn, kind, x, Pg, Pu)
            torch.cuda.synchronize()
            assert torch.equal(out.view(torch.int16) if out.dtype == torch.bfloat16 else out.view(torch.int32),
                               want.view(torch.int16) if want.dtype == torch.bfloat16 else want.view(torch.int32)), \
                f"replay {replay}, call {i} ({kind}) differs from the eager call"
    st.close()


def test_step_agrees_with_oracle(gpu_lib):
    """Replay of a small step against the float64 oracle, call by call."""
    import torch
    fn = gpu_lib
    st = fn.Step()
    cases = []
    for i, (M, K, N, sw) in enumerate([(8, 256, 520, False), (8, 1032, 270, True), (3, 40, 37, False)]):
        inp = W.random_inputs(M, K, N, "bf16", seed=200 + i, swiglu=sw)
        x = to_dev(inp.x, "bf16")
        Pg = fn.fold_weights(to_dev(inp.g, "bf16"), to_dev(inp.W, "bf16"))
        out = torch.empty((M, N), dtype=torch.bfloat16, device="cuda")
        if sw:
            Pu = fn.fold_weights(to_dev(inp.g, "bf16"), to_dev(inp.W_up, "bf16"))
            st.norm_proj_swiglu(x, Pg, Pu, out, 1e-6)
            ref = oracle.norm_proj_swiglu(inp.x, inp.g, inp.W, inp.W_up, 1e-6)
        else:
            st.norm_proj(x, Pg, out, 1e-6)
            ref = oracle.norm_proj(inp.x, inp.g, inp.W, 1e-6)
        cases.append((out, ref))
    st.record()
    st.launch()
    torch.cuda.synchronize()
    for i, (out, ref) in enumerate(cases):
        assert_close(to_f64(out), ref, "bf16", f"step call {i}")
    st.close()


def test_decode_step_graph_matches_eager(gpu_lib):
    """Four layers and the head of the M=8 decode step (real shapes) recorded
    as one step: every output equals the eager calls' bit for bit."""
    import torch
    fn = gpu_lib
    calls = W.decode_step_calls(4)
    st = fn.Step()
    items = []
    for c in calls:
        x, g, Wm, Wu = W.make_inputs_device(c)
        Pg = fn.fold_weights(g, Wm)
        Pu = fn.fold_weights(g, Wu) if c.swiglu else None
        out = torch.empty((c.M, c.N), dtype=torch.bfloat16, device="cuda")
        if c.swiglu:
            st.norm_proj_swiglu(x, Pg, Pu, out, c.eps)
        else:
            st.norm_proj(x, Pg, out, c.eps)
        items.append((x, Pg, Pu, out, c))
        del Wm, Wu
    st.record()
    for replay in range(2):
        for *_r, out, _c in items:
            out.fill_(float("nan"))
        st.launch()
        torch.cuda.synchronize()
        for x, Pg, Pu, out, c in items:
            want = fn.norm_proj_swiglu(x, Pg, Pu, c.eps) if c.swiglu else fn.norm_proj(x, Pg, c.eps)
            torch.cuda.synchronize()
            assert torch.equal(out.view(torch.int16), want.view(torch.int16)), f"replay {replay}: {c.name}"
    st.close()


def test_step_binding_rejects(gpu_lib):
    import torch
    fn = gpu_lib
    st = fn.Step()
    P = fn.fold_weights(None, torch.zeros((64, 32), dtype=torch.bfloat16, device="cuda"))
    with pytest.raises(ValueError):
        st.norm_proj(torch.zeros((2, 48), dtype=torch.bfloat16, device="cuda"), P,
                     torch.empty((2, 32), dtype=torch.bfloat16, device="cuda"))
    with pytest.raises(ValueError):
        st.norm_proj(torch.zeros((2, 64), dtype=torch.bfloat16, device="cuda"), P,
                     torch.empty((2, 31), dtype=torch.bfloat16, device="cuda"))
    with pytest.raises(RuntimeError):
        st.launch()
    x = torch.zeros((2, 64), dtype=torch.bfloat16, device="cuda")
    y = x[:, :32]                                    # output overlapping x: rejected by the C side
    st.norm_proj(x, P, torch.empty((2, 32), dtype=torch.bfloat16, device="cuda"))
    st._calls[-1].y = x.data_ptr()
    with pytest.raises(fn.FlashNormError, match="call 0"):
        st.record()
    del y
