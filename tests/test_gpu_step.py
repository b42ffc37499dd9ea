"""Recorded steps (fn_step_create / fn_step_launch): a sequence of fused
calls replayed with one HIP graph launch gives bit for bit what the same
calls give launched one by one, on every replay, with inputs refreshed in
place between replays; calls run in order, so a later call reads an earlier
call's output; and the replay agrees with the float64 oracle.  A grouped
step (fn_step_create_grouped) runs independent calls as one launch: with
bf16 weights the same bits as the eager calls that take the same tile, with
fp8 weights the eager outputs up to the order of the sum of squares, and the
oracle's values within tolerance for every call."""
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


def test_grouped_decode_step_matches_eager(gpu_lib):
    """The same four layers and head recorded as ONE grouped launch: every
    call is wide enough that its own entry point takes the one-wave tile, so
    each output equals the eager call's bit for bit, on every replay, with
    the inputs refreshed in place between replays."""
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
    st.record(grouped=True)
    assert st.num_kernels == 1
    gen = torch.Generator(device="cuda")
    for replay in range(3):
        if replay:
            gen.manual_seed(300 + replay)
            for x, *_r in items:
                x.copy_(torch.randn(x.shape, generator=gen, device="cuda").to(x.dtype))
        for *_r, out, _c in items:
            out.fill_(float("nan"))
        torch.cuda.synchronize()
        st.launch()
        torch.cuda.synchronize()
        for x, Pg, Pu, out, c in items:
            want = fn.norm_proj_swiglu(x, Pg, Pu, c.eps) if c.swiglu else fn.norm_proj(x, Pg, c.eps)
            torch.cuda.synchronize()
            assert torch.equal(out.view(torch.int16), want.view(torch.int16)), f"replay {replay}: {c.name}"
    st.close()


@pytest.mark.parametrize("seed", [0, 1])
def test_grouped_ragged_calls_agree_with_oracle(gpu_lib, seed):
    """Ragged calls in one grouped launch -- one row up to sixteen, K from 8
    to 4104, N from 1 to 1100 (narrow ones, which their own entry points
    split over k), an empty call between them -- each against the float64
    oracle; and the outputs of a second replay are the first's bits."""
    import torch
    fn = gpu_lib
    shapes = [(1, 8, 1, False), (16, 4104, 1100, True), (3, 264, 37, False), (0, 64, 32, False),
              (7, 1032, 270, True), (16, 520, 16, False), (9, 40, 600, False), (12, 2056, 33, True),
              (16, 4096, 530, False), (5, 136, 17, True)]
    st = fn.Step()
    cases = []
    for i, (M, K, N, sw) in enumerate(shapes):
        inp = W.random_inputs(M, K, N, "bf16", seed=400 + 20 * seed + i, swiglu=sw)
        x = to_dev(inp.x, "bf16")
        Pg = fn.fold_weights(to_dev(inp.g, "bf16"), to_dev(inp.W, "bf16"))
        out = torch.full((M, N), float("nan"), dtype=torch.bfloat16, device="cuda")
        if sw:
            Pu = fn.fold_weights(to_dev(inp.g, "bf16"), to_dev(inp.W_up, "bf16"))
            st.norm_proj_swiglu(x, Pg, Pu, out, 1e-6)
            ref = oracle.norm_proj_swiglu(inp.x, inp.g, inp.W, inp.W_up, 1e-6)
        else:
            st.norm_proj(x, Pg, out, 1e-6)
            ref = oracle.norm_proj(inp.x, inp.g, inp.W, 1e-6)
        cases.append((out, ref, (M, K, N, sw)))
    st.record(grouped=True)
    st.launch()
    torch.cuda.synchronize()
    first = [out.clone() for out, _r, _s in cases]
    for out, ref, shape in cases:
        assert_close(to_f64(out), ref, "bf16", f"grouped call {shape}")
        out.fill_(float("nan"))
    st.launch()
    torch.cuda.synchronize()
    for (out, _r, shape), f in zip(cases, first):
        assert torch.equal(out.view(torch.int16), f.view(torch.int16)), f"second replay differs: {shape}"
    st.close()


@pytest.mark.parametrize("seed", [0, 1])
def test_grouped_fp8_ragged_calls_agree_with_oracle(gpu_lib, seed):
    """fp8-weight calls in one grouped launch -- one row up to sixteen, K from
    8 to 4104 (odd counts of k-blocks, so a last pair with one k-block, and
    K % 32 != 0), N from 1 to 1100, an empty call between them -- each
    against the float64 oracle on the codes and scales of the oracle's own
    fold; a second replay gives the first's bits."""
    import torch
    fn = gpu_lib
    shapes = [(1, 8, 1, False), (16, 4104, 1100, True), (3, 264, 37, False), (0, 64, 32, True),
              (7, 1032, 270, True), (16, 520, 16, False), (9, 40, 600, False), (12, 2056, 33, True),
              (16, 4096, 530, False), (5, 136, 17, True), (8, 96, 70, False), (2, 4096, 3000, False)]
    st = fn.Step()
    cases = []
    for i, (M, K, N, sw) in enumerate(shapes):
        inp = W.random_inputs(M, K, N, "bf16", seed=700 + 20 * seed + i, swiglu=sw)
        x = to_dev(inp.x, "bf16")
        Pg = fn.fold_weights_fp8(to_dev(inp.g, "bf16"), to_dev(inp.W, "bf16"))
        cg, sg = oracle.fold_weights_fp8(inp.g, inp.W, "bf16")
        out = torch.full((M, N), float("nan"), dtype=torch.bfloat16, device="cuda")
        if sw:
            Pu = fn.fold_weights_fp8(to_dev(inp.g, "bf16"), to_dev(inp.W_up, "bf16"))
            cu, su = oracle.fold_weights_fp8(inp.g, inp.W_up, "bf16")
            st.norm_proj_swiglu_fp8(x, Pg, Pu, out, 1e-6)
            ref = oracle.norm_proj_swiglu_fp8(inp.x, cg, sg, cu, su, 1e-6)
        else:
            st.norm_proj_fp8(x, Pg, out, 1e-6)
            ref = oracle.norm_proj_fp8(inp.x, cg, sg, 1e-6)
        cases.append((out, ref, (M, K, N, sw)))
    st.record(grouped=True)
    assert st.num_kernels == 1
    st.launch()
    torch.cuda.synchronize()
    first = [out.clone() for out, _r, _s in cases]
    for out, ref, shape in cases:
        assert_close(to_f64(out), ref, "bf16", f"grouped fp8 call {shape}")
        out.fill_(float("nan"))
    st.launch()
    torch.cuda.synchronize()
    for (out, _r, shape), f in zip(cases, first):
        assert torch.equal(out.view(torch.int16), f.view(torch.int16)), f"second replay differs: {shape}"
    st.close()


def test_grouped_fp8_decode_step_agrees_with_eager(gpu_lib):
    """Four layers and the head with fp8 weights as ONE grouped launch, on
    three replays with the inputs refreshed in place: each output against
    the eager call's.  The products follow the same k order; only the sum of
    squares is added in another order (one chain over k here, per-wave
    partials in the eager kernel), so 1/RMS may differ in its last fp32 bit
    and an output by at most one bf16 step, rarely."""
    import torch
    fn = gpu_lib
    calls = W.decode_step_calls(4)
    st = fn.Step()
    items = []
    for c in calls:
        x, g, Wm, Wu = W.make_inputs_device(c)
        Pg = fn.fold_weights_fp8(g, Wm)
        Pu = fn.fold_weights_fp8(g, Wu) if c.swiglu else None
        out = torch.empty((c.M, c.N), dtype=torch.bfloat16, device="cuda")
        if c.swiglu:
            st.norm_proj_swiglu_fp8(x, Pg, Pu, out, c.eps)
        else:
            st.norm_proj_fp8(x, Pg, out, c.eps)
        items.append((x, Pg, Pu, out, c))
        del Wm, Wu
    st.record(grouped=True)
    assert st.num_kernels == 1
    gen = torch.Generator(device="cuda")
    for replay in range(3):
        if replay:
            gen.manual_seed(500 + replay)
            for x, *_r in items:
                x.copy_(torch.randn(x.shape, generator=gen, device="cuda").to(x.dtype))
        for *_r, out, _c in items:
            out.fill_(float("nan"))
        torch.cuda.synchronize()
        st.launch()
        torch.cuda.synchronize()
        for x, Pg, Pu, out, c in items:
            want = fn.norm_proj_swiglu_fp8(x, Pg, Pu, c.eps) if c.swiglu else fn.norm_proj_fp8(x, Pg, c.eps)
            torch.cuda.synchronize()
            a, b = out.double(), want.double()
            assert bool(torch.isfinite(a).all()), f"replay {replay}: {c.name} not finite"
            same = float((out.view(torch.int16) == want.view(torch.int16)).double().mean())
            assert same >= 0.999, f"replay {replay}: {c.name}: {same:.5f} of the outputs identical"
            assert bool(((a - b).abs() <= b.abs() * 2.0 ** -7 + 1e-30).all()), f"replay {replay}: {c.name}"
    st.close()


def _fold_any(fn, g, Wm, fp8):
    return fn.fold_weights_fp8(g, Wm) if fp8 else fn.fold_weights(g, Wm)


def _add_call(st, x, Pg, Pu, out, eps, fp8):
    if Pu is not None:
        (st.norm_proj_swiglu_fp8 if fp8 else st.norm_proj_swiglu)(x, Pg, Pu, out, eps)
    else:
        (st.norm_proj_fp8 if fp8 else st.norm_proj)(x, Pg, out, eps)


@pytest.mark.parametrize("fp8", [False, True])
@pytest.mark.parametrize("seed", [0, 1])
def test_grouped_wide_ragged_calls_agree_with_oracle(gpu_lib, fp8, seed):
    """A grouped step with calls of more than 16 rows takes the LDS-shared-x
    tile for every call (rows 1 to 128 in one launch, two 64-row blocks for
    the largest, K from 8 to 4104, N from 1 to 1100, an empty call): each
    output against the float64 oracle; a second replay gives the first's
    bits."""
    import torch
    fn = gpu_lib
    shapes = [(64, 4096, 530, True), (17, 8, 1, False), (3, 264, 37, True), (0, 64, 32, False),
              (40, 1032, 270, False), (64, 4104, 1100, False), (33, 40, 600, True), (16, 2056, 33, False),
              (1, 136, 17, True), (50, 96, 70, False), (128, 1032, 270, True), (97, 264, 530, False)]
    st = fn.Step()
    cases = []
    for i, (M, K, N, sw) in enumerate(shapes):
        inp = W.random_inputs(M, K, N, "bf16", seed=900 + 20 * seed + i, swiglu=sw)
        x = to_dev(inp.x, "bf16")
        g = to_dev(inp.g, "bf16")
        Pg = _fold_any(fn, g, to_dev(inp.W, "bf16"), fp8)
        Pu = _fold_any(fn, g, to_dev(inp.W_up, "bf16"), fp8) if sw else None
        out = torch.full((M, N), float("nan"), dtype=torch.bfloat16, device="cuda")
        _add_call(st, x, Pg, Pu, out, 1e-6, fp8)
        if fp8:
            cg, sg = oracle.fold_weights_fp8(inp.g, inp.W, "bf16")
            if sw:
                cu, su = oracle.fold_weights_fp8(inp.g, inp.W_up, "bf16")
                ref = oracle.norm_proj_swiglu_fp8(inp.x, cg, sg, cu, su, 1e-6)
            else:
                ref = oracle.norm_proj_fp8(inp.x, cg, sg, 1e-6)
        else:
            ref = (oracle.norm_proj_swiglu(inp.x, inp.g, inp.W, inp.W_up, 1e-6) if sw else
                   oracle.norm_proj(inp.x, inp.g, inp.W, 1e-6))
        cases.append((out, ref, (M, K, N, sw)))
    st.record(grouped=True)
    assert st.num_kernels == 1
    st.launch()
    torch.cuda.synchronize()
    first = [out.clone() for out, _r, _s in cases]
    for out, ref, shape in cases:
        assert_close(to_f64(out), ref, "bf16", f"wide grouped call {shape} fp8={fp8}")
        out.fill_(float("nan"))
    st.launch()
    torch.cuda.synchronize()
    for (out, _r, shape), f in zip(cases, first):
        assert torch.equal(out.view(torch.int16), f.view(torch.int16)), f"second replay differs: {shape}"
    st.close()


@pytest.mark.parametrize("rows", [64, 128])
@pytest.mark.parametrize("fp8", [False, True])
def test_grouped_wide_decode_step_agrees_with_eager(gpu_lib, fp8, rows):
    """Four layers and the head at 64 or 128 rows as one grouped launch (the
    LDS-shared-x tile, twelve column blocks and 64 rows per workgroup), on
    two replays with the inputs refreshed in place: each output against the
    eager call's, whichever kernel the row ladder gives it.  The products
    follow the same k order; the per-wave partial sums of
    squares are grouped differently, so 1/RMS may differ in its last fp32
    bit and an output by one bf16 step, rarely."""
    import torch
    fn = gpu_lib
    calls = W.decode_step_calls(4)
    st = fn.Step()
    items = []
    gen = torch.Generator(device="cuda")
    gen.manual_seed(610 + fp8 + rows)
    for c in calls:
        _x8, g, Wm, Wu = W.make_inputs_device(c)
        x = torch.randn((rows, c.K), generator=gen, device="cuda").to(torch.bfloat16)
        Pg = _fold_any(fn, g, Wm, fp8)
        Pu = _fold_any(fn, g, Wu, fp8) if c.swiglu else None
        out = torch.empty((rows, c.N), dtype=torch.bfloat16, device="cuda")
        _add_call(st, x, Pg, Pu, out, c.eps, fp8)
        items.append((x, Pg, Pu, out, c))
        del Wm, Wu
    st.record(grouped=True)
    for replay in range(2):
        if replay:
            for x, *_r in items:
                x.copy_(torch.randn(x.shape, generator=gen, device="cuda").to(x.dtype))
        for *_r, out, _c in items:
            out.fill_(float("nan"))
        torch.cuda.synchronize()
        st.launch()
        torch.cuda.synchronize()
        for x, Pg, Pu, out, c in items:
            if fp8:
                want = fn.norm_proj_swiglu_fp8(x, Pg, Pu, c.eps) if c.swiglu else fn.norm_proj_fp8(x, Pg, c.eps)
            else:
                want = fn.norm_proj_swiglu(x, Pg, Pu, c.eps) if c.swiglu else fn.norm_proj(x, Pg, c.eps)
            torch.cuda.synchronize()
            a, b = out.double(), want.double()
            assert bool(torch.isfinite(a).all()), f"replay {replay}: {c.name} not finite"
            same = float((out.view(torch.int16) == want.view(torch.int16)).double().mean())
            assert same >= 0.999, f"replay {replay}: {c.name}: {same:.5f} of the outputs identical"
            assert bool(((a - b).abs() <= b.abs() * 2.0 ** -7 + 1e-30).all()), f"replay {replay}: {c.name}"
    st.close()


def test_grouped_step_rejects_chained_calls(gpu_lib):
    """A call that reads another call's output cannot run at the same time
    as it: the grouped form refuses it (the recorded graph takes it)."""
    import torch
    fn = gpu_lib
    P1 = fn.fold_weights(None, torch.zeros((64, 64), dtype=torch.bfloat16, device="cuda"))
    P2 = fn.fold_weights(None, torch.zeros((64, 32), dtype=torch.bfloat16, device="cuda"))
    x = torch.zeros((2, 64), dtype=torch.bfloat16, device="cuda")
    h = torch.empty((2, 64), dtype=torch.bfloat16, device="cuda")
    y = torch.empty((2, 32), dtype=torch.bfloat16, device="cuda")
    st = fn.Step()
    st.norm_proj(x, P1, h)
    st.norm_proj(h, P2, y)
    with pytest.raises(fn.FlashNormError, match="at once"):
        st.record(grouped=True)
    st2 = fn.Step()
    st2.norm_proj(x, P1, h)
    st2.norm_proj(h, P2, y)
    st2.record()
    st2.close()
