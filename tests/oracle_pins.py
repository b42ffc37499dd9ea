"""Pins for the float64 oracle: checks that tie it to something other than
itself (hand-derived cases, brute force, a library routine, algebraic
invariants of the method).

Each check takes the oracle module as an argument so the same checks can be
run against deliberately broken copies of the oracle (see
test_oracle.py::test_pins_catch_planted_mistakes).  A check raises
AssertionError (or any exception) when the oracle disagrees.
"""
from __future__ import annotations

import json
import math
import os

import numpy as np

GOLDEN = os.path.join(os.path.dirname(__file__), "golden", "hand_cases.json")


def load_golden():
    with open(GOLDEN) as f:
        return json.load(f)


def _case_W(case):
    W = case["W"]
    if W == "diag_then_2diag":
        K = len(case["g"])
        W = np.zeros((K, 2 * K))
        for k in range(K):
            W[k, k] = 1.0
            W[k, k + K] = 2.0
    return np.asarray(W, dtype=np.float64)


def _close(a, b, tol, what):
    a = np.asarray(a, dtype=np.float64)
    b = np.asarray(b, dtype=np.float64)
    assert a.shape == b.shape, f"{what}: shape {a.shape} != {b.shape}"
    err = np.max(np.abs(a - b) / (np.abs(b) + 1.0)) if a.size else 0.0
    assert err <= tol, f"{what}: max rel err {err:.3e} > {tol:.1e}\n{a}\nvs\n{b}"


# --------------------------------------------------------------------------
# hand-derived worked cases (tests/golden/hand_cases.json)
# --------------------------------------------------------------------------
def check_hand_cases(o):
    from scipy.special import expit
    for case in load_golden()["cases"]:
        x = np.asarray(case["x"], dtype=np.float64)
        g = np.asarray(case["g"], dtype=np.float64)
        W = _case_W(case)
        eps = case["eps"]
        name = case["name"]
        _close(o.rms(x, eps), case["r"], 1e-15, f"{name}: r")
        _close(o.norm_proj(x, g, W, eps), case["y"], 1e-14, f"{name}: y")
        if "W_folded" in case:
            _close(o.fold_exact(g, W), case["W_folded"], 0.0, f"{name}: W'")
            _close(o.norm_proj_folded(x, case["W_folded"], eps), case["y"], 1e-14, f"{name}: folded y")
        if "W_up" in case:
            a = np.asarray(case["swiglu_a"], dtype=np.float64)
            b = np.asarray(case["swiglu_b"], dtype=np.float64)
            expected = a * expit(a) * b       # SiLU via scipy's logistic function
            _close(o.norm_proj_swiglu(x, g, W, case["W_up"], eps), expected, 1e-14, f"{name}: swiglu")


def check_silu_closed_forms(o):
    from scipy.special import expit
    t = np.array([-30.0, -2.5, -1.0, 0.0, 0.5, 1.5, 2.0, 30.0])
    _close(o.silu(t), t * expit(t), 1e-15, "silu vs t*expit(t)")
    # sigmoid(ln 3) = 3/4 exactly in real arithmetic
    _close(o.silu(np.log(3.0)), 0.75 * np.log(3.0), 1e-15, "silu(ln 3)")
    assert o.silu(np.array([0.0]))[0] == 0.0


# --------------------------------------------------------------------------
# brute force on tiny inputs: scalar loops over Python floats
# --------------------------------------------------------------------------
def _brute_norm_proj(x, g, W, eps, W_up=None):
    M, K = len(x), len(x[0])
    N = len(W[0])
    eps = float(np.float32(eps))
    out = []
    for m in range(M):
        s = 0.0
        for k in range(K):
            s += x[m][k] * x[m][k]
        r = math.sqrt(s / K + eps)
        xh = [x[m][k] / r * g[k] for k in range(K)]
        row = []
        for n in range(N):
            a = 0.0
            for k in range(K):
                a += xh[k] * W[k][n]
            if W_up is None:
                row.append(a)
            else:
                b = 0.0
                for k in range(K):
                    b += xh[k] * W_up[k][n]
                row.append(a / (1.0 + math.exp(-a)) * b)
        out.append(row)
    return out


def check_brute_force(o, seed=11):
    rng = np.random.default_rng(seed)
    for (M, K, N, eps) in [(1, 1, 1, 0.0), (3, 5, 4, 1e-6), (2, 7, 3, 0.5), (4, 6, 6, 0.0)]:
        x = rng.standard_normal((M, K))
        g = rng.uniform(0.5, 1.5, K)
        W = rng.standard_normal((K, N))
        Wu = rng.standard_normal((K, N))
        ref = _brute_norm_proj(x.tolist(), g.tolist(), W.tolist(), eps)
        _close(o.norm_proj(x, g, W, eps), ref, 1e-13, f"brute norm_proj {M}x{K}x{N}")
        ref = _brute_norm_proj(x.tolist(), g.tolist(), W.tolist(), eps, Wu.tolist())
        _close(o.norm_proj_swiglu(x, g, W, Wu, eps), ref, 1e-13, f"brute swiglu {M}x{K}x{N}")


# --------------------------------------------------------------------------
# library special case: torch's float64 rms_norm, then a float64 matmul
# --------------------------------------------------------------------------
def check_torch_rms_norm(o, seed=12):
    import torch
    rng = np.random.default_rng(seed)
    for (M, K, N, eps) in [(5, 64, 24, 1e-6), (3, 40, 9, 0.25), (2, 16, 16, 0.0)]:
        x = rng.standard_normal((M, K))
        g = rng.uniform(0.5, 1.5, K)
        W = rng.standard_normal((K, N))
        eps32 = float(np.float32(eps))
        xt = torch.from_numpy(x)
        ref = torch.nn.functional.rms_norm(xt, (K,), torch.from_numpy(g), eps32) @ torch.from_numpy(W)
        _close(o.norm_proj(x, g, W, eps), ref.numpy(), 1e-13, f"torch rms_norm@W {M}x{K}x{N}")
        # g = 1: plain rms_norm without weight
        ref1 = torch.nn.functional.rms_norm(xt, (K,), None, eps32).numpy() @ W
        _close(o.norm_proj(x, np.ones(K), W, eps), ref1, 1e-13, "g=1 rms_norm@W")
    # rows pre-scaled to RMS 1 with eps = 0: the norm is the identity, y = x @ W
    x = rng.standard_normal((4, 32))
    x = x / np.sqrt(np.mean(x * x, axis=1, keepdims=True))
    W = rng.standard_normal((32, 8))
    _close(o.norm_proj(x, np.ones(32), W, 0.0), x @ W, 1e-13, "unit-RMS rows give x@W")


# --------------------------------------------------------------------------
# algebraic invariants of the method
# --------------------------------------------------------------------------
def check_fold_identity(o, seed=13):
    """Proposal 1 + 2: folded + deferred equals the unfolded definition."""
    rng = np.random.default_rng(seed)
    M, K, N = 6, 48, 20
    x = rng.standard_normal((M, K))
    g = rng.uniform(0.5, 1.5, K)
    W = rng.standard_normal((K, N))
    Wu = rng.standard_normal((K, N))
    for eps in (0.0, 1e-6, 0.3):
        _close(o.norm_proj_folded(x, o.fold_exact(g, W), eps), o.norm_proj(x, g, W, eps), 1e-13, "I1 fold")
        _close(o.norm_proj_swiglu_folded(x, o.fold_exact(g, W), o.fold_exact(g, Wu), eps),
               o.norm_proj_swiglu(x, g, W, Wu, eps), 1e-13, "I1 fold swiglu")


def check_scale_invariance(o, seed=14):
    """RMSNorm(c x) = RMSNorm(x) for c > 0 at eps = 0 (proposal 3's premise)."""
    rng = np.random.default_rng(seed)
    M, K, N = 5, 40, 12
    x = rng.standard_normal((M, K))
    g = rng.uniform(0.5, 1.5, K)
    W = rng.standard_normal((K, N))
    base = o.norm_proj(x, g, W, 0.0)
    for p in (-3, 5):
        assert np.array_equal(o.norm_proj(x * 2.0 ** p, g, W, 0.0), base), f"I2 bit-exact for 2^{p}"
    for c in (0.3, 7.1):
        _close(o.norm_proj(c * x, g, W, 0.0), base, 1e-14, f"I2 c={c}")
    # with eps > 0 the difference is bounded by about eps / mean(x^2)
    eps = 1e-3
    d = np.max(np.abs(o.norm_proj(10.0 * x, g, W, eps) - o.norm_proj(x, g, W, eps)))
    scale = np.max(np.abs(base))
    assert 0 < d <= 2 * eps / np.min(np.mean(x * x, axis=1)) * scale, "I2 eps>0 bound"
    # and scaling x down must change y when eps dominates (eps really enters)
    small = o.norm_proj(1e-6 * x, g, W, 1.0)
    assert np.max(np.abs(small)) < 1e-5 * scale


def check_double_norm(o, seed=15):
    """A gain-free norm followed by RMSNorm_g equals RMSNorm_g alone at eps=0
    (proposal 3, double-norm removal)."""
    rng = np.random.default_rng(seed)
    x = rng.standard_normal((7, 33))
    g = rng.uniform(0.5, 1.5, 33)
    once = o.rmsnorm(x, g, 0.0)
    twice = o.rmsnorm(o.rmsnorm(x, np.ones(33), 0.0), g, 0.0)
    _close(twice, once, 1e-15, "I3 double norm")
    _close(o.rms(o.rmsnorm(x, np.ones(33), 0.0), 0.0), np.ones(7), 1e-15, "I3 unit rms")


def check_rows_and_columns(o, seed=16):
    """Rows are independent (permutation, NaN isolation); columns are
    independent and the map is linear in W (concatenation, scaling)."""
    rng = np.random.default_rng(seed)
    M, K, N = 8, 24, 10
    x = rng.standard_normal((M, K))
    g = rng.uniform(0.5, 1.5, K)
    W1 = rng.standard_normal((K, N))
    W2 = rng.standard_normal((K, 3))
    y = o.norm_proj(x, g, W1, 1e-6)
    perm = rng.permutation(M)
    assert np.array_equal(o.norm_proj(x[perm], g, W1, 1e-6), y[perm]), "I6 permutation"
    xn = x.copy()
    xn[3, 5] = np.nan
    yn = o.norm_proj(xn, g, W1, 1e-6)
    assert np.all(np.isnan(yn[3])), "I6 NaN row"
    assert np.array_equal(np.delete(yn, 3, 0), np.delete(y, 3, 0)), "I6 NaN isolated"
    cat = o.norm_proj(x, g, np.concatenate([W1, W2], axis=1), 1e-6)
    _close(cat, np.concatenate([y, o.norm_proj(x, g, W2, 1e-6)], axis=1), 1e-14, "I7 concat")
    _close(o.norm_proj(x, g, 2.5 * W1, 1e-6), 2.5 * y, 1e-14, "I7 linear")


# --------------------------------------------------------------------------
# storage rounding
# --------------------------------------------------------------------------
def check_rounding(o, seed=17):
    import torch
    gold = load_golden()
    for desc, v, want in gold["rne_bf16"]["pairs"]:
        got = o.round_to_bf16(np.array([v]))[0]
        assert got == want, f"bf16 RNE {desc}: {got!r} != {want!r}"
    for desc, v, want in gold["rne_f32"]["pairs"]:
        got = o.round_to_f32(np.array([v]))[0]
        assert got == want, f"f32 RNE {desc}: {got!r} != {want!r}"
    # library cross-check: torch's CPU float32 -> bfloat16 conversion (RNE)
    rng = np.random.default_rng(seed)
    bits = rng.integers(0, 2 ** 32, size=200000, dtype=np.uint64).astype(np.uint32)
    f = bits.view(np.float32)
    f = f[np.isfinite(f)]
    ties = (rng.integers(0, 2 ** 16, size=5000).astype(np.uint32) << 16) | np.uint32(0x8000)
    f = np.concatenate([f, ties.view(np.float32)])
    f = f[np.isfinite(f)]
    ref = torch.from_numpy(f).to(torch.bfloat16).to(torch.float64).numpy()
    got = o.round_to_bf16(f.astype(np.float64))
    assert np.array_equal(got, ref), "bf16 RNE vs torch"
    assert np.isnan(o.round_to_bf16(np.array([np.nan]))[0])
    assert o.round_to_bf16(np.array([3.5e38]))[0] == np.inf


def check_fold_rounding(o, seed=18):
    """W' = one rounding of the exact product: bf16 against torch's conversion
    of the (exact) fp32 product, fp32 against numpy's IEEE fp32 multiply."""
    import torch
    rng = np.random.default_rng(seed)
    K, N = 64, 48
    g32 = torch.from_numpy(rng.uniform(0.5, 1.5, K).astype(np.float32)).to(torch.bfloat16).float()
    W32 = torch.from_numpy(rng.standard_normal((K, N)).astype(np.float32)).to(torch.bfloat16).float()
    ref = (g32[:, None] * W32).to(torch.bfloat16).double().numpy()
    got = o.fold_weights(g32.double().numpy(), W32.double().numpy(), "bf16")
    assert np.array_equal(got, ref), "fold bf16"
    gf = rng.uniform(0.5, 1.5, K).astype(np.float32)
    Wf = rng.standard_normal((K, N)).astype(np.float32)
    ref = (gf[:, None] * Wf).astype(np.float64)
    got = o.fold_weights(gf.astype(np.float64), Wf.astype(np.float64), "f32")
    assert np.array_equal(got, ref), "fold f32"
    ones = np.ones(K)
    assert np.array_equal(o.fold_weights(ones, W32.double().numpy(), "bf16"), W32.double().numpy()), "g=1 fold"


ALL_CHECKS = [check_hand_cases, check_silu_closed_forms, check_brute_force, check_torch_rms_norm,
              check_fold_identity, check_scale_invariance, check_double_norm,
              check_rows_and_columns, check_rounding, check_fold_rounding]


# --------------------------------------------------------------------------
# fp8 (E4M3) weights
# --------------------------------------------------------------------------
def check_e4m3_codes(o, seed=19):
    """Decode and encode against hand-evaluated codes, the format's
    structure, and torch's float8_e4m3fn conversion (RNE) as a library
    cross-check."""
    import torch
    gold = load_golden()["e4m3"]
    for desc, code, want in gold["decode"]:
        got = o.e4m3_decode(np.array([code]))[0]
        assert got == want and np.signbit(got) == np.signbit(want), f"decode {desc}: {got!r} != {want!r}"
    for desc, v, want in gold["encode"]:
        got = int(o.e4m3_encode(np.array([v]))[0])
        assert got == want, f"encode {desc}: {got:#x} != {want:#x}"
    codes = np.arange(256, dtype=np.uint8)
    vals = o.e4m3_decode(codes)
    finite = ~np.isnan(vals)
    assert finite.sum() == 254 and not finite[0x7F] and not finite[0xFF]
    pos = vals[:0x7F]
    assert np.all(np.diff(pos) > 0), "positive codes are not increasing"
    assert np.array_equal(vals[0x80:0xFF], -pos), "negative codes mirror the positive ones"
    assert np.array_equal(o.e4m3_encode(vals[finite]), codes[finite]), "round trip"
    ref = torch.from_numpy(codes).view(torch.float8_e4m3fn).to(torch.float64).numpy()
    assert np.array_equal(np.isnan(ref), np.isnan(vals)) and np.array_equal(ref[finite], vals[finite]), "decode vs torch"
    # random fp32 values in range, plus every midpoint between neighbours
    rng = np.random.default_rng(seed)
    f = np.concatenate([rng.uniform(-448, 448, 20000), rng.standard_normal(20000) * 0.01,
                        (pos[1:] + pos[:-1]) / 2, -(pos[1:] + pos[:-1]) / 2]).astype(np.float32)
    ref = torch.from_numpy(f).to(torch.float8_e4m3fn).view(torch.uint8).numpy()
    got = o.e4m3_encode(f.astype(np.float64))
    assert np.array_equal(got, ref), "encode vs torch"


def check_e4m3_quantize(o, seed=20):
    """Per-column quantisation: a hand-evaluated column, an all-zero column,
    each column's largest magnitude landing on +-448, and the rounding error
    bound (half a quantum of the scaled value)."""
    gold = load_golden()["e4m3"]["quantize_column"]
    W = np.zeros((4, 2))
    W[:, 0] = gold["W"]
    codes, s, r = o.quantize_e4m3_columns(W)
    assert [int(c) for c in codes[:, 0]] == gold["codes"], codes[:, 0]
    assert float(s[0]) == gold["s"], s[0]
    assert np.all(codes[:, 1] == 0) and s[1] == 1.0 and r[1] == 1.0, "all-zero column"
    rng = np.random.default_rng(seed)
    Wf = (rng.standard_normal((96, 40)) / 8).astype(np.float32)
    Wf[:, 3] *= 1e-3
    codes, s, r = o.quantize_e4m3_columns(Wf)
    vals = o.e4m3_decode(codes)
    top = np.argmax(np.abs(Wf), axis=0)
    assert np.all(np.abs(vals[top, np.arange(40)]) == 448.0), "column maximum maps to +-448"
    scaled = Wf.astype(np.float64) * r.astype(np.float64)[None, :]
    _, e = np.frexp(np.abs(scaled))
    half_quantum = np.ldexp(1.0, np.maximum(e, -5) - 5)
    assert np.all(np.abs(vals - scaled) <= half_quantum * (1 + 1e-6)), "E4M3 rounding error bound"
    assert np.allclose(s.astype(np.float64) * r.astype(np.float64), 1.0, rtol=2e-7), "s = 1/r"


def check_norm_proj_fp8(o, seed=21):
    """With weights whose scaled values are exact E4M3 values the fp8 path is
    the deferred bf16 path, exactly; brute force on a tiny case."""
    rng = np.random.default_rng(seed)
    K, N, M = 48, 24, 5
    pool = o.e4m3_decode(np.arange(0, 0x7F, dtype=np.uint8))
    pick = rng.choice(pool, size=(K, N)) * rng.choice([-1.0, 1.0], size=(K, N))
    pick[0, :] = 448.0                          # each column's amax is 448 -> r = s = 1
    Wf = (pick * np.ldexp(1.0, -6)).astype(np.float32)   # power-of-two rescale keeps exactness
    codes, s, r = o.quantize_e4m3_columns(Wf)
    assert np.all(r == 448.0 / (448.0 * 2.0 ** -6))
    x = rng.standard_normal((M, K))
    y = o.norm_proj_fp8(x, codes, s, 1e-6)
    ref = o.norm_proj_folded(x, Wf.astype(np.float64), 1e-6)
    _close(y, ref, 1e-12, "fp8 exact weights vs deferred form")
    codes_u, s_u, _ = o.quantize_e4m3_columns(Wf[::-1].copy())
    a = o.norm_proj_swiglu_fp8(x, codes, s, codes_u, s_u, 1e-6)
    ref = o.norm_proj_swiglu_folded(x, Wf.astype(np.float64), Wf[::-1].astype(np.float64), 1e-6)
    _close(a, ref, 1e-12, "fp8 SwiGLU exact weights vs deferred form")
    # brute force, arbitrary weights
    Wr = rng.standard_normal((6, 3)).astype(np.float32)
    c2, s2, _ = o.quantize_e4m3_columns(Wr)
    xs = rng.standard_normal((2, 6))
    got = o.norm_proj_fp8(xs, c2, s2, 0.25)
    for m in range(2):
        ms = sum(float(v) ** 2 for v in xs[m]) / 6
        rr = math.sqrt(ms + float(np.float32(0.25)))
        for n in range(3):
            acc = 0.0
            for k in range(6):
                acc += float(xs[m, k]) * float(o.e4m3_decode(np.array([c2[k, n]]))[0])
            want = acc * float(s2[n]) / rr
            assert abs(got[m, n] - want) <= 1e-12 * (abs(want) + 1), (m, n, got[m, n], want)


def check_fold_fp8(o):
    """Fold, store, then quantise per column: the hand-derived case (a
    product that bf16 storage rounds, so quantising the unrounded product or
    the unfolded W gives other scales and codes), and the composition on
    random bf16 values against torch (the fp32 product rounded to bf16, the
    column maxima, and torch's float8_e4m3fn conversion of the scaled
    values): the codes and scales of the stored W', not of W or of g*W
    before rounding."""
    import torch
    c = load_golden()["e4m3"]["fold_fp8"]
    codes, s = o.fold_weights_fp8(np.array(c["g"]), np.array(c["W"]), "bf16")
    assert codes.tolist() == c["codes"], codes
    assert s.dtype == np.float32 and [float(v) for v in s] == c["s"], s
    rng = np.random.default_rng(28)
    K, N = 40, 24
    g = torch.from_numpy(rng.uniform(0.5, 1.5, K).astype(np.float32)).to(torch.bfloat16).float()
    W = torch.from_numpy(rng.standard_normal((K, N)).astype(np.float32)).to(torch.bfloat16).float()
    stored = (g[:, None] * W).to(torch.bfloat16).float()        # fp32 product (exact), RNE to bf16
    amax = stored.abs().amax(dim=0)
    r = torch.tensor(448.0) / amax
    want = (stored * r[None, :]).to(torch.float8_e4m3fn).view(torch.uint8).numpy()
    codes, s = o.fold_weights_fp8(g.double().numpy(), W.double().numpy(), "bf16")
    assert np.array_equal(codes, want), "codes of the stored W' (torch float8_e4m3fn)"
    assert np.array_equal(s, (amax / torch.tensor(448.0)).numpy()), "scales of the stored W'"


ALL_CHECKS += [check_e4m3_codes, check_e4m3_quantize, check_norm_proj_fp8, check_fold_fp8]


# --------------------------------------------------------------------------
# fp8 output: E4M3 codes with one scale per 16-column row block
# --------------------------------------------------------------------------
def check_e4m3_row_blocks(o, seed=22):
    """Row-block quantisation: a hand-evaluated case (ties, a subnormal, a
    ragged last block, an all-zero row), codes equal to torch's
    float8_e4m3fn conversion of the scaled fp32 values (scales computed here
    block by block in plain loops), the rounding error bound of the values
    read back, and independence of blocks and rows."""
    import torch
    gold = load_golden()["e4m3"]["quantize_row_blocks"]
    codes, s = o.quantize_e4m3_row_blocks(np.array(gold["v"]))
    assert codes.tolist() == gold["codes"], codes
    assert s.tolist() == gold["s"], s
    assert o.Q8_BLOCK == 16
    rng = np.random.default_rng(seed)
    M, N, B = 5, 37, 16
    v = (rng.standard_normal((M, N)) * np.exp(rng.uniform(-6, 3, (M, 1)))).astype(np.float32)
    v[2, 16:32] = 0.0                                   # an all-zero block inside a row
    codes, s = o.quantize_e4m3_row_blocks(v)
    assert codes.shape == (M, N) and s.shape == (M, 3) and codes.dtype == np.uint8
    for m in range(M):
        for b in range(3):
            blk = v[m, b * B:(b + 1) * B]
            amax = np.float32(max(abs(float(t)) for t in blk))
            if amax == 0:
                assert s[m, b] == 1.0 and np.all(codes[m, b * B:(b + 1) * B] == 0)
                continue
            r = np.float32(np.float32(448.0) / amax)
            assert s[m, b] == np.float32(amax / np.float32(448.0)), (m, b)
            scaled = (blk * r).astype(np.float32)
            ref = torch.from_numpy(scaled.copy()).to(torch.float8_e4m3fn).view(torch.uint8).numpy()
            assert np.array_equal(codes[m, b * B:(b + 1) * B], ref), (m, b)
    back = o.dequantize_row_blocks(codes, s)
    blk_s = np.repeat(s.astype(np.float64), B, axis=1)[:, :N]
    _, e = np.frexp(np.abs(v.astype(np.float64) / blk_s))
    bound = np.ldexp(1.0, np.maximum(e, -5) - 5) * blk_s * (1 + 1e-6)
    assert np.all(np.abs(back - v) <= bound), "row-block rounding error bound"
    w = v.copy()
    w[0, 16:32] *= 1000.0                               # another block of row 0, and other rows untouched
    w[4] = -w[4]
    c2, s2 = o.quantize_e4m3_row_blocks(w)
    assert np.array_equal(c2[0, :16], codes[0, :16]) and np.array_equal(c2[0, 32:], codes[0, 32:])
    assert np.array_equal(c2[1:4], codes[1:4]) and np.array_equal(s2[1:4], s[1:4])
    assert np.array_equal(o.dequantize_row_blocks(c2, s2)[4], -back[4]) and np.array_equal(s2[4], s[4]), "sign symmetry"


def check_norm_proj_swiglu_q8(o, seed=23):
    """The quantised SwiGLU output is the row-block quantisation of the
    SwiGLU output (bf16 and fp8 weights), and reads back within the E4M3
    bound of it."""
    rng = np.random.default_rng(seed)
    M, K, N = 3, 32, 20
    x = rng.standard_normal((M, K))
    g = rng.uniform(0.5, 1.5, K)
    Wg, Wu = rng.standard_normal((K, N)) / 6, rng.standard_normal((K, N)) / 6
    codes, s, v = o.norm_proj_swiglu_q8(x, g, Wg, Wu, 1e-6)
    _close(v, o.norm_proj_swiglu(x, g, Wg, Wu, 1e-6), 0.0, "q8 value")
    c2, s2 = o.quantize_e4m3_row_blocks(v)
    assert np.array_equal(codes, c2) and np.array_equal(s, s2)
    back = o.dequantize_row_blocks(codes, s)
    assert np.all(np.abs(back - v) <= np.abs(v) / 16 + np.repeat(s, 16, axis=1)[:, :N] * 2.0 ** -9 + 1e-9)
    cg, sg, _ = o.quantize_e4m3_columns(Wg.astype(np.float32))
    cu, su, _ = o.quantize_e4m3_columns(Wu.astype(np.float32))
    c8, s8, v8 = o.norm_proj_swiglu_fp8_q8(x, cg, sg, cu, su, 1e-6)
    _close(v8, o.norm_proj_swiglu_fp8(x, cg, sg, cu, su, 1e-6), 0.0, "fp8 q8 value")
    c3, s3 = o.quantize_e4m3_row_blocks(v8)
    assert np.array_equal(c8, c3) and np.array_equal(s8, s3)


ALL_CHECKS += [check_e4m3_row_blocks, check_norm_proj_swiglu_q8]


# --------------------------------------------------------------------------
# AdaLN prologue
# --------------------------------------------------------------------------
def check_adaln(o, seed=24):
    """AdaLN after the norm: the hand-derived case, the reductions to the
    plain path (zero tables; a constant scale), row permutation together
    with idx, table row duplication, and brute force of the definition."""
    gold = load_golden()["adaln"]
    h = o.adaln_modulate(gold["x"], gold["g"], gold["scale"], gold["shift"], gold["idx"], 0.0)
    assert np.array_equal(h, np.array(gold["h"])), h
    y = o.adaln_norm_proj(gold["x"], gold["g"], gold["scale"], gold["shift"], gold["idx"], gold["W"], 0.0)
    assert np.array_equal(y[:, 0], np.array(gold["y"])), y
    out = o.adaln_norm_proj_swiglu(gold["x"], gold["g"], gold["scale"], gold["shift"], gold["idx"], gold["W"],
                                   gold["W_up"], 0.0)
    want = [a / (1 + math.exp(-a)) * b for a, b in zip(gold["a"], gold["b"])]
    _close(out[:, 0], np.array(want), 1e-15, "adaln swiglu hand case")

    rng = np.random.default_rng(seed)
    M, K, N, T = 7, 24, 10, 3
    x = rng.standard_normal((M, K))
    g = rng.uniform(0.5, 1.5, K)
    W = rng.standard_normal((K, N)) / 5
    Wu = rng.standard_normal((K, N)) / 5
    sc = rng.standard_normal((T, K)) * 0.3
    sh = rng.standard_normal((T, K)) * 0.3
    idx = rng.integers(0, T, M)
    zeros = np.zeros((T, K))
    assert np.array_equal(o.adaln_norm_proj(x, g, zeros, zeros, idx, W, 1e-6), o.norm_proj(x, g, W, 1e-6)), \
        "zero tables give the plain path"
    assert np.array_equal(o.adaln_norm_proj_swiglu(x, g, zeros, zeros, idx, W, Wu, 1e-6),
                          o.norm_proj_swiglu(x, g, W, Wu, 1e-6))
    const = np.full((T, K), 0.25)
    _close(o.adaln_norm_proj(x, g, const, zeros, idx, W, 1e-6), 1.25 * o.norm_proj(x, g, W, 1e-6), 1e-13,
           "constant scale")
    perm = rng.permutation(M)
    _close(o.adaln_norm_proj(x[perm], g, sc, sh, idx[perm], W, 1e-6),
           o.adaln_norm_proj(x, g, sc, sh, idx, W, 1e-6)[perm], 1e-14, "row permutation with idx")
    sc2, sh2 = np.vstack([sc, sc[1:2]]), np.vstack([sh, sh[1:2]])
    idx2 = np.where(idx == 1, T, idx)
    _close(o.adaln_norm_proj(x, g, sc2, sh2, idx2, W, 1e-6), o.adaln_norm_proj(x, g, sc, sh, idx, W, 1e-6), 1e-14,
           "duplicated table row")
    # brute force
    xs, gs, Ws = x[:2, :5], g[:5], W[:5, :3]
    got = o.adaln_norm_proj(xs, gs, sc[:, :5], sh[:, :5], idx[:2], Ws, 0.5)
    for m in range(2):
        r = math.sqrt(sum(float(v) ** 2 for v in xs[m]) / 5 + float(np.float32(0.5)))
        for n in range(3):
            acc = 0.0
            for k in range(5):
                hk = float(xs[m, k]) / r * float(gs[k]) * (1 + float(sc[idx[m], k])) + float(sh[idx[m], k])
                acc += hk * float(Ws[k, n])
            assert abs(got[m, n] - acc) <= 1e-12 * (abs(acc) + 1), (m, n)


def check_adaln_fold_table(o, seed=29):
    """The gain folded into the modulation table: hand-derived values (one
    where float64-then-float32 differs from float32 steps), the reductions
    scale 0 -> g and scale -1 -> 0, and on random bf16 values a float32
    value within half a float32 step of the exact product."""
    for c in load_golden()["adaln_fold_table"]["cases"]:
        got = o.adaln_fold_table(np.array([c["g"]]), np.array([[c["s"]]]))
        assert got.shape == (1, 1) and got[0, 0] == c["mod"], (c, got)
    rng = np.random.default_rng(seed)
    T, K = 4, 64
    g = o.round_to_bf16(rng.uniform(0.5, 1.5, K))
    sc = o.round_to_bf16(rng.standard_normal((T, K)) * 0.3)
    assert np.array_equal(o.adaln_fold_table(g, np.zeros((T, K))), np.tile(g, (T, 1)))
    assert np.array_equal(o.adaln_fold_table(g, -np.ones((T, K))), np.zeros((T, K)))
    got = o.adaln_fold_table(g, sc)
    assert np.array_equal(o.round_to_f32(got), got), "float32 values"
    from fractions import Fraction
    for t in range(T):
        for k in range(0, K, 7):
            exact = Fraction(float(g[k])) * (1 + Fraction(float(sc[t, k])))
            step = Fraction(2) ** (math.frexp(float(exact))[1] - 24)
            assert abs(Fraction(float(got[t, k])) - exact) <= step / 2, (t, k)


def check_adaln_fold(o, seed=30):
    """The folded and deferred AdaLN form against the definition: with the
    unrounded table g * (1 + scale) and bias rows shift @ W it equals
    adaln_norm_proj and adaln_norm_proj_swiglu; an index outside the table
    gives a zero row (h = 0); brute force."""
    rng = np.random.default_rng(seed)
    M, K, N, T = 7, 24, 10, 3
    x = rng.standard_normal((M, K))
    g = rng.uniform(0.5, 1.5, K)
    W = rng.standard_normal((K, N)) / 5
    Wu = rng.standard_normal((K, N)) / 5
    sc = rng.standard_normal((T, K)) * 0.3
    sh = rng.standard_normal((T, K)) * 0.3
    idx = rng.integers(0, T, M)
    mod = g[None, :] * (1 + sc)
    bias, bias_u = o.adaln_shift_bias(sh, W), o.adaln_shift_bias(sh, Wu)
    for t in range(T):          # brute force of the bias rows
        for n in range(0, N, 3):
            want = sum(float(sh[t, k]) * float(W[k, n]) for k in range(K))
            assert abs(bias[t, n] - want) <= 1e-13 * (abs(want) + 1), (t, n)
    _close(o.adaln_norm_proj_fold(x, W, mod, bias, idx, 1e-6), o.adaln_norm_proj(x, g, sc, sh, idx, W, 1e-6),
           1e-12, "folded/deferred AdaLN identity")
    _close(o.adaln_norm_proj_swiglu_fold(x, W, Wu, mod, bias, bias_u, idx, 1e-6),
           o.adaln_norm_proj_swiglu(x, g, sc, sh, idx, W, Wu, 1e-6), 1e-12, "folded/deferred AdaLN SwiGLU")
    bad = idx.copy()
    bad[0], bad[-1] = -1, T
    y = o.adaln_norm_proj_fold(x, W, mod, bias, bad, 1e-6)
    assert np.all(y[[0, M - 1]] == 0), "rows outside the table are zero"
    assert np.array_equal(y[1:M - 1], o.adaln_norm_proj_fold(x, W, mod, bias, idx, 1e-6)[1:M - 1])
    sc1 = np.vstack([sc, -np.ones((1, K))])
    sh1 = np.vstack([sh, np.zeros((1, K))])
    _close(o.adaln_norm_proj_fold(x, W, mod, bias, bad, 1e-6),
           o.adaln_norm_proj(x, g, sc1, sh1, np.where(bad == -1, T, np.minimum(bad, T)), W, 1e-6), 1e-12,
           "an index outside the table is scale -1, shift 0")
    xs = x[:2, :5]
    got = o.adaln_norm_proj_fold(xs, W[:5, :3], mod[:, :5], bias[:, :3], idx[:2], 0.25)
    for m in range(2):
        r = math.sqrt(sum(float(v) ** 2 for v in xs[m]) / 5 + float(np.float32(0.25)))
        for n in range(3):
            acc = sum(float(xs[m, k]) * float(mod[idx[m], k]) * float(W[k, n]) for k in range(5))
            want = acc / r + float(bias[idx[m], n])
            assert abs(got[m, n] - want) <= 1e-12 * (abs(want) + 1), (m, n)


ALL_CHECKS += [check_adaln, check_adaln_fold_table, check_adaln_fold]


def check_adaln_operand(o, seed=25):
    """The AdaLN operand: hand-derived roundings (ties to even both ways, a
    rounding up and down off the midpoint, exact zero and doubling, indices
    outside the table, the float32 step before the bf16 one), and on random
    values the reductions that fix it without rounding: mod 1 gives x, mod 0
    gives 0, mod 2 gives 2x, and a per-row table lookup equals the
    row-by-row computation."""
    for c in load_golden()["adaln_operand"]["cases"]:
        got = o.adaln_operand(np.array([[c["x"]]]), np.array([[c["mod"]]]), np.array([c["idx"]]))
        assert got.shape == (1, 1) and got[0, 0] == c["u"], (c, got)
    rng = np.random.default_rng(seed)
    M, K, T = 6, 40, 3
    x = o.round_to_bf16(rng.standard_normal((M, K)))
    mod = o.round_to_f32(rng.uniform(0.2, 2.0, (T, K)))
    idx = rng.integers(0, T, M)
    assert np.array_equal(o.adaln_operand(x, np.ones((T, K)), idx), x)
    assert np.array_equal(o.adaln_operand(x, np.zeros((T, K)), idx), np.zeros((M, K)))
    assert np.array_equal(o.adaln_operand(x, 2 * np.ones((T, K)), idx), 2 * x)
    got = o.adaln_operand(x, mod, idx)
    for m in range(M):
        row = o.adaln_operand(x[m:m + 1], mod[idx[m]:idx[m] + 1], np.array([0]))
        assert np.array_equal(got[m], row[0]), m
    # every result is a bf16 value within half a bf16 step (plus the float32 step) of the exact product
    exact = x * mod[idx]
    step = np.ldexp(1.0, np.frexp(exact)[1] - 8)
    assert np.all(np.abs(got - exact) <= step / 2 * (1 + 2.0 ** -15) + 1e-300)
    assert np.array_equal(o.round_to_bf16(got), got)


ALL_CHECKS += [check_adaln_operand]


def check_adaln_fp8(o, seed=26):
    """AdaLN with E4M3 weights: with weights whose scaled values are exact
    E4M3 values it is the folded/deferred AdaLN form on those weights
    (itself pinned to the definition above); a table of ones and zero bias
    give the plain fp8 path; brute force on a tiny case."""
    rng = np.random.default_rng(seed)
    K, N, M, T = 48, 24, 6, 3
    pool = o.e4m3_decode(np.arange(0, 0x7F, dtype=np.uint8))
    pick = rng.choice(pool, size=(K, N)) * rng.choice([-1.0, 1.0], size=(K, N))
    pick[0, :] = 448.0
    Wf = (pick * np.ldexp(1.0, -6)).astype(np.float32)
    codes, s, _ = o.quantize_e4m3_columns(Wf)
    codes_u, s_u, _ = o.quantize_e4m3_columns(Wf[::-1].copy())
    x = rng.standard_normal((M, K))
    mod = rng.uniform(0.2, 2.0, (T, K))
    bias = rng.standard_normal((T, N))
    bias_u = rng.standard_normal((T, N))
    idx = rng.integers(0, T, M)
    _close(o.adaln_norm_proj_fp8(x, codes, s, mod, bias, idx, 1e-6),
           o.adaln_norm_proj_fold(x, Wf.astype(np.float64), mod, bias, idx, 1e-6), 1e-12,
           "fp8 AdaLN exact weights vs folded AdaLN")
    a = o.adaln_norm_proj_fold(x, Wf.astype(np.float64), mod, bias, idx, 1e-6)
    b = o.adaln_norm_proj_fold(x, Wf[::-1].astype(np.float64), mod, bias_u, idx, 1e-6)
    _close(o.adaln_norm_proj_swiglu_fp8(x, codes, s, codes_u, s_u, mod, bias, bias_u, idx, 1e-6),
           a / (1 + np.exp(-a)) * b, 1e-12, "fp8 AdaLN SwiGLU exact weights")
    ones, zb = np.ones((T, K)), np.zeros((T, N))
    _close(o.adaln_norm_proj_fp8(x, codes, s, ones, zb, idx, 1e-6), o.norm_proj_fp8(x, codes, s, 1e-6), 1e-14,
           "a table of ones and zero bias give the plain fp8 path")
    # brute force, arbitrary weights
    Wr = rng.standard_normal((5, 3)).astype(np.float32)
    c2, s2, _ = o.quantize_e4m3_columns(Wr)
    xs, ms, bs, ids = x[:2, :5], mod[:, :5], bias[:, :3], np.array([2, 0])
    got = o.adaln_norm_proj_fp8(xs, c2, s2, ms, bs, ids, 0.25)
    for m in range(2):
        rr = math.sqrt(sum(float(v) ** 2 for v in xs[m]) / 5 + float(np.float32(0.25)))
        for n in range(3):
            acc = 0.0
            for k in range(5):
                w = float(o.e4m3_decode(np.array([c2[k, n]]))[0]) * float(s2[n])
                acc += float(xs[m, k]) * float(ms[ids[m], k]) * w
            want = acc / rr + float(bs[ids[m], n])
            assert abs(got[m, n] - want) <= 1e-12 * (abs(want) + 1), (m, n, got[m, n], want)


ALL_CHECKS += [check_adaln_fp8]


def check_adaln_q8(o, seed=27):
    """AdaLN with fp8 row-block output: the values quantised are the SwiGLU
    output of the definition (bf16 weights) or of the fp8 AdaLN form (E4M3
    weights), and the codes and scales are quantize_e4m3_row_blocks of
    them; with E4M3-exact weights and the unrounded table the fp8 form's
    values are the definition's."""
    rng = np.random.default_rng(seed)
    M, K, N, T = 5, 32, 40, 3
    x = o.round_to_bf16(rng.standard_normal((M, K)))
    g = o.round_to_bf16(rng.uniform(0.5, 1.5, K))
    Wg = o.round_to_bf16(rng.standard_normal((K, N)) / 4)
    Wu = o.round_to_bf16(rng.standard_normal((K, N)) / 4)
    sc = o.round_to_bf16(rng.standard_normal((T, K)) * 0.3)
    sh = o.round_to_bf16(rng.standard_normal((T, K)) * 0.3)
    idx = rng.integers(0, T, M)
    c, s, v = o.adaln_norm_proj_swiglu_q8(x, g, sc, sh, idx, Wg, Wu, 1e-6)
    assert np.array_equal(v, o.adaln_norm_proj_swiglu(x, g, sc, sh, idx, Wg, Wu, 1e-6)), "values of the definition"
    c2, s2 = o.quantize_e4m3_row_blocks(v)
    assert np.array_equal(c, c2) and np.array_equal(s, s2)
    pool = o.e4m3_decode(np.arange(0, 0x7F, dtype=np.uint8))
    pick = rng.choice(pool, size=(K, N)) * rng.choice([-1.0, 1.0], size=(K, N))
    pick[0, :] = 448.0
    W8 = pick * np.ldexp(1.0, -6)
    cg, sg, _ = o.quantize_e4m3_columns(W8.astype(np.float32))
    cu, su, _ = o.quantize_e4m3_columns(W8[::-1].astype(np.float32).copy())
    mod = g[None, :] * (1 + sc)
    bg, bu = sh @ W8, sh @ W8[::-1]
    c8, s8, v8 = o.adaln_norm_proj_swiglu_fp8_q8(x, cg, sg, cu, su, mod, bg, bu, idx, 1e-6)
    assert np.array_equal(v8, o.adaln_norm_proj_swiglu_fp8(x, cg, sg, cu, su, mod, bg, bu, idx, 1e-6))
    c3, s3 = o.quantize_e4m3_row_blocks(v8)
    assert np.array_equal(c8, c3) and np.array_equal(s8, s3)
    _close(v8, o.adaln_norm_proj_swiglu(x, g, sc, sh, idx, W8, W8[::-1], 1e-6), 1e-12,
           "fp8-weight AdaLN q8 values vs the definition on E4M3-exact weights")


ALL_CHECKS += [check_adaln_q8]
