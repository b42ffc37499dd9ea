"""Helpers shared by the GPU parity tests: device transfer, host-side packing
of folded weights (layout from include/flashnorm.h), and the tolerance rule."""
from __future__ import annotations

import numpy as np

# Tolerances: max |gpu - oracle| <= TOL * (|oracle| + 1), elementwise.
TOL = {"bf16": 2e-2, "f32": 1e-5}


def tdtype(dtype: str):
    import torch
    return {"bf16": torch.bfloat16, "f32": torch.float32}[dtype]


def to_dev(a: np.ndarray, dtype: str):
    """Storage-exact numpy values -> device tensor of the storage dtype."""
    import torch
    return torch.from_numpy(np.ascontiguousarray(a, dtype=np.float32)).to(tdtype(dtype)).cuda()


def to_f64(t) -> np.ndarray:
    import torch
    return t.detach().to(torch.float64).cpu().numpy()


def max_rel_err(got: np.ndarray, ref: np.ndarray) -> float:
    got = np.asarray(got, dtype=np.float64)
    ref = np.asarray(ref, dtype=np.float64)
    if got.size == 0:
        return 0.0
    return float(np.max(np.abs(got - ref) / (np.abs(ref) + 1.0)))


def assert_close(got, ref, dtype: str, what: str = ""):
    got = np.asarray(got, dtype=np.float64)
    ref = np.asarray(ref, dtype=np.float64)
    assert got.shape == ref.shape, f"{what}: shape {got.shape} vs {ref.shape}"
    assert np.all(np.isfinite(got)), f"{what}: non-finite outputs"
    err = max_rel_err(got, ref)
    assert err <= TOL[dtype], f"{what}: max |err|/(|ref|+1) = {err:.3e} > {TOL[dtype]:.0e}"
    return err


def stale_failures(outs, refs):
    """The staleness check: every output must match its own input's oracle
    within the tolerance, and differ from the previous call's oracle by more
    than the tolerance (so a one-step-stale result is caught: the failure
    mode of the two-stream FlashNorm bug).  Returns the failures."""
    bad = []
    for t, (got, ref) in enumerate(zip(outs, refs)):
        err = np.max(np.abs(got - ref) / (np.abs(ref) + 1.0))
        if not (np.all(np.isfinite(got)) and err <= TOL["bf16"]):
            bad.append(f"call {t}: max |err|/(|ref|+1) = {err:.3e}")
        if t > 0:
            stale = np.max(np.abs(got - refs[t - 1]) / (np.abs(refs[t - 1]) + 1.0))
            if not stale > TOL["bf16"]:
                bad.append(f"call {t} indistinguishable from call {t - 1}")
    return bad


def storage_bits(values: np.ndarray, dtype: str) -> np.ndarray:
    """Bit patterns of storage-exact values."""
    f = np.ascontiguousarray(values, dtype=np.float32)
    u = f.view(np.uint32)
    if dtype == "f32":
        return u
    assert np.all((u & 0xFFFF) == 0), "values are not bf16-exact"
    return (u >> 16).astype(np.uint16)


def pack_host(W_store: np.ndarray, dtype: str) -> np.ndarray:
    """Packed fragment layout of a [K,N] matrix of storage values, as raw
    bytes: element (k, n) at fragment (n//16, k//KB), lane ((k%KB)//V)*16 +
    n%16, slot k%V; padding zero."""
    K, N = W_store.shape
    e = 4 if dtype == "f32" else 2
    V = 16 // e
    KB = 4 * V
    kbl = -(-K // KB)
    nbl = -(-N // 16)
    bits = storage_bits(W_store, dtype)
    pad = np.zeros((kbl * KB, nbl * 16), dtype=bits.dtype)
    pad[:K, :N] = bits
    # [kb, grp, v, nb, j] -> [nb, kb, grp, j, v]
    p = pad.reshape(kbl, 4, V, nbl, 16).transpose(3, 0, 1, 4, 2)
    return np.ascontiguousarray(p).view(np.uint8).reshape(-1)


def pack_fp8_host(codes: np.ndarray) -> np.ndarray:
    """Packed fp8 layout of a [K,N] matrix of E4M3 codes, as raw bytes: code
    (k, n) at fragment (n//16, k//64), lane ((k%32)//8)*16 + n%16, byte
    (k%64 >= 32)*8 + k%8; padding zero."""
    K, N = codes.shape
    kp = -(-K // 64)
    nbl = -(-N // 16)
    pad = np.zeros((kp * 64, nbl * 16), dtype=np.uint8)
    pad[:K, :N] = codes
    # k = ((kp*2 + h)*4 + grp)*8 + j, n = nb*16 + c -> [nb, kp, grp, c, h, j]
    p = pad.reshape(kp, 2, 4, 8, nbl, 16).transpose(4, 0, 2, 5, 1, 3)
    return np.ascontiguousarray(p).reshape(-1)


def assert_q8_close(codes, scales, v_ref, what: str, margin: float = 0.02, v_atol: float = 1e-5,
                    s_rtol: float = 1e-4, max_flip_frac: float = 1e-3, v_err=None):
    """fp8 row-block output (codes [M,N] uint8, scales [M,nb] fp32, from the
    GPU) against the oracle's quantisation of the float64 reference v_ref.
    Scales agree to s_rtol (the block maximum of the GPU's fp32 values);
    codes agree exactly except where the reference's scaled value lies
    within `margin` quanta, or within v_atol * (block maximum) before
    scaling (the absolute error of an fp32 dot product over K terms), of a
    rounding midpoint: there the GPU may take the neighbouring code.  At most
    max_flip_frac of the codes may do so.

    v_err (per-element bound on |GPU value - v_ref| before quantisation,
    from the kernel's arithmetic): the scales may then also differ by the
    block's largest v_err / 448, and a differing code must be a correct
    rounding of some value within v_err of the reference -- its value read
    back with the GPU's scale lies within v_err plus half an E4M3 step of
    v_ref -- however many such codes there are."""
    import oracle
    codes = np.asarray(codes, dtype=np.uint8)
    scales = np.asarray(scales, dtype=np.float64)
    ref_codes, ref_s = oracle.quantize_e4m3_row_blocks(v_ref)
    ref_s = ref_s.astype(np.float64)
    assert codes.shape == ref_codes.shape and scales.shape == ref_s.shape, f"{what}: shapes"
    M, N = codes.shape
    nb = ref_s.shape[1]
    if v_err is not None:
        v_err = np.broadcast_to(np.asarray(v_err, np.float64), (M, N))
        pad = np.zeros((M, nb * 16))
        pad[:, :N] = v_err
        blk_err = pad.reshape(M, nb, 16).max(axis=2)
    else:
        blk_err = np.zeros_like(ref_s)
    nan_rows = np.isnan(ref_s)
    assert np.array_equal(np.isnan(scales), nan_rows), f"{what}: NaN scales differ"
    ok = ~nan_rows
    s_tol = s_rtol * ref_s + blk_err / 448.0 * (1 + 1e-6)
    assert np.all(np.abs(scales[ok] - ref_s[ok]) <= s_tol[ok]), \
        f"{what}: scales differ by {np.max(np.abs(scales[ok] - ref_s[ok]) / ref_s[ok]):.3e} relative"
    diff = codes != ref_codes
    if not diff.any():
        return 0
    m_idx, n_idx = np.nonzero(diff)
    blk = n_idx // 16
    dg = oracle.e4m3_decode(codes[m_idx, n_idx])
    dr = oracle.e4m3_decode(ref_codes[m_idx, n_idx])
    both_zero = (dg == 0) & (dr == 0)
    if v_err is not None:
        _, e = np.frexp(np.maximum(np.abs(dg), 2.0 ** -6))     # |dg| in [2^(e-1), 2^e)
        half_step = np.ldexp(1.0, e - 5)                        # half the E4M3 step of that binade
        sg = scales[m_idx, blk]
        vr = np.asarray(v_ref, np.float64)[m_idx, n_idx]
        close = np.abs(dg * sg - vr) <= v_err[m_idx, n_idx] + half_step * sg * (1 + 1e-6) + 1e-30
        bad = ~(both_zero | close)
        assert not bad.any(), (f"{what}: {bad.sum()} codes are no rounding of a value within the derived error, "
                               f"first at {(m_idx[bad][0], n_idx[bad][0])}: {codes[m_idx[bad][0], n_idx[bad][0]]:#x} "
                               f"vs {ref_codes[m_idx[bad][0], n_idx[bad][0]]:#x}")
        return int(diff.sum())
    r = np.float32(448.0) / np.maximum(ref_s[m_idx, blk] * 448.0, 1e-300)
    u = np.abs(np.asarray(v_ref, dtype=np.float32)[m_idx, n_idx].astype(np.float64) * r)
    _, e = np.frexp(np.maximum(u, 1e-300))
    quantum = np.ldexp(1.0, np.maximum(e, -5) - 4)
    frac = u / quantum - np.floor(u / quantum)
    near = np.abs(frac - 0.5) * quantum <= margin * quantum + v_atol * 448.0
    neighbour = ((codes[m_idx, n_idx] & 0x80) == (ref_codes[m_idx, n_idx] & 0x80)) & \
        (np.abs(codes[m_idx, n_idx].astype(int) - ref_codes[m_idx, n_idx].astype(int)) == 1)
    bad = ~(both_zero | (near & neighbour))
    assert not bad.any(), (f"{what}: {bad.sum()} codes differ away from a rounding midpoint, first at "
                           f"{(m_idx[bad][0], n_idx[bad][0])}: {codes[m_idx[bad][0], n_idx[bad][0]]:#x} vs "
                           f"{ref_codes[m_idx[bad][0], n_idx[bad][0]]:#x}")
    assert diff.sum() <= max(2, max_flip_frac * diff.size), f"{what}: {diff.sum()} codes at midpoints"
    return int(diff.sum())


# ---------------------------------------------------------------- AdaLN --
def _rows_or_zero(table, idx):
    from oracle.flashnorm_oracle import _rows_or_zero as rows
    return rows(table, idx)


def idx_dev(idx):
    import torch
    return torch.from_numpy(np.ascontiguousarray(idx, dtype=np.int32)).cuda()


class AdalnCase:
    """Seeded AdaLN inputs on the host (storage-exact numpy values) and on
    the device in the library's offline forms: the gain folded into the
    fp32 modulation table, the plain weights packed (or quantised to E4M3),
    the bias rows shift @ W.  Indices outside [0, T) are planted in the first
    and last row when bad_idx is set; the oracle's definition then sees an
    extra table row with scale -1 and shift 0 (h = 0 for that row)."""

    def __init__(self, fn, M, K, N, T, swiglu, seed, bad_idx=False, weights="bf16"):
        import workloads as Wl
        self.M, self.K, self.N, self.T, self.swiglu, self.weights = M, K, N, T, swiglu, weights
        self.inp = Wl.random_inputs(M, K, N, "bf16", seed=seed, swiglu=swiglu)
        self.scale, self.shift, self.idx = Wl.adaln_tables(T, K, M, seed=seed + 1)
        if bad_idx and M >= 3:
            self.idx[0], self.idx[-1] = -1, T
        self.eps = self.inp.call.eps
        # the definition's view: an extra row for the indices outside the table
        self.scale1 = np.vstack([self.scale, -np.ones((1, K), np.float32)])
        self.shift1 = np.vstack([self.shift, np.zeros((1, K), np.float32)])
        self.idx1 = np.where((self.idx < 0) | (self.idx >= T), T, self.idx)
        self.x = to_dev(self.inp.x, "bf16")
        g = to_dev(self.inp.g, "bf16")
        sc, sh = to_dev(self.scale, "bf16"), to_dev(self.shift, "bf16")
        self.mod = fn.adaln_fold_table(g, sc)
        self.idx_d = idx_dev(self.idx)
        mats = [self.inp.W] + ([self.inp.W_up] if swiglu else [])
        self.Wp, self.bias = [], []
        for Wm in mats:
            Wd = to_dev(Wm, "bf16")
            self.Wp.append(fn.fold_weights(None, Wd) if weights == "bf16" else fn.fold_weights_fp8(None, Wd))
            self.bias.append(fn.adaln_shift_bias(sh, Wd))

    def args(self):
        """Positional arguments after x of the library calls."""
        if self.swiglu:
            return (self.mod, self.idx_d, self.Wp[0], self.bias[0], self.Wp[1], self.bias[1])
        return (self.mod, self.idx_d, self.Wp[0], self.bias[0])

    def mod_host(self):
        import oracle
        return oracle.adaln_fold_table(self.inp.g, self.scale)

    def reference(self, rows=None):
        """float64 oracle: the definition for bf16 weights, the fp8 AdaLN
        form on the E4M3 codes for fp8 weights; rows: a subset of x rows."""
        import oracle
        pick = slice(None) if rows is None else rows
        x, idx1, idx = self.inp.x[pick], self.idx1[pick], self.idx[pick]
        if self.weights == "bf16":
            if self.swiglu:
                return oracle.adaln_norm_proj_swiglu(x, self.inp.g, self.scale1, self.shift1, idx1, self.inp.W,
                                                     self.inp.W_up, self.eps)
            return oracle.adaln_norm_proj(x, self.inp.g, self.scale1, self.shift1, idx1, self.inp.W, self.eps)
        mod = self.mod_host()
        ones = np.ones(self.K)
        cg, sg = oracle.fold_weights_fp8(ones, self.inp.W, "bf16")
        bg = oracle.adaln_shift_bias(self.shift, self.inp.W)
        if self.swiglu:
            cu, su = oracle.fold_weights_fp8(ones, self.inp.W_up, "bf16")
            bu = oracle.adaln_shift_bias(self.shift, self.inp.W_up)
            return oracle.adaln_norm_proj_swiglu_fp8(x, cg, sg, cu, su, mod, bg, bu, idx, self.eps)
        return oracle.adaln_norm_proj_fp8(x, cg, sg, mod, bg, idx, self.eps)

    def value_error_bound(self, rows=None, split=None):
        """Per-element bound on |kernel value - reference| before the output
        rounding, from the arithmetic: the bf16 operand x * mod rounded once
        is within 2^-8 of its value (relative: an 8-bit significand rounded
        to nearest; split in two bf16 parts, 2^-16), the
        weights are exact (bf16, or E4M3 codes decoded exactly), sums are
        fp32 (1e-5 of the sum of magnitudes), and the table itself is an fp32
        rounding of g * (1 + scale) (2^-24).  SwiGLU propagates the bounds on
        a and b by |silu'(a)| |b| E_a + |silu(a)| E_b + E_a E_b."""
        import oracle
        pick = slice(None) if rows is None else rows
        split = self.swiglu if split is None else split
        x = np.asarray(self.inp.x[pick], np.float64)
        idx = self.idx[pick]
        mod = _rows_or_zero(self.mod_host(), idx)
        r = oracle.rms(x, self.eps)[:, None]
        xm = np.abs(x * mod)
        ones = np.ones(self.K)
        rel = (2.0 ** -16 if split else 2.0 ** -8) + 2.0 ** -23 + 1e-5

        def err(Wm):
            if self.weights == "bf16":
                Wa = np.abs(np.asarray(Wm, np.float64))
            else:
                c, s = oracle.fold_weights_fp8(ones, Wm, "bf16")
                Wa = np.abs(oracle.e4m3_decode(c) * np.asarray(s, np.float64)[None, :])
            sh = np.abs(_rows_or_zero(self.shift, idx)) @ np.abs(np.asarray(Wm, np.float64))
            return rel * (xm @ Wa) / r + 1e-5 * sh + 1e-6

        Ea = err(self.inp.W)
        if not self.swiglu:
            return Ea
        ref_a = self._proj(self.inp.W, pick)
        ref_b = self._proj(self.inp.W_up, pick)
        Eb = err(self.inp.W_up)
        sig = 1.0 / (1.0 + np.exp(-ref_a))
        dsilu = sig * (1.0 + ref_a * (1.0 - sig))
        return np.abs(dsilu) * np.abs(ref_b) * Ea + np.abs(ref_a * sig) * Eb + Ea * Eb + 1e-6

    def _proj(self, Wm, pick):
        import oracle
        if self.weights == "bf16":
            return oracle.adaln_norm_proj(self.inp.x[pick], self.inp.g, self.scale1, self.shift1, self.idx1[pick], Wm,
                                          self.eps)
        c, s = oracle.fold_weights_fp8(np.ones(self.K), Wm, "bf16")
        return oracle.adaln_norm_proj_fp8(self.inp.x[pick], c, s, self.mod_host(), oracle.adaln_shift_bias(
            self.shift, Wm), self.idx[pick], self.eps)


def assert_adaln_close(y, ref, value_err, what):
    """Every output within the tolerance rule (2e-2 (|ref| + 1)) and within
    the bound derived from the arithmetic plus the bf16 output rounding."""
    y = np.asarray(y, np.float64)
    assert y.shape == ref.shape and np.all(np.isfinite(y)), what
    bound = value_err + 2.0 ** -8 * np.abs(ref)
    bad = np.abs(y - ref) > bound
    assert not bad.any(), (f"{what}: {bad.sum()} outputs outside the derived bound, worst "
                           f"{np.max(np.abs(y - ref) / bound):.2f}x")
    return assert_close(y, ref, "bf16", what)
