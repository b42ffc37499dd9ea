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
                    s_rtol: float = 1e-4, max_flip_frac: float = 1e-3):
    """fp8 row-block output (codes [M,N] uint8, scales [M,nb] fp32, from the
    GPU) against the oracle's quantisation of the float64 reference v_ref.
    Scales agree to s_rtol (the block maximum of the GPU's fp32 values);
    codes agree exactly except where the reference's scaled value lies
    within `margin` quanta, or within v_atol * (block maximum) before
    scaling (the absolute error of an fp32 dot product over K terms), of a
    rounding midpoint: there the GPU may take the neighbouring code.  At most
    max_flip_frac of the codes may do so."""
    import oracle
    codes = np.asarray(codes, dtype=np.uint8)
    scales = np.asarray(scales, dtype=np.float64)
    ref_codes, ref_s = oracle.quantize_e4m3_row_blocks(v_ref)
    ref_s = ref_s.astype(np.float64)
    assert codes.shape == ref_codes.shape and scales.shape == ref_s.shape, f"{what}: shapes"
    nan_rows = np.isnan(ref_s)
    assert np.array_equal(np.isnan(scales), nan_rows), f"{what}: NaN scales differ"
    ok = ~nan_rows
    assert np.all(np.abs(scales[ok] - ref_s[ok]) <= s_rtol * ref_s[ok]), \
        f"{what}: scales differ by {np.max(np.abs(scales[ok] - ref_s[ok]) / ref_s[ok]):.3e} relative"
    diff = codes != ref_codes
    if not diff.any():
        return 0
    m_idx, n_idx = np.nonzero(diff)
    blk = n_idx // 16
    r = np.float32(448.0) / np.maximum(ref_s[m_idx, blk] * 448.0, 1e-300)
    u = np.abs(np.asarray(v_ref, dtype=np.float32)[m_idx, n_idx].astype(np.float64) * r)
    _, e = np.frexp(np.maximum(u, 1e-300))
    quantum = np.ldexp(1.0, np.maximum(e, -5) - 4)
    frac = u / quantum - np.floor(u / quantum)
    near = np.abs(frac - 0.5) * quantum <= margin * quantum + v_atol * 448.0
    dg = oracle.e4m3_decode(codes[m_idx, n_idx])
    dr = oracle.e4m3_decode(ref_codes[m_idx, n_idx])
    neighbour = ((codes[m_idx, n_idx] & 0x80) == (ref_codes[m_idx, n_idx] & 0x80)) & \
        (np.abs(codes[m_idx, n_idx].astype(int) - ref_codes[m_idx, n_idx].astype(int)) == 1)
    both_zero = (dg == 0) & (dr == 0)
    bad = ~(both_zero | (near & neighbour))
    assert not bad.any(), (f"{what}: {bad.sum()} codes differ away from a rounding midpoint, first at "
                           f"{(m_idx[bad][0], n_idx[bad][0])}: {codes[m_idx[bad][0], n_idx[bad][0]]:#x} vs "
                           f"{ref_codes[m_idx[bad][0], n_idx[bad][0]]:#x}")
    assert diff.sum() <= max(2, max_flip_frac * diff.size), f"{what}: {diff.sum()} codes at midpoints"
    return int(diff.sum())
