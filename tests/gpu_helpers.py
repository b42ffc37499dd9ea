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
