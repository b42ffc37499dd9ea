"""Seeded synthetic inputs for fused RMSNorm + projection.

This module is shared by the oracle-side tests and by the HIP path's tests and
benchmark.  It holds input generation only: random draws, the storage-dtype
rounding of those draws, and the table of workload shapes.  None of the
normalisation, projection, folding or SwiGLU arithmetic lives here.

Every array is returned as a numpy ``float32`` array whose values are exactly
representable in the workload's storage dtype (bf16 values are a subset of
float32), so the oracle can up-cast it to float64 exactly and the GPU side can
cast it to its storage dtype without a second rounding.

Recipe (applies to every workload):
  * generator: ``numpy.random.default_rng(seed)`` (PCG64);
  * draw order: x, then outlier channel indices (if any), then g, then W
    (then W_up for the gate/up pair);
  * x ~ N(0, 1); g ~ U(0.5, 1.5); W ~ N(0, 1/K); all drawn in float32;
  * outlier channels: round(fraction * K) distinct channel indices drawn
    without replacement; those columns of x are multiplied by the factor;
  * bf16 workloads: each array is rounded to bf16 with round-to-nearest-even
    (torch's CPU conversion) after drawing;
  * eps = 1e-6.
"""
from __future__ import annotations

import dataclasses
from typing import Dict, List, Optional, Tuple

import numpy as np

EPS = 1e-6


@dataclasses.dataclass(frozen=True)
class Call:
    """One fused call: x[M,K] normalised and projected by one matrix [K,N]
    (``swiglu=False``) or by a gate/up pair of [K,N] matrices (``swiglu=True``)."""
    name: str
    M: int
    K: int
    N: int
    swiglu: bool
    dtype: str          # "f32" or "bf16"
    seed: int
    outlier_fraction: float = 0.0
    outlier_factor: float = 1.0
    eps: float = EPS

    @property
    def mats(self) -> int:
        return 2 if self.swiglu else 1

    @property
    def elem_bytes(self) -> int:
        return 4 if self.dtype == "f32" else 2

    def algorithmic_bytes(self) -> int:
        """W' read once, x read once, y written once (g is folded away)."""
        e = self.elem_bytes
        return e * (self.mats * self.K * self.N + self.M * self.K + self.M * self.N)

    def flops(self) -> int:
        return 2 * self.M * self.K * self.N * self.mats


@dataclasses.dataclass
class Inputs:
    call: Call
    x: np.ndarray                 # [M, K]
    g: np.ndarray                 # [K]
    W: np.ndarray                 # [K, N]
    W_up: Optional[np.ndarray]    # [K, N] for the SwiGLU pair, else None
    outlier_channels: Optional[np.ndarray] = None


# Workload table.  Shapes follow Llama-7B-class layers: hidden 4096, fused
# QKV 3*4096, FFN 11008, vocabulary 32000.
TINY = Call("tiny decode x[4,256] f32, W[256,768]", 4, 256, 768, False, "f32", 1)
QKV_DECODE = Call("QKV decode x[16,4096] bf16 (1% outlier channels x20), W[4096,12288]",
                  16, 4096, 12288, False, "bf16", 2,
                  outlier_fraction=0.01, outlier_factor=20.0)
FFN_DECODE = Call("FFN gate/up SwiGLU decode x[64,4096] bf16, W_gate,W_up[4096,11008]",
                  64, 4096, 11008, True, "bf16", 3)
PREFILL_QKV = Call("prefill QKV x[4096,4096] bf16, W[4096,12288]",
                   4096, 4096, 12288, False, "bf16", 4)

DECODE_STEP_LAYERS = 32
DECODE_STEP_M = 8


def decode_step_calls(layers: int = DECODE_STEP_LAYERS, rows: int = DECODE_STEP_M, shard: int = 1) -> List[Call]:
    """The 32-layer decode step at M=8 (``rows`` other batch sizes): per
    layer an attention norm + QKV projection and an FFN norm + gate/up
    SwiGLU; then the final norm + LM head.  Every call gets its own seeded x
    (calls are independent, not chained).  ``shard`` > 1: one GPU's column
    share of every projection under tensor parallelism over that many GPUs
    (N / shard columns, the full x)."""
    if shard < 1 or any(n % (16 * shard) for n in (12288, 11008, 32000)):
        raise ValueError(f"shard={shard} must split every projection into 16-column blocks")
    calls: List[Call] = []
    for l in range(layers):
        calls.append(Call(f"layer{l}.attn_qkv", rows, 4096, 12288 // shard, False, "bf16", 5000 + 2 * l))
        calls.append(Call(f"layer{l}.ffn_gate_up", rows, 4096, 11008 // shard, True, "bf16", 5001 + 2 * l))
    calls.append(Call("head", rows, 4096, 32000 // shard, False, "bf16", 5064))
    return calls


WORKLOADS: Dict[str, Call] = {
    "tiny": TINY,
    "qkv_decode": QKV_DECODE,
    "ffn_decode": FFN_DECODE,
    "prefill_qkv": PREFILL_QKV,
}


def _to_storage(a: np.ndarray, dtype: str) -> np.ndarray:
    a = np.ascontiguousarray(a, dtype=np.float32)
    if dtype == "f32":
        return a
    if dtype == "bf16":
        import torch  # CPU conversion only; round-to-nearest-even
        return torch.from_numpy(a).to(torch.bfloat16).to(torch.float32).numpy()
    raise ValueError(f"unknown dtype {dtype!r}")


def make_inputs(call: Call, seed: Optional[int] = None) -> Inputs:
    """Draw the inputs of ``call`` with the recipe in the module docstring."""
    rng = np.random.default_rng(call.seed if seed is None else seed)
    M, K, N = call.M, call.K, call.N
    x = rng.standard_normal((M, K), dtype=np.float32)
    outliers = None
    if call.outlier_fraction > 0:
        n_out = int(round(call.outlier_fraction * K))
        outliers = np.sort(rng.choice(K, size=n_out, replace=False))
        x[:, outliers] *= np.float32(call.outlier_factor)
    g = rng.uniform(0.5, 1.5, size=K).astype(np.float32)
    std = np.float32(1.0 / np.sqrt(K))
    W = rng.standard_normal((K, N), dtype=np.float32) * std
    W_up = None
    if call.swiglu:
        W_up = rng.standard_normal((K, N), dtype=np.float32) * std
    return Inputs(call,
                  _to_storage(x, call.dtype),
                  _to_storage(g, call.dtype),
                  _to_storage(W, call.dtype),
                  None if W_up is None else _to_storage(W_up, call.dtype),
                  outliers)


def random_inputs(M: int, K: int, N: int, dtype: str, seed: int, swiglu: bool = False,
                  eps: float = EPS) -> Inputs:
    """Same recipe at an arbitrary shape (ragged and edge-case tests)."""
    return make_inputs(Call(f"random M={M} K={K} N={N}", M, K, N, swiglu, dtype, seed, eps=eps))


def make_x(M: int, K: int, dtype: str, seed: int) -> np.ndarray:
    """A fresh activation batch only (used for back-to-back call sequences)."""
    rng = np.random.default_rng(seed)
    return _to_storage(rng.standard_normal((M, K), dtype=np.float32), dtype)


def make_inputs_device(call: Call, device="cuda"):
    """The same distributions drawn by torch's generator on the device, for
    benchmark-only inputs too large to draw on the host quickly (the 32-layer
    decode step holds 9.3 GB of weights).  Seeded by ``call.seed``; values
    differ from make_inputs (different generator) and are rounded to bf16 by
    torch's round-to-nearest-even conversion.  Returns (x, g, W, W_up)
    tensors of the storage dtype."""
    import torch
    tdt = torch.bfloat16 if call.dtype == "bf16" else torch.float32
    gen = torch.Generator(device=device)
    gen.manual_seed(call.seed)
    M, K, N = call.M, call.K, call.N
    x = torch.randn((M, K), generator=gen, device=device, dtype=torch.float32)
    if call.outlier_fraction > 0:
        n_out = int(round(call.outlier_fraction * K))
        idx = torch.randperm(K, generator=gen, device=device)[:n_out]
        x[:, idx] *= call.outlier_factor
    g = torch.rand((K,), generator=gen, device=device, dtype=torch.float32) + 0.5
    std = 1.0 / float(np.sqrt(K))
    W = torch.randn((K, N), generator=gen, device=device, dtype=torch.float32).mul_(std).to(tdt)
    W_up = None
    if call.swiglu:
        W_up = torch.randn((K, N), generator=gen, device=device, dtype=torch.float32).mul_(std).to(tdt)
    return x.to(tdt), g.to(tdt), W, W_up


def adaln_tables(T: int, K: int, M: int, seed: int, dtype: str = "bf16"):
    """AdaLN inputs of the same family: scale and shift tables [T, K] drawn
    N(0, 0.3^2) and rounded to the storage dtype, and a table row per x row
    (uniform in [0, T)).  Returns (scale, shift, idx int32)."""
    rng = np.random.default_rng(seed)
    scale = _to_storage(rng.standard_normal((T, K), dtype=np.float32) * np.float32(0.3), dtype)
    shift = _to_storage(rng.standard_normal((T, K), dtype=np.float32) * np.float32(0.3), dtype)
    idx = rng.integers(0, T, M).astype(np.int32)
    return scale, shift, idx


def sample_indices(n: int, count: int, seed: int) -> np.ndarray:
    """Seeded sorted subset of range(n), always including the first and last index."""
    if count >= n:
        return np.arange(n)
    rng = np.random.default_rng(seed)
    mid = rng.choice(np.arange(1, n - 1), size=max(count - 2, 0), replace=False)
    return np.unique(np.concatenate([[0, n - 1], mid]))


__all__ = ["Call", "Inputs", "EPS", "TINY", "QKV_DECODE", "FFN_DECODE", "PREFILL_QKV",
           "WORKLOADS", "decode_step_calls", "make_inputs", "make_inputs_device", "random_inputs", "make_x",
           "sample_indices", "DECODE_STEP_LAYERS", "DECODE_STEP_M", "adaln_tables"]
