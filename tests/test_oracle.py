"""The float64 oracle against its pins (CPU only)."""
import numpy as np
import pytest

import oracle.flashnorm_oracle as O
from tests import oracle_pins as P


@pytest.mark.parametrize("check", P.ALL_CHECKS, ids=lambda c: c.__name__)
def test_oracle_pin(check):
    check(O)


def _K(x):
    return np.asarray(x).shape[-1]


# Plausible mistakes, planted in the oracle module; every one must be caught
# by at least one pin.
MUTANTS = {
    "eps outside the root": ("rms", lambda x, eps: np.sqrt(np.sum(np.asarray(x, float) ** 2, -1) / _K(x)) + eps),
    "mean over K-1": ("rms", lambda x, eps: np.sqrt(np.sum(np.asarray(x, float) ** 2, -1) / (_K(x) - 1) + eps)),
    "eps dropped": ("rms", lambda x, eps: np.sqrt(np.sum(np.asarray(x, float) ** 2, -1) / _K(x))),
    "root dropped": ("rms", lambda x, eps: np.sum(np.asarray(x, float) ** 2, -1) / _K(x) + eps),
    "gain dropped": ("rmsnorm", lambda x, g, eps: np.asarray(x, float) / O.rms(x, eps)[..., None]),
    "multiply by r": ("rmsnorm", lambda x, g, eps: np.asarray(x, float) * O.rms(x, eps)[..., None] * g),
    "gain reversed": ("rmsnorm", lambda x, g, eps: np.asarray(x, float) / O.rms(x, eps)[..., None]
                      * np.asarray(g, float)[::-1]),
    "W transposed": ("norm_proj", lambda x, g, W, eps: O.rmsnorm(x, g, eps) @ np.asarray(W, float).T),
    "sigmoid sign": ("silu", lambda a: np.asarray(a, float) / (1.0 + np.exp(np.asarray(a, float)))),
    "gate/up swapped": ("norm_proj_swiglu", lambda x, g, Wg, Wu, eps:
                        O.silu(O.rmsnorm(x, g, eps) @ np.asarray(Wu, float))
                        * (O.rmsnorm(x, g, eps) @ np.asarray(Wg, float))),
    "up not normalised": ("norm_proj_swiglu", lambda x, g, Wg, Wu, eps:
                          O.silu(O.rmsnorm(x, g, eps) @ np.asarray(Wg, float))
                          * ((np.asarray(x, float) * g) @ np.asarray(Wu, float))),
    "scale after silu": ("norm_proj_swiglu", lambda x, g, Wg, Wu, eps:
                         O.silu((np.asarray(x, float) * g) @ np.asarray(Wg, float))
                         * (O.rmsnorm(x, g, eps) @ np.asarray(Wu, float))),
    "bf16 truncation": ("round_to_bf16", lambda a: np.trunc(np.ldexp(np.asarray(a, float),
                        8 - np.maximum(np.frexp(np.asarray(a, float))[1], -125)))
                        * np.ldexp(1.0, np.maximum(np.frexp(np.asarray(a, float))[1], -125) - 8)),
    "bf16 ties away": ("round_to_bf16", lambda a: np.sign(a) * np.floor(np.ldexp(np.abs(np.asarray(a, float)),
                       8 - np.maximum(np.frexp(np.asarray(a, float))[1], -125)) + 0.5)
                       * np.ldexp(1.0, np.maximum(np.frexp(np.asarray(a, float))[1], -125) - 8)),
    "fold on the output axis": ("fold_exact", lambda g, W: np.asarray(W, float) * np.asarray(g, float)[None, :]),
    "deferred multiply": ("norm_proj_folded", lambda x, Wf, eps: (np.asarray(x, float) @ np.asarray(Wf, float))
                          * O.rms(x, eps)[:, None]),
    "e4m3 ties away": ("e4m3_encode", lambda a: _encode_with(a, lambda v: np.floor(v + 0.5))),
    "e4m3 truncation": ("e4m3_encode", lambda a: _encode_with(a, np.floor)),
    "e4m3 bias 8": ("e4m3_decode", lambda c: _decode_bias(c, 8)),
    "fp8 scale dropped": ("norm_proj_fp8", lambda x, c, s, eps: (np.asarray(x, float) @ O.e4m3_decode(c))
                          / O.rms(x, eps)[:, None]),
    "fp8 scale inverted": ("norm_proj_fp8", lambda x, c, s, eps: (np.asarray(x, float) @ O.e4m3_decode(c))
                           / np.asarray(s, float)[None, :] / O.rms(x, eps)[:, None]),
    "fp8 scale per row": ("quantize_e4m3_columns", lambda W: _quantize_rows(W)),
    "q8 blocks down the columns": ("quantize_e4m3_row_blocks", lambda v, block=16: _q8_columns(v, block)),
    "q8 block of 32": ("quantize_e4m3_row_blocks", lambda v, block=16: _q8_ref(v, 32)),
    "q8 blocks across rows": ("quantize_e4m3_row_blocks", lambda v, block=16: _q8_flat(v, block)),
    "adaln modulation before the norm": ("adaln_modulate", lambda x, g, sc, sh, idx, eps: O.rmsnorm(
        np.asarray(x, float) * (1 + np.asarray(sc, float)[np.asarray(idx)]), g, eps) + np.asarray(sh, float)[np.asarray(idx)]),
    "adaln scale without the one": ("adaln_modulate", lambda x, g, sc, sh, idx, eps: O.rmsnorm(x, g, eps)
                                    * np.asarray(sc, float)[np.asarray(idx)] + np.asarray(sh, float)[np.asarray(idx)]),
    "adaln shift inside the scale": ("adaln_modulate", lambda x, g, sc, sh, idx, eps: (O.rmsnorm(x, g, eps)
                                     + np.asarray(sh, float)[np.asarray(idx)]) * (1 + np.asarray(sc, float)[np.asarray(idx)])),
    "adaln index ignored": ("adaln_modulate", lambda x, g, sc, sh, idx, eps: O.rmsnorm(x, g, eps)
                            * (1 + np.asarray(sc, float)[0]) + np.asarray(sh, float)[0]),
    "adaln bias on the folded weights": ("adaln_shift_bias", lambda sh, W: np.asarray(sh, float) @ np.asarray(W, float) * 1.5),
    "adaln table without the one": ("adaln_fold_table", lambda g, sc: O.round_to_f32(
        np.asarray(g, float)[None, :] * np.asarray(sc, float))),
    "adaln table gain dropped": ("adaln_fold_table", lambda g, sc: O.round_to_f32(1.0 + np.asarray(sc, float))),
    "adaln table in float32 steps": ("adaln_fold_table", lambda g, sc: O.round_to_f32(
        O.round_to_f32(1.0 + np.asarray(sc, float)) * np.asarray(g, float)[None, :])),
    "adaln table stored in bf16": ("adaln_fold_table", lambda g, sc: O.round_to_bf16(
        np.asarray(g, float)[None, :] * (1.0 + np.asarray(sc, float)))),
    "adaln fold bias dropped": ("adaln_norm_proj_fold", lambda x, W, mod, b, idx, eps: _fold_ref(
        x, W, mod, np.zeros_like(np.asarray(b, float)), idx, eps)),
    "adaln fold deferred multiply": ("adaln_norm_proj_fold", lambda x, W, mod, b, idx, eps: (
        (np.asarray(x, float) * O._rows_or_zero(mod, idx)) @ np.asarray(W, float)) * O.rms(x, eps)[:, None]
        + O._rows_or_zero(b, idx)),
    "adaln fold index clamped": ("adaln_norm_proj_fold", lambda x, W, mod, b, idx, eps: _fold_ref(
        x, W, mod, b, np.clip(np.asarray(idx), 0, np.asarray(mod).shape[0] - 1), eps)),
    "adaln operand without the table": ("adaln_operand", lambda x, mod, idx: O.round_to_bf16(np.asarray(x, float))),
    "adaln operand ties away": ("adaln_operand", lambda x, mod, idx: _operand_with(x, mod, idx, lambda v: np.floor(v + 0.5))),
    "adaln operand truncated": ("adaln_operand", lambda x, mod, idx: _operand_with(x, mod, idx, np.trunc)),
    "adaln operand rounded once": ("adaln_operand", lambda x, mod, idx: O.round_to_bf16(
        np.asarray(x, float) * O._rows_or_zero(mod, idx))),
    "adaln operand unrounded": ("adaln_operand", lambda x, mod, idx: np.asarray(x, float) * O._rows_or_zero(mod, idx)),
    "adaln operand index clamped": ("adaln_operand", lambda x, mod, idx: _operand_ref(
        x, mod, np.clip(np.asarray(idx), 0, np.asarray(mod).shape[0] - 1))),
    "adaln fp8 column scale dropped": ("adaln_norm_proj_fp8", lambda x, c, s, mod, b, idx, eps: _adaln_fp8_ref(
        x, c, np.ones_like(np.asarray(s, float)), mod, b, idx, eps)),
    "adaln fp8 bias dropped": ("adaln_norm_proj_fp8", lambda x, c, s, mod, b, idx, eps: _adaln_fp8_ref(
        x, c, s, mod, np.zeros_like(np.asarray(b, float)), idx, eps)),
    "adaln fp8 modulation dropped": ("adaln_norm_proj_fp8", lambda x, c, s, mod, b, idx, eps: _adaln_fp8_ref(
        x, c, s, np.ones_like(np.asarray(mod, float)), b, idx, eps)),
    "adaln q8 on the bf16 operand": ("adaln_norm_proj_swiglu_q8", lambda x, g, sc, sh, idx, Wg, Wu, eps: _q8_on_operand(
        x, g, sc, sh, idx, Wg, Wu, eps)),
    "adaln fp8 q8 without the bias": ("adaln_norm_proj_swiglu_fp8_q8", lambda x, cg, sg, cu, su, mod, bg, bu, idx, eps:
                                      _adaln_fp8_q8_ref(x, cg, sg, cu, su, mod, 0 * np.asarray(bg, float),
                                                        0 * np.asarray(bu, float), idx, eps)),
    "adaln bias on the wrong rows": ("_rows_or_zero", lambda t, idx: np.asarray(t, float)[
        (np.asarray(idx) + 1) % np.asarray(t).shape[0]]),
    "fp8 fold quantises the unfolded W": ("fold_weights_fp8", lambda g, W, dtype: O.quantize_e4m3_columns(
        O.round_to(W, dtype))[:2]),
    "fp8 fold without storage rounding": ("fold_weights_fp8", lambda g, W, dtype: O.quantize_e4m3_columns(
        O.fold_exact(g, W))[:2]),
    "q8 scale inverted": ("dequantize_row_blocks", lambda c, s, block=16: _deq_ref(c, 1.0 / np.asarray(s, float),
                                                                                 block)),
}


_encode_ref = O.e4m3_encode
_operand_ref = O.adaln_operand
_adaln_fp8_ref = O.adaln_norm_proj_fp8
_fold_ref = O.adaln_norm_proj_fold
_adaln_fp8_q8_ref = O.adaln_norm_proj_swiglu_fp8_q8


def _operand_with(x, mod, idx, rnd):
    """The AdaLN operand with another rounding of the positive magnitude to
    the bf16 grid (8 significant bits)."""
    v = O.round_to_f32(np.asarray(x, float) * O._rows_or_zero(mod, idx))
    mag = np.abs(v)
    with np.errstate(all="ignore"):
        _, e = np.frexp(mag)
        q = np.ldexp(rnd(np.ldexp(mag, 8 - e)), e - 8)
    return np.copysign(q, v)


def _q8_on_operand(x, g, sc, sh, idx, Wg, Wu, eps):
    """The AdaLN q8 values formed on a bf16-rounded modulated operand
    (the arithmetic of a kernel, not the definition)."""
    mod = O.adaln_fold_table(g, sc)
    u = O.adaln_operand(x, mod, idx)
    r = O.rms(x, eps)[:, None]
    a = (u @ np.asarray(Wg, float)) / r + (np.asarray(sh, float) @ np.asarray(Wg, float))[np.asarray(idx)]
    b = (u @ np.asarray(Wu, float)) / r + (np.asarray(sh, float) @ np.asarray(Wu, float))[np.asarray(idx)]
    v = O.silu(a) * b
    c, s = O.quantize_e4m3_row_blocks(v)
    return c, s, v
_decode_ref = O.e4m3_decode
_quantize_ref = O.quantize_e4m3_columns


def _encode_with(a, rnd):
    """E4M3 encoder with a different rounding of the scaled magnitude."""
    a = np.asarray(a, float)
    mag = np.abs(a)
    with np.errstate(all="ignore"):
        _, e = np.frexp(mag)
        e = np.maximum(e, -5)
        val = np.minimum(np.ldexp(rnd(np.ldexp(mag, 4 - e)), e - 4), 448.0)
    return _encode_ref(np.copysign(val, a))


def _decode_bias(c, bias):
    c = np.asarray(c, dtype=np.int64) & 0xFF
    e = (c >> 3) & 0xF
    m = (c & 7) / 8.0
    v = np.where(e == 0, np.ldexp(m, 1 - bias), np.ldexp(1 + m, e - bias))
    v = np.where((c & 0x7F) == 0x7F, np.nan, v)
    return np.where(c & 0x80, -v, v)


def _quantize_rows(W):
    Wt = np.asarray(W, dtype=np.float32).T.copy()
    codes, s, r = _quantize_ref(Wt)
    n = np.asarray(W).shape[1]
    return codes.T.copy(), np.resize(s, n).astype(np.float32), np.resize(r, n).astype(np.float32)


_q8_ref = O.quantize_e4m3_row_blocks
_deq_ref = O.dequantize_row_blocks


def _q8_columns(v, block):
    """Blocks of 16 rows of one column instead of 16 columns of one row."""
    c, s = _q8_ref(np.asarray(v, dtype=np.float32).T.copy(), block)
    nb = -(-np.asarray(v).shape[1] // block)
    return c.T.copy(), np.resize(s.T, (np.asarray(v).shape[0], nb)).astype(np.float32)


def _q8_flat(v, block):
    """Blocks of 16 consecutive values of the flattened matrix (rows not
    padded: the last block of a row runs into the next row)."""
    v32 = np.asarray(v, dtype=np.float32)
    M, N = v32.shape
    flat = v32.reshape(1, M * N)
    c, s = _q8_ref(flat, block)
    nb = -(-N // block)
    return c.reshape(M, N), np.resize(s, (M, nb)).astype(np.float32)


@pytest.mark.parametrize("name", sorted(MUTANTS))
def test_pins_catch_planted_mistakes(name, monkeypatch):
    attr, fn = MUTANTS[name]
    original = {k: getattr(O, k) for k in ("rms", "rmsnorm", "silu", "e4m3_encode", "e4m3_decode")}
    monkeypatch.setattr(O, attr, fn)
    # mutants that call O.rms / O.rmsnorm / O.silu must see the unmutated
    # helpers unless the helper itself is the mutant
    caught = []
    for check in P.ALL_CHECKS:
        try:
            check(O)
        except Exception as e:  # noqa: BLE001 - any failure counts as detection
            caught.append(f"{check.__name__}: {type(e).__name__}")
    assert caught, f"no pin caught planted mistake {name!r}"
    assert original  # keep reference for readability


def test_eps_is_the_float32_value():
    assert O.eps_as_received(1e-6) == float(np.float32(1e-6))
    assert O.eps_as_received(1e-6) != 1e-6
