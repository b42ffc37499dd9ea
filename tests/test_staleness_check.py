"""Negative control of the staleness check the GPU tests apply to
back-to-back calls (tests/gpu_helpers.py, stale_failures), on the CPU: the
outputs a post-scale produces when it does not wait for its product -- the
FlashNorm talk's two-stream bug ([FlashNorm digest], the bug / cause / fix
bullets): each call scaled the previous call's product -- must be flagged,
and the correct outputs must pass.  The outputs are formed from the float64
oracle and rounded to bf16 as a kernel would store them."""
import numpy as np

import oracle
import workloads as W
from tests.gpu_helpers import stale_failures


def _calls(T=8, M=16, K=1024, N=512):
    base = W.random_inputs(M, K, N, "bf16", seed=15)
    xs = [W.make_x(M, K, "bf16", seed=2000 + t) for t in range(T)]
    Wf = oracle.fold_weights(base.g, base.W, "bf16")
    refs = [oracle.norm_proj(x, base.g, base.W, 1e-6) for x in xs]
    prods = [np.asarray(x, np.float64) @ Wf for x in xs]
    inv = [1.0 / oracle.rms(x, 1e-6)[:, None] for x in xs]
    return refs, prods, inv


def test_correct_post_scale_passes():
    refs, prods, inv = _calls()
    outs = [oracle.round_to_bf16(p * r) for p, r in zip(prods, inv)]
    assert stale_failures(outs, refs) == []


def test_post_scale_of_the_previous_product_is_flagged():
    refs, prods, inv = _calls()
    # call t scales the product call t-1 left behind (call 0 finds the NaN-poisoned buffer)
    stale = [np.full_like(prods[0], np.nan)] + prods[:-1]
    outs = [oracle.round_to_bf16(p * r) for p, r in zip(stale, inv)]
    bad = stale_failures(outs, refs)
    assert len(bad) >= len(refs), bad


def test_a_single_stale_call_is_flagged():
    refs, prods, inv = _calls()
    outs = [oracle.round_to_bf16(p * r) for p, r in zip(prods, inv)]
    outs[5] = oracle.round_to_bf16(prods[4] * inv[5])
    bad = stale_failures(outs, refs)
    assert any(b.startswith("call 5") for b in bad), bad
