"""The benchmark's measurement definitions, pinned to the scope table's
figures (algorithmic bytes count W' once, x once and y once; FLOPs are
2*M*K*N*mats) and to hand-computed values for the fp8 and fp8-output forms,
so the roofline denominators cannot drift from the contract.  CPU only."""
import numpy as np

import bench
import workloads as W


def test_algorithmic_bytes_and_flops_of_the_five_configs():
    wl = W.WORKLOADS
    assert wl["tiny"].algorithmic_bytes() == 802_816 and wl["tiny"].flops() == 1_572_864
    assert wl["qkv_decode"].algorithmic_bytes() == 101_187_584 and wl["qkv_decode"].flops() == 1_610_612_736
    assert wl["ffn_decode"].algorithmic_bytes() == 182_288_384 and wl["ffn_decode"].flops() == 11_542_724_608
    assert wl["prefill_qkv"].algorithmic_bytes() == 234_881_024 and wl["prefill_qkv"].flops() == 412_316_860_416
    step = W.decode_step_calls()
    assert len(step) == 65
    assert sum(c.algorithmic_bytes() for c in step) == 9_271_431_168
    assert sum(c.flops() for c in step) == 74_037_854_208
    # bench's own per-call figure is the same definition for bf16 weights and output
    for name in ("qkv_decode", "ffn_decode", "prefill_qkv"):
        assert bench.call_bytes(wl[name], fp8=False, q8=False) == wl[name].algorithmic_bytes()


def test_decode_step_shards():
    """One GPU's column share of the step under tensor parallelism: every
    projection's N divided by the GPU count, x whole, the bytes summing to
    the share of the weights plus each call's x and y."""
    full, share = W.decode_step_calls(), W.decode_step_calls(shard=8)
    assert len(share) == 65
    assert [c.N for c in share[:2]] + [share[-1].N] == [1536, 1376, 4000]
    assert all(c.K == 4096 and c.M == 8 for c in share)
    w_full = sum(c.mats * c.K * c.N * 2 for c in full)
    w_share = sum(c.mats * c.K * c.N * 2 for c in share)
    assert w_share * 8 == w_full
    assert sum(c.algorithmic_bytes() for c in share) == w_share + sum(2 * (c.M * c.K + c.M * c.N) for c in share)
    import pytest
    with pytest.raises(ValueError):
        W.decode_step_calls(shard=3)
    assert bench.parse_args(["--workload", "decode_step", "--step-shard", "8"]).step_shard == 8


def test_fp8_and_fp8_output_bytes():
    c = W.WORKLOADS["qkv_decode"]            # 16 x 4096 -> 12288
    # codes (1 B each) and one fp32 scale per column, bf16 x and y
    assert bench.fp8_bytes(c) == 4096 * 12288 + 4 * 12288 + 2 * (16 * 4096 + 16 * 12288)
    assert bench.call_bytes(c, fp8=True, q8=False) == bench.fp8_bytes(c)
    f = W.WORKLOADS["ffn_decode"]            # 64 x 4096 -> 2 x 11008, E4M3 output + a scale per 16 columns
    out_q8 = 64 * 11008 + 4 * 64 * (11008 // 16)
    assert bench.call_bytes(f, fp8=False, q8=True) == 2 * 4096 * 11008 * 2 + 2 * 64 * 4096 + out_q8
    # the AdaLN inputs: the fp32 modulation table, the row indices and the fp32 bias rows
    assert bench.adaln_extra_bytes(f) == 4 * bench.ADALN_T * 4096 + 4 * 64 + 4 * bench.ADALN_T * 11008 * 2


def test_percentile_and_parity_report():
    assert bench.pct([1.0, 2.0, 3.0, 4.0, 5.0], 0.5) == 3.0
    assert bench.pct([1.0, 2.0, 3.0, 4.0, 5.0], 0.1) == 1.0 and bench.pct([1.0, 2.0, 3.0, 4.0, 5.0], 0.9) == 5.0
    y = np.array([[1.0, 2.0], [3.0, 4.0], [9.0, 9.0]], dtype=np.float32)
    ref = np.array([[1.0, 2.5], [3.0, 3.0]])
    r = bench.parity_report(y, ref)
    assert r["rows"] == 2 and r["cols"] == 2
    assert abs(r["max_err_rel"] - 1.0 / 4.0) < 1e-3            # max of |err| / (|ref| + 1): 1 / (3 + 1)
    assert abs(r["mean_abs_err"] - 1.5 / 4) < 1e-3
