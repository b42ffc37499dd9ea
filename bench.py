#!/usr/bin/env python3
"""Benchmark of fused RMSNorm + projection (libflashnorm) on one MI355X.

    python bench.py [--steps K] [--warmup W] [--workload NAME] [--configs LIST|none]

A step is one pass of the hot path over one batch: one fused call for the
single-call workloads, or the 65 calls of the 32-layer decode step.  Inputs
are seeded synthetics already resident in HBM when timing starts.  Decode
workloads rotate distinct copies of the folded weights (>= 1 GiB in total)
so the 256 MB Infinity Cache cannot serve repeated calls ("cold", the
headline); the single-buffer ("hot") figure is reported beside it.

Timing: after a clock warm-up and W untimed steps, K steps run back to back
in blocks, an event pair around each block (no event per call); the mean
over the region gives ms_per_step and roofline.achieved, the median block
gives `value` (with p10/p90 of the blocks beside it).

Prints ONE JSON line: the headline workload (default: the QKV decode
projection, x[16,4096] bf16 -> W'[4096,12288]) at the top level, and under
"configs" every other workload of the metric measured in the same process
(tiny fp32 decode, FFN SwiGLU decode, prefill QKV, the 32-layer decode step,
and the two decode shapes with fp8 weights), each with its own rate,
roofline fraction, unfused-chain speed-ups and CPU-oracle baseline.
"""
from __future__ import annotations

import argparse
import hashlib
import json
import math
import os
import re
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

METRIC = "fused RMSNorm+proj: decode µs/call & HBM GB/s; prefill TFLOP/s; % roofline"
HBM_PEAK_GBS = 8000.0          # MI355X HBM3E, vendor figure
BF16_PEAK_TFLOPS = 2500.0      # MI355X dense bf16 MFMA, vendor figure
F32_PEAK_TFLOPS = 157.3        # MI355X fp32 vector
ROTATE_BYTES = 1 << 30


def parse_args(argv=None):
    p = argparse.ArgumentParser(description=__doc__, formatter_class=argparse.RawDescriptionHelpFormatter)
    p.add_argument("--gpus", type=int, default=1)
    p.add_argument("--steps", type=int, default=200)
    p.add_argument("--warmup", type=int, default=20)
    p.add_argument("--workload", default="qkv_decode",
                   choices=["tiny", "qkv_decode", "ffn_decode", "prefill_qkv", "decode_step"])
    p.add_argument("--step-rows", type=int, default=8,
                   help="decode_step: rows of every call (1..128; the step is quoted at 8)")
    p.add_argument("--step-shard", type=int, default=1, choices=[1, 2, 4, 8],
                   help="decode_step: one GPU's column share of every projection under tensor parallelism over "
                        "that many GPUs (1: the whole step)")
    p.add_argument("--weights", default="native", choices=["native", "fp8"],
                   help="weight storage: the activations' dtype, or E4M3 codes with per-column scales "
                        "(bf16 decode workloads only)")
    p.add_argument("--output", default="native", choices=["native", "q8"],
                   help="q8: SwiGLU output as E4M3 codes + one scale per 16-column row block (ffn_decode)")
    p.add_argument("--prologue", default="none", choices=["none", "adaln"],
                   help="adaln: AdaLN modulation after the norm (scale/shift tables of ADALN_T rows, per-row index)")
    p.add_argument("--no-chain", action="store_true",
                   help="skip the comparison runs (unfused chains; bf16 weights beside fp8)")
    p.add_argument("--no-cpu-baseline", action="store_true", help="skip timing the CPU oracle")
    p.add_argument("--no-measured-peak", dest="measured_peak", action="store_false",
                   help="skip measuring the attainable peak (roofline.measured_peak, frac_measured)")
    p.add_argument("--no-plain-read", dest="plain_read", action="store_false",
                   help="skip timing a plain streaming read of each HBM-bound call's bytes")
    p.add_argument("--cpu-seconds", type=float, default=10.0, help="CPU oracle sample budget")
    p.add_argument("--configs", default=",".join(DEFAULT_CONFIGS),
                   help="other workloads to measure in the same run, comma-separated names from "
                        f"{', '.join(CONFIG_CHOICES)}, or 'none'")
    p.add_argument("--hot", action="store_true", help="time a single weight buffer only (no rotation)")
    p.add_argument("--clock-warmup-s", type=float, default=0.5,
                   help="untimed seconds of steps before warmup (clock ramp-up); 0 under a profiler")
    p.add_argument("--calibrate-copy", action="store_true",
                   help="run 1 GiB device-to-device copies (counter calibration) and exit")
    return p.parse_args(argv)


# Workloads measured beside the headline (name: workload, weights).
CONFIG_CHOICES = {"tiny": ("tiny", "native"), "qkv_decode": ("qkv_decode", "native"),
                  "ffn_decode": ("ffn_decode", "native"), "prefill_qkv": ("prefill_qkv", "native"),
                  "decode_step": ("decode_step", "native"), "qkv_decode_fp8": ("qkv_decode", "fp8"),
                  "ffn_decode_fp8": ("ffn_decode", "fp8"), "decode_step_fp8": ("decode_step", "fp8")}
DEFAULT_CONFIGS = ("tiny", "ffn_decode", "prefill_qkv", "decode_step", "qkv_decode_fp8", "ffn_decode_fp8",
                   "decode_step_fp8")
# steps and warmup of a config run: the headline's, capped where one step is long
CONFIG_STEP_CAP = {"prefill_qkv": (50, 5), "decode_step": (20, 3)}


# ----------------------------------------------------------------- timing --
CLOCK_WARMUP_S = 0.5


def clock_warmup(torch, launch):
    """Run the step untimed for CLOCK_WARMUP_S so the GPU leaves its idle
    power state before anything is timed (the first ~second runs at lower
    clocks on MI355X)."""
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    i = 0
    while CLOCK_WARMUP_S > 0 and time.perf_counter() - t0 < CLOCK_WARMUP_S:
        for _ in range(8):
            launch(i)
            i += 1
        torch.cuda.synchronize()


def time_blocks(torch, launch, steps, warmup):
    """(mean ms per step over the region, sorted per-block ms per step):
    after a clock warm-up and `warmup` untimed steps, `steps` back-to-back
    steps in up to 20 blocks with an event recorded between blocks (events
    on the current stream, which is the stream every launch uses), bracketed
    by device synchronisations."""
    clock_warmup(torch, launch)
    for i in range(warmup):
        launch(i)
    torch.cuda.synchronize()
    nb = max(1, min(20, steps))
    bounds = [steps * b // nb for b in range(nb + 1)]
    evs = [torch.cuda.Event(enable_timing=True) for _ in range(nb + 1)]
    evs[0].record()
    for b in range(nb):
        for i in range(bounds[b], bounds[b + 1]):
            launch(i)
        evs[b + 1].record()
    torch.cuda.synchronize()
    blocks = sorted(evs[b].elapsed_time(evs[b + 1]) / (bounds[b + 1] - bounds[b]) for b in range(nb))
    return evs[0].elapsed_time(evs[nb]) / steps, blocks


def time_region(torch, launch, steps, warmup):
    """Mean ms per step over the region (time_blocks)."""
    return time_blocks(torch, launch, steps, warmup)[0]


def pct(sorted_vals, q):
    i = min(len(sorted_vals) - 1, max(0, int(round(q * (len(sorted_vals) - 1)))))
    return sorted_vals[i]


# Sources each workload's dominant kernel is built from.
KERNEL_SOURCES = {"prefill_qkv": ("prefill.hip", "fn_device.h"), "ffn_decode": ("decode_x.hip", "fn_device.h"),
                  "qkv_decode_fp8": ("decode_x.hip", "fn_device.h"), "ffn_decode_fp8": ("decode_x.hip", "fn_device.h"),
                  # a decode step's HBM traffic is counted on its grouped launch (decode_grouped*_kernel)
                  "decode_step_fp8": ("decode.hip", "fn_device.h"), "ffn_decode_q8": ("decode_x.hip", "fn_device.h"),
                  "ffn_decode_fp8_q8": ("decode_x.hip", "fn_device.h"), "qkv_decode_adaln": ("decode_x.hip", "fn_device.h"),
                  "qkv_decode_fp8_adaln": ("decode_x.hip", "adaln.hip", "fn_device.h"),
                  "ffn_decode_fp8_adaln": ("decode_x.hip", "adaln.hip", "fn_device.h"),
                  "ffn_decode_q8_adaln": ("decode_x.hip", "adaln.hip", "fn_device.h"),
                  "ffn_decode_fp8_q8_adaln": ("decode_x.hip", "adaln.hip", "fn_device.h"),
                  "ffn_decode_adaln": ("decode_x.hip", "adaln.hip", "fn_device.h"), "prefill_qkv_adaln": ("prefill.hip", "adaln.hip", "fn_device.h"),
                  "prefill_qkv_fp8": ("prefill.hip", "fn_device.h"),
                  "prefill_qkv_fp8_adaln": ("prefill.hip", "adaln.hip", "fn_device.h")}
DEFAULT_KERNEL_SOURCES = ("decode.hip", "fn_device.h")


def _code_only(text):
    """Source text without comments and with whitespace collapsed, so that
    editing a comment does not mark counters taken on the same code stale."""
    text = re.sub(r"/\*.*?\*/", " ", text, flags=re.S)
    text = re.sub(r"//[^\n]*", " ", text)
    return " ".join(text.split())


def kernel_source_hash(workload):
    h = hashlib.sha256()
    csrc = os.path.join(ROOT, "rmsnorm_projection_gemm_amd", "csrc")
    for f in KERNEL_SOURCES.get(workload, DEFAULT_KERNEL_SOURCES):
        with open(os.path.join(csrc, f), encoding="utf-8") as fh:
            h.update(f.encode() + _code_only(fh.read()).encode())
    return h.hexdigest()[:16]


def counter_traffic(workload):
    """HBM bytes per launch from the committed rocprofv3 counter summary, if
    it was taken on the current sources of the workload's kernel; else None."""
    path = os.path.join(ROOT, "profiles", f"{workload}_traffic.json")
    if not os.path.exists(path):
        return None
    with open(path) as f:
        d = json.load(f)
    if d.get("kernel_source_hash") != kernel_source_hash(workload):
        return None
    return d.get("hbm_bytes_per_launch")


def fp8_bytes(call):
    """Algorithmic bytes of one call with fp8 weights: the codes and the
    column scales once, x and y (bf16) once."""
    return call.mats * (call.K * call.N + 4 * call.N) + 2 * (call.M * call.K + call.M * call.N)


ADALN_T = 4


def adaln_extra_bytes(call):
    """AdaLN inputs read once: the modulation table [T, K] fp32, the row
    indices [M] int32 and the bias rows [T, N] fp32 per weight matrix."""
    return 4 * ADALN_T * call.K + 4 * call.M + 4 * ADALN_T * call.N * call.mats


def call_bytes(call, fp8, q8):
    """Algorithmic bytes of one call: weights (bf16 W', or E4M3 codes and
    column scales) once, x once, and the output once (bf16 y, or E4M3 codes
    plus one fp32 scale per 16-column row block)."""
    w = call.mats * (call.K * call.N + 4 * call.N) if fp8 else call.mats * call.K * call.N * (2 if call.dtype == "bf16" else 4)
    e = 2 if call.dtype == "bf16" else 4
    out = call.M * call.N + 4 * call.M * (-(-call.N // 16)) if q8 else e * call.M * call.N
    return w + e * call.M * call.K + out


# ------------------------------------------------------------ CPU oracle --
def cpu_model():
    try:
        with open("/proc/cpuinfo") as f:
            for line in f:
                if line.startswith("model name"):
                    return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return None


def cpu_baseline(call, inp, budget_s, metric_unit, fp8=False, q8=False, adaln=False, one_thread_s=0.0):
    """The float64 oracle as it stands, on the host cores, on a bounded sample
    of the same workload; scaled to the metric's unit.  one_thread_s > 0: the
    same sample again with the BLAS pool limited to one thread."""
    if one_thread_s > 0:
        out = cpu_baseline(call, inp, budget_s, metric_unit, fp8, q8, adaln)
        from threadpoolctl import threadpool_limits
        with threadpool_limits(limits=1):
            one = cpu_baseline(call, inp, one_thread_s, metric_unit, fp8, q8, adaln)
        out["one_thread"] = {"value": one["value"], "unit": one["unit"], "cores": one["cores"],
                             "sample": one["sample"]}
        return out
    import numpy as np
    import oracle
    try:
        from threadpoolctl import threadpool_info
        cores = max([i.get("num_threads", 1) for i in threadpool_info()] or [1])
    except Exception:  # noqa: BLE001
        cores = 1
    rows = call.M
    # keep one oracle call to a few seconds at most: sample rows for big M
    if call.M * call.K * call.N * call.mats > 2e10:
        rows = max(1, int(2e10 // (call.K * call.N * call.mats)))
    x = inp.x[:rows]
    calls, t0 = 0, time.perf_counter()
    w8 = None
    ref = None
    if fp8:
        # the AdaLN calls quantise the plain W (the gain goes into the table)
        gq = np.ones(call.K) if adaln else inp.g
        w8 = [oracle.fold_weights_fp8(gq, inp.W, call.dtype)]
        if call.swiglu:
            w8.append(oracle.fold_weights_fp8(gq, inp.W_up, call.dtype))
    if adaln:
        import workloads
        sc, sh, idx = workloads.adaln_tables(ADALN_T, call.K, call.M, seed=call.seed + 100)
        idx = idx[:rows]
        mod = oracle.adaln_fold_table(inp.g, sc)
        bias8 = [oracle.adaln_shift_bias(sh, inp.W)] + ([oracle.adaln_shift_bias(sh, inp.W_up)] if call.swiglu else [])
    while True:
        if adaln and q8 and fp8:
            oracle.adaln_norm_proj_swiglu_fp8_q8(x, w8[0][0], w8[0][1], w8[1][0], w8[1][1], mod, bias8[0], bias8[1],
                                                 idx, call.eps)
        elif adaln and q8:
            oracle.adaln_norm_proj_swiglu_q8(x, inp.g, sc, sh, idx, inp.W, inp.W_up, call.eps)
        elif adaln and fp8 and call.swiglu:
            ref = oracle.adaln_norm_proj_swiglu_fp8(x, w8[0][0], w8[0][1], w8[1][0], w8[1][1], mod, bias8[0], bias8[1], idx,
                                              call.eps)
        elif adaln and fp8:
            ref = oracle.adaln_norm_proj_fp8(x, w8[0][0], w8[0][1], mod, bias8[0], idx, call.eps)
        elif adaln and call.swiglu:
            ref = oracle.adaln_norm_proj_swiglu(x, inp.g, sc, sh, idx, inp.W, inp.W_up, call.eps)
        elif adaln:
            ref = oracle.adaln_norm_proj(x, inp.g, sc, sh, idx, inp.W, call.eps)
        elif q8 and fp8:
            oracle.norm_proj_swiglu_fp8_q8(x, w8[0][0], w8[0][1], w8[1][0], w8[1][1], call.eps)
        elif q8:
            oracle.norm_proj_swiglu_q8(x, inp.g, inp.W, inp.W_up, call.eps)
        elif fp8 and call.swiglu:
            ref = oracle.norm_proj_swiglu_fp8(x, w8[0][0], w8[0][1], w8[1][0], w8[1][1], call.eps)
        elif fp8:
            ref = oracle.norm_proj_fp8(x, w8[0][0], w8[0][1], call.eps)
        elif call.swiglu:
            ref = oracle.norm_proj_swiglu(x, inp.g, inp.W, inp.W_up, call.eps)
        else:
            ref = oracle.norm_proj(x, inp.g, inp.W, call.eps)
        calls += 1
        el = time.perf_counter() - t0
        if el >= budget_s:
            break
    per_call = el / calls * (call.M / rows)       # seconds per full call
    if metric_unit == "TFLOP/s":
        value = call.flops() / per_call / 1e12
    elif metric_unit == "GB/s":
        value = (call_bytes(call, fp8, q8) + (adaln_extra_bytes(call) if adaln else 0)) / per_call / 1e9
    else:
        value = per_call * 1e6
    sample = (f"{calls} oracle call(s) on x[{rows},{call.K}] (of M={call.M}) x W[{call.K},{call.N}]"
              f"{' x2 (gate, up)' if call.swiglu else ''}{' (E4M3 codes)' if fp8 else ''}"
              f"{', E4M3 row-block output' if q8 else ''}{', AdaLN prologue' if adaln else ''}, float64, {el:.1f} s;"
              f" scaled by M/{rows}")
    return {"value": round(value, 4), "unit": metric_unit, "cores": cores, "kind": "oracle",
            "sample": sample, "seconds_per_call": per_call, "cpu_model": cpu_model(), "nproc": os.cpu_count(),
            "_ref": ref}


PARITY_ROWS = 512


def parity_report(y_head, ref):
    """The fused call's output against the oracle's on the sampled rows:
    max |err| / (|ref| + 1) and mean |err| (the tests hold every output to
    the tolerance; this reports the margin at the benchmarked size)."""
    import numpy as np
    n = min(y_head.shape[0], ref.shape[0])
    err = np.abs(y_head[:n].astype(np.float64) - ref[:n])
    return {"rows": int(n), "cols": int(ref.shape[1]), "max_err_rel": float(f"{(err / (np.abs(ref[:n]) + 1)).max():.3e}"),
            "mean_abs_err": float(f"{err.mean():.3e}"), "reference": "float64 oracle, same seeded inputs"}


# ---------------------------------------------------------- single calls --
def to_dev(torch, a, dtype):
    t = torch.from_numpy(a)
    return t.to(torch.bfloat16 if dtype == "bf16" else torch.float32).cuda()


TINY_STEP_CALLS = 64


def run_single(args, torch, fn, workloads):
    call = workloads.WORKLOADS[args.workload]
    inp = workloads.make_inputs(call)
    x = to_dev(torch, inp.x, call.dtype)
    g = to_dev(torch, inp.g, call.dtype)
    Wg = to_dev(torch, inp.W, call.dtype)
    Wu = to_dev(torch, inp.W_up, call.dtype) if call.swiglu else None
    fp8 = args.weights == "fp8"
    adaln = args.prologue == "adaln"
    gw = None if adaln else g      # AdaLN: the gain folds into the modulation table, the weights stay plain
    if fp8:
        Pg = fn.fold_weights_fp8(gw, Wg)
        Pu = fn.fold_weights_fp8(gw, Wu) if call.swiglu else None
        wbytes = (Pg.data.numel() + Pg.scales.numel() * 4) * call.mats

        def clone(P):
            return fn.PackedFp8(P.data.clone(), P.scales.clone(), P.K, P.N)
        proj, proj_sw = fn.norm_proj_fp8, fn.norm_proj_swiglu_fp8
    else:
        Pg = fn.fold_weights(gw, Wg)
        Pu = fn.fold_weights(gw, Wu) if call.swiglu else None
        wbytes = Pg.data.numel() * call.mats

        def clone(P):
            return fn.PackedWeights(P.data.clone(), P.K, P.N, P.dtype)
        proj, proj_sw = fn.norm_proj, fn.norm_proj_swiglu
    rot = 1 if args.hot else max(1, math.ceil(ROTATE_BYTES / wbytes))
    pgs = [Pg] + [clone(Pg) for _ in range(rot - 1)]
    pus = ([Pu] + [clone(Pu) for _ in range(rot - 1)]) if call.swiglu else None
    y = torch.empty((call.M, call.N), dtype=x.dtype, device="cuda")
    eps = call.eps
    if adaln:
        sc_np, sh_np, idx_np = workloads.adaln_tables(ADALN_T, call.K, call.M, seed=call.seed + 100)
        sc_t, sh_t = to_dev(torch, sc_np, "bf16"), to_dev(torch, sh_np, "bf16")
        mod_t = fn.adaln_fold_table(g, sc_t)
        idx_t = torch.from_numpy(idx_np).cuda()
        bg_t = fn.adaln_shift_bias(sh_t, Wg)
        bu_t = fn.adaln_shift_bias(sh_t, Wu) if call.swiglu else None
        # the two-launch form above 16 rows, and with fp8 weights (pre-pass into a workspace allocated here, once)
        nws = (fn.adaln_prepass_bytes(call.M, call.K) if fp8 or args.output == "q8" else
               fn.adaln_workspace_bytes(call.M, call.K))
        ws_t = torch.empty((nws,), dtype=torch.uint8, device="cuda") if nws else None
        f1, f2 = ((fn.norm_proj_adaln_fp8_ws, fn.norm_proj_swiglu_adaln_fp8_ws) if fp8 else
                  (fn.norm_proj_adaln_ws, fn.norm_proj_swiglu_adaln_ws))
        proj = lambda x_, P_, e_, out=None: f1(x_, mod_t, idx_t, P_, bg_t, e_, out=out, workspace=ws_t)  # noqa: E731
        proj_sw = lambda x_, a_, b_, e_, out=None: f2(  # noqa: E731
            x_, mod_t, idx_t, a_, bg_t, b_, bu_t, e_, out=out, workspace=ws_t)
    q8 = args.output == "q8"
    if q8:
        # SwiGLU quantised in the epilogue: E4M3 codes + row-block scales
        qout = (torch.empty((call.M, call.N), dtype=torch.uint8, device="cuda"),
                torch.empty((call.M, -(-call.N // 16)), dtype=torch.float32, device="cuda"))
        if adaln:
            fq = fn.norm_proj_swiglu_adaln_fp8_q8_ws if fp8 else fn.norm_proj_swiglu_adaln_q8_ws
            proj_sw = lambda x_, a_, b_, e_, out=None: fq(  # noqa: E731
                x_, mod_t, idx_t, a_, bg_t, b_, bu_t, e_, out=qout, workspace=ws_t)
        else:
            proj_q8 = fn.norm_proj_swiglu_fp8_q8 if fp8 else fn.norm_proj_swiglu_q8
            proj_sw = lambda x_, a_, b_, e_, out=None: proj_q8(x_, a_, b_, e_, out=qout)  # noqa: E731

    if call.swiglu:
        def fused(i):
            proj_sw(x, pgs[i % rot], pus[i % rot], eps, out=y)
    else:
        def fused(i):
            proj(x, pgs[i % rot], eps, out=y)

    ms, blocks = time_blocks(torch, fused, args.steps, args.warmup)
    hot_ms = time_region(torch, lambda i: (proj_sw(x, Pg, Pu, eps, out=y) if call.swiglu
                                           else proj(x, Pg, eps, out=y)), args.steps, args.warmup)
    result = {"ms": ms, "blocks": blocks, "hot_ms": hot_ms, "rot": rot, "wbytes": wbytes}
    if not q8:
        torch.cuda.synchronize()
        result["y_head"] = y[:PARITY_ROWS].float().cpu().numpy()   # the fused output's first rows, for the parity report
    if args.workload == "tiny":
        # launch-bound: the same call recorded TINY_STEP_CALLS times into one
        # step, replayed with one graph launch; reported per call
        step = fn.Step()
        for _ in range(TINY_STEP_CALLS):
            step.norm_proj(x, Pg, y, eps)
        step.record()
        result["graph_ms"] = time_region(torch, lambda _: step.launch(), args.steps, args.warmup) / TINY_STEP_CALLS
        torch.cuda.synchronize()
        step.close()
    if fp8 and not args.no_chain:
        # the same call with bf16 folded weights, same rotation rule, for comparison
        del pgs, pus
        Bg = fn.fold_weights(g, Wg)
        Bu = fn.fold_weights(g, Wu) if call.swiglu else None
        brot = max(1, math.ceil(ROTATE_BYTES / (Bg.data.numel() * call.mats)))
        bgs = [Bg] + [fn.PackedWeights(Bg.data.clone(), Bg.K, Bg.N, Bg.dtype) for _ in range(brot - 1)]
        bus = ([Bu] + [fn.PackedWeights(Bu.data.clone(), Bu.K, Bu.N, Bu.dtype) for _ in range(brot - 1)]
               if call.swiglu else None)
        bsw = ((lambda x_, a_, b_, e_, out=None: fn.norm_proj_swiglu_q8(x_, a_, b_, e_, out=qout)) if q8
               else fn.norm_proj_swiglu)
        result["bf16_ms"] = time_region(
            torch, lambda i: (bsw(x, bgs[i % brot], bus[i % brot], eps, out=y) if call.swiglu
                              else fn.norm_proj(x, bgs[i % brot], eps, out=y)), args.steps, args.warmup)
        del bgs, bus

    if not args.no_chain:
        # unfused chains on row-major weights, same rotation
        Wcat = torch.cat([Wg, Wu], dim=1).contiguous() if call.swiglu else Wg
        ws = [Wcat] + [Wcat.clone() for _ in range(rot - 1)]
        xhat = torch.empty_like(x)
        N = call.N

        def quantize(v):
            # the chain's own quantisation step: row-block amax, scale, E4M3
            nb = -(-N // 16)
            vb = torch.nn.functional.pad(v.float(), (0, nb * 16 - N)).view(call.M, nb, 16)
            amax = vb.abs().amax(-1, keepdim=True)
            r = torch.where(amax > 0, 448.0 / amax, torch.ones_like(amax))
            qout[0].copy_((vb * r).to(torch.float8_e4m3fn).view(torch.uint8).view(call.M, nb * 16)[:, :N])
            qout[1].copy_(torch.where(amax > 0, amax / 448.0, torch.ones_like(amax)).view(call.M, nb))

        def chain_own(i):
            fn.rmsnorm(x, g, eps, out=xhat)
            h = torch.matmul(xhat * (1 + sc_t[idx_t]) + sh_t[idx_t] if adaln else xhat, ws[i % rot])
            if call.swiglu:
                fn.silu_mul(h, out=y)
                if q8:
                    quantize(y)

        def chain_torch(i):
            xn = torch.nn.functional.rms_norm(x, (call.K,), g, eps)
            if adaln:
                xn = xn * (1 + sc_t[idx_t]) + sh_t[idx_t]
            h = torch.matmul(xn, ws[i % rot])
            if call.swiglu:
                torch.mul(torch.nn.functional.silu(h[:, :N]), h[:, N:], out=y)
                if q8:
                    quantize(y)

        result["chain_own_ms"] = time_region(torch, chain_own, args.steps, args.warmup)
        result["chain_torch_ms"] = time_region(torch, chain_torch, args.steps, args.warmup)
        del ws
    return call, inp, result


def run_decode_step(args, torch, fn, workloads):
    calls = workloads.decode_step_calls(rows=getattr(args, "step_rows", 8), shard=getattr(args, "step_shard", 1))
    items = []
    fp8 = args.weights == "fp8"
    fold = fn.fold_weights_fp8 if fp8 else fn.fold_weights
    proj = fn.norm_proj_fp8 if fp8 else fn.norm_proj
    proj_sw = fn.norm_proj_swiglu_fp8 if fp8 else fn.norm_proj_swiglu
    for c in calls:
        x, g, Wg, Wu = workloads.make_inputs_device(c)
        Pg = fold(g, Wg)
        Pu = fold(g, Wu) if c.swiglu else None
        item = {"call": c, "x": x, "g": g, "Pg": Pg, "Pu": Pu,
                "y": torch.empty((c.M, c.N), dtype=x.dtype, device="cuda")}
        if not args.no_chain:
            item["Wcat"] = torch.cat([Wg, Wu], dim=1).contiguous() if c.swiglu else Wg
            item["xhat"] = torch.empty_like(x)
        del Wg, Wu
        items.append(item)

    def fused(_):
        for it in items:
            c = it["call"]
            if c.swiglu:
                proj_sw(it["x"], it["Pg"], it["Pu"], c.eps, out=it["y"])
            else:
                proj(it["x"], it["Pg"], c.eps, out=it["y"])

    ms, blocks = time_blocks(torch, fused, args.steps, args.warmup)
    # the same 65 calls recorded once into a HIP graph, replayed with one launch
    step = fn.Step()
    for it in items:
        c = it["call"]
        if c.swiglu:
            (step.norm_proj_swiglu_fp8 if fp8 else step.norm_proj_swiglu)(it["x"], it["Pg"], it["Pu"], it["y"], c.eps)
        else:
            (step.norm_proj_fp8 if fp8 else step.norm_proj)(it["x"], it["Pg"], it["y"], c.eps)
    step.record()
    graph_ms = time_region(torch, lambda _: step.launch(), args.steps, args.warmup)
    torch.cuda.synchronize()
    step.close()
    # the calls are independent: one grouped launch runs them all
    gstep = fn.Step()
    for it in items:
        c = it["call"]
        if c.swiglu:
            (gstep.norm_proj_swiglu_fp8 if fp8 else gstep.norm_proj_swiglu)(it["x"], it["Pg"], it["Pu"], it["y"], c.eps)
        else:
            (gstep.norm_proj_fp8 if fp8 else gstep.norm_proj)(it["x"], it["Pg"], it["y"], c.eps)
    gstep.record(grouped=True)
    grouped_ms = time_region(torch, lambda _: gstep.launch(), args.steps, args.warmup)
    torch.cuda.synchronize()
    gstep.close()
    result = {"ms": ms, "blocks": blocks, "hot_ms": None, "rot": 1, "graph_ms": graph_ms, "grouped_ms": grouped_ms,
              "wbytes": sum((it["Pg"].data.numel() + (it["Pg"].scales.numel() * 4 if fp8 else 0)) * it["call"].mats
                            for it in items)}
    if not args.no_chain:
        def chain_own(_):
            for it in items:
                c = it["call"]
                fn.rmsnorm(it["x"], it["g"], c.eps, out=it["xhat"])
                h = torch.matmul(it["xhat"], it["Wcat"])
                if c.swiglu:
                    fn.silu_mul(h, out=it["y"])

        def chain_torch(_):
            for it in items:
                c = it["call"]
                xn = torch.nn.functional.rms_norm(it["x"], (c.K,), it["g"], c.eps)
                h = torch.matmul(xn, it["Wcat"])
                if c.swiglu:
                    torch.mul(torch.nn.functional.silu(h[:, :c.N]), h[:, c.N:], out=it["y"])

        result["chain_own_ms"] = time_region(torch, chain_own, args.steps, args.warmup)
        result["chain_torch_ms"] = time_region(torch, chain_torch, args.steps, args.warmup)
    return calls, result


def measured_peak(torch, fn, bound):
    """What this GPU sustains, measured with the library's probes right after
    the timed region: a streaming read of 1 GiB (beyond the 256 MB
    Infinity Cache) for HBM, an MFMA-only loop (v_mfma_f32_16x16x32_bf16,
    register operands) for bf16 matrix work.  Median of five rounds of ten
    back-to-back calls."""
    times = []
    if bound == "hbm":
        buf = torch.empty(1 << 30, dtype=torch.uint8, device="cuda")
        buf.fill_(3)
        fn.probe_hbm_read(buf)
        work = float(buf.numel())
        call = lambda: fn.probe_hbm_read(buf)   # noqa: E731
        scale, unit = 1e9, "GB/s"
    else:
        iters, wgs = 2048, 2048
        fn.probe_mfma_bf16(iters, wgs)
        work = float(wgs * iters * fn.PROBE_MFMA_FLOPS_PER_WG_ITER)
        call = lambda: fn.probe_mfma_bf16(iters, wgs)   # noqa: E731
        scale, unit = 1e12, "TFLOP/s"
    torch.cuda.synchronize()
    for _ in range(5):   # five rounds of ten back-to-back calls
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record()
        for _ in range(10):
            call()
        e1.record()
        torch.cuda.synchronize()
        times.append(e0.elapsed_time(e1) * 1e-3 / 10)
    return round(work / pct(sorted(times), 0.5) / scale, 1), unit


def plain_read_us(torch, fn, nbytes):
    """The time of a plain streaming read of nbytes (fn_probe_hbm_read, 2048
    workgroups) from cold buffers (rotated over >= 1 GiB, beyond the 256 MB
    Infinity Cache): the floor a kernel that must read that many bytes meets
    on this GPU, fixed launch and ramp costs included.  Median of ten blocks
    of ten calls."""
    n16 = max(16, nbytes // 16 * 16)
    nbuf = max(2, -(-(1 << 30) // n16))
    bufs = [torch.empty(n16, dtype=torch.uint8, device="cuda").fill_(3) for _ in range(nbuf)]
    for i in range(nbuf):
        fn.probe_hbm_read(bufs[i])
    torch.cuda.synchronize()
    times = []
    j = 0
    for _ in range(10):
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record()
        for _ in range(10):
            fn.probe_hbm_read(bufs[j % nbuf])
            j += 1
        e1.record()
        torch.cuda.synchronize()
        times.append(e0.elapsed_time(e1) * 1e3 / 10)
    del bufs
    torch.cuda.empty_cache()
    return pct(sorted(times), 0.5)


def calibrate_copy(torch):
    n = 1 << 30
    a = torch.empty(n, dtype=torch.uint8, device="cuda")
    a.fill_(1)
    b = torch.empty_like(a)
    torch.cuda.synchronize()
    for _ in range(5):
        b.copy_(a)
    torch.cuda.synchronize()
    print(json.dumps({"calibrate_copy_bytes": n, "copies": 5}), flush=True)


def measure(args, torch, fn, workloads):
    """Run one workload as args describes; returns the measurement fields
    (the headline line's, or a config's)."""
    fp8 = args.weights == "fp8"
    q8 = args.output == "q8"
    adaln = args.prologue == "adaln"
    suffix = ("_fp8" if fp8 else "") + ("_q8" if q8 else "") + ("_adaln" if adaln else "")
    if args.workload == "decode_step":
        calls, r = run_decode_step(args, torch, fn, workloads)
        bytes_step = sum((fp8_bytes(c) if fp8 else c.algorithmic_bytes()) for c in calls)
        flops_step = sum(c.flops() for c in calls)
        rows, shard = calls[0].M, args.step_shard
        nq, nf, nh = calls[0].N, calls[1].N, calls[-1].N
        name = (f"32-layer decode step, M={rows}: 32 x (norm+QKV 4096->{nq}, norm+gate/up SwiGLU 4096->2x{nf}) + "
                f"norm+head 4096->{nh}" + (f" (one GPU's column share under {shard}-way tensor parallelism)"
                                          if shard > 1 else ""))
        config = {"workload": name, "calls_per_step": len(calls), "M": rows, "K": 4096, "shard": shard,
                  "weights_bytes": r["wbytes"],
                  "cache": f"cold ({r['wbytes'] / 1e9:.2f} GB of distinct weights per step)"}
        kernel = (fn.kernel_name_fp8(rows, 4096, nq, False) if fp8 else
                  fn.kernel_name(rows, 4096, nq, False, torch.bfloat16))
        cpu_call, cpu_inp = calls[-1], None
        unit = "GB/s"
        work = bytes_step
        roof = {"bound": "hbm", "peak": HBM_PEAK_GBS, "unit": "GB/s",
                "traffic": counter_traffic("decode_step" + suffix) if rows == 8 and shard == 1 else None}
        dtype = "bf16"
        per_unit = {"algorithmic_bytes_per_step": bytes_step, "flops_per_step": flops_step}
    else:
        call, inp, r = run_single(args, torch, fn, workloads)
        bytes_call = call_bytes(call, fp8, q8) + (adaln_extra_bytes(call) if adaln else 0)
        flops_call = call.flops()
        kernel = (fn.kernel_name_adaln_q8(call.M, call.K, call.N, ADALN_T, fp8) if adaln and q8 else
                  fn.kernel_name_adaln_fp8(call.M, call.K, call.N, ADALN_T, call.swiglu) if adaln and fp8 else
                  fn.kernel_name_adaln_ws(call.M, call.K, call.N, ADALN_T, call.swiglu) if adaln else
                  fn.kernel_name_q8(call.M, call.K, call.N, fp8) if q8 else
                  fn.kernel_name_fp8(call.M, call.K, call.N, call.swiglu) if fp8 else
                  fn.kernel_name(call.M, call.K, call.N, call.swiglu,
                                 torch.bfloat16 if call.dtype == "bf16" else torch.float32))
        config = {"workload": call.name, "M": call.M, "K": call.K, "N": call.N, "mats": call.mats,
                  "eps": call.eps, "kernel": kernel,
                  "cache": (f"cold ({r['rot']} rotated W' copies, {r['rot'] * r['wbytes'] / 2**30:.2f} GiB)"
                            if r["rot"] > 1 else "hot (one weight buffer)")}
        cpu_call, cpu_inp = call, inp
        dtype = call.dtype
        per_unit = {"algorithmic_bytes_per_call": bytes_call, "flops_per_call": flops_call}
        if args.workload == "prefill_qkv":
            unit, work = "TFLOP/s", flops_call
            roof = {"bound": "mfma", "peak": BF16_PEAK_TFLOPS, "unit": "TFLOP/s",
                    "traffic": counter_traffic(args.workload + suffix)}
        elif args.workload == "tiny":
            unit, work = "us/call", bytes_call
            roof = {"bound": "hbm", "peak": HBM_PEAK_GBS, "unit": "GB/s", "traffic": counter_traffic(args.workload),
                    "note": "launch-latency bound; the fraction is not meaningful here"}
        else:
            unit, work = "GB/s", bytes_call
            roof = {"bound": "hbm", "peak": HBM_PEAK_GBS, "unit": "GB/s",
                    "traffic": counter_traffic(args.workload + suffix)}
        if fp8:
            config["weights"] = "fp8 E4M3 codes + one fp32 scale per output column"
        if q8:
            config["output"] = "fp8 E4M3 codes + one fp32 scale per 16-column row block"
        if adaln:
            config["prologue"] = (f"AdaLN: h = RMSNorm_g(x) * (1 + scale[idx]) + shift[idx], tables of {ADALN_T} rows, "
                                  "per-row index, the gain folded into the fp32 modulation table"
                                  + (", two launches (adaln_modulate pre-pass, then the kernel named)"
                                     if fp8 or q8 or fn.adaln_workspace_bytes(call.M, call.K) else ", one launch"))
    # achieved: work per step / the region's mean step time (the kernel's
    # average launch duration for the single-kernel workloads); value: the
    # same work priced at the median block
    scale = 1e12 if roof["unit"] == "TFLOP/s" else 1e9
    med = pct(r["blocks"], 0.5)
    achieved = work / (r["ms"] * 1e-3) / scale
    roof["achieved"] = round(achieved, 6 if unit == "us/call" else 2)
    roof["frac"] = round(achieved / roof["peak"], 6 if unit == "us/call" else 4)
    roof = {k: roof[k] for k in ("bound", "achieved", "peak", "unit", "frac", "traffic", "note") if k in roof}
    value = med * 1e3 if unit == "us/call" else work / (med * 1e-3) / scale
    if args.measured_peak and roof["bound"] in ("hbm", "mfma") and unit != "us/call":
        peak, peak_unit = measured_peak(torch, fn, roof["bound"])
        if peak_unit == roof["unit"]:
            roof["measured_peak"] = peak
            roof["frac_measured"] = round(roof["achieved"] / peak, 4)
            roof["measured_peak_probe"] = ("fn_probe_hbm_read over 1 GiB" if roof["bound"] == "hbm"
                                           else "fn_probe_mfma_bf16 (MFMA-only loop)")
    if args.plain_read and roof["bound"] == "hbm" and unit != "us/call" and args.workload != "decode_step":
        # the same bytes read by a plain streaming kernel, cold: what a kernel
        # of this size can reach at all (launch and ramp included)
        pr = plain_read_us(torch, fn, int(work))
        roof["plain_read_same_bytes_us"] = round(pr, 3)
        roof["frac_of_plain_read"] = round(pr / (med * 1e3), 4)
    out = {
        "value": round(value, 4), "unit": unit, "steps": args.steps, "warmup": args.warmup,
        "ms_per_step": round(r["ms"], 6), "dtype": dtype, "config": config, "roofline": roof,
        "us_per_step": round(r["ms"] * 1e3, 3),
        "us_median_p10_p90": [round(pct(r["blocks"], q) * 1e3, 3) for q in (0.5, 0.1, 0.9)],
        "timing": f"{len(r['blocks'])} blocks of back-to-back steps, an event pair per block; "
                  "value at the median block, ms_per_step and roofline.achieved the region mean",
        "hot_us_per_step": None if r["hot_ms"] is None else round(r["hot_ms"] * 1e3, 3),
        "kernel": kernel,
        **per_unit,
    }
    if "graph_ms" in r:
        out["recorded_step"] = {"us_per_step" if args.workload == "decode_step" else "us_per_call":
                                round(r["graph_ms"] * 1e3, 3),
                                "speedup_vs_eager": round(r["ms"] / r["graph_ms"], 3),
                                "note": ("the same calls recorded once (fn_step_create), one graph launch per step"
                                         if args.workload == "decode_step" else
                                         f"{TINY_STEP_CALLS} calls recorded into one step (fn_step_create), "
                                         "one graph launch, time per call")}
    if r.get("grouped_ms") is not None:
        out["grouped_step"] = {"us_per_step": round(r["grouped_ms"] * 1e3, 3),
                               "speedup_vs_eager": round(r["ms"] / r["grouped_ms"], 3),
                               "weights_GB/s": round(r["wbytes"] / (r["grouped_ms"] * 1e-3) / 1e9, 2),
                               "note": "the same independent calls as one kernel launch (fn_step_create_grouped)"}
    if "bf16_ms" in r:
        out["bf16_weights_us"] = round(r["bf16_ms"] * 1e3, 3)
        out["speedup_vs_bf16_weights"] = round(r["bf16_ms"] / r["ms"], 3)
    if "chain_own_ms" in r:
        out["chain"] = {
            "own_rmsnorm_then_hipblaslt_us": round(r["chain_own_ms"] * 1e3, 3),
            "torch_rms_norm_then_matmul_us": round(r["chain_torch_ms"] * 1e3, 3),
            "fused_speedup_vs_own_chain": round(r["chain_own_ms"] / r["ms"], 3),
            "fused_speedup_vs_torch_chain": round(r["chain_torch_ms"] / r["ms"], 3),
        }
    if args.no_cpu_baseline and getattr(args, "parity_only", False) and r.get("y_head") is not None:
        cb = cpu_baseline(cpu_call, cpu_inp, 0.0, unit, fp8=fp8, q8=q8, adaln=adaln)
        if cb.get("_ref") is not None:
            out["parity"] = parity_report(r["y_head"], cb["_ref"])
    if not args.no_cpu_baseline:
        if cpu_inp is None:
            cpu_inp = workloads.make_inputs(cpu_call)
        cb = cpu_baseline(cpu_call, cpu_inp, args.cpu_seconds, unit if unit != "us/call" else "us/call", fp8=fp8,
                          q8=q8, adaln=adaln, one_thread_s=getattr(args, "one_thread_s", 0.0))
        per_call = cb.pop("seconds_per_call")
        ref = cb.pop("_ref", None)
        if ref is not None and r.get("y_head") is not None:
            out["parity"] = parity_report(r["y_head"], ref)
        if args.workload == "decode_step":
            # one head call sampled; scale to the whole step by algorithmic bytes
            step_s = per_call * bytes_step / (fp8_bytes(cpu_call) if fp8 else cpu_call.algorithmic_bytes())
            cb["value"] = round(bytes_step / step_s / 1e9, 4)
            cb["sample"] += "; scaled to the 65-call step by algorithmic bytes"
        out["cpu_baseline"] = cb
    return out


def main(argv=None):
    args = parse_args(argv)
    global CLOCK_WARMUP_S
    CLOCK_WARMUP_S = args.clock_warmup_s
    if args.gpus != 1:
        print(f"bench.py: --gpus {args.gpus} is not supported: libflashnorm runs on one GPU; "
              "the multi-GPU column split is a design note, not a measured path.", file=sys.stderr)
        return 2
    import torch
    import rmsnorm_projection_gemm_amd as fn
    import workloads
    if not torch.cuda.is_available():
        print("bench.py: no GPU visible", file=sys.stderr)
        return 1
    fn.load()
    if args.calibrate_copy:
        calibrate_copy(torch)
        return 0
    fp8 = args.weights == "fp8"
    if fp8 and args.workload == "tiny":
        print(f"bench.py: --weights fp8 applies to the bf16 workloads, not {args.workload}", file=sys.stderr)
        return 2
    q8 = args.output == "q8"
    if q8 and args.workload != "ffn_decode":
        print(f"bench.py: --output q8 applies to the SwiGLU workload ffn_decode, not {args.workload}", file=sys.stderr)
        return 2
    adaln = args.prologue == "adaln"
    if adaln and args.workload not in ("qkv_decode", "ffn_decode", "prefill_qkv"):
        print("bench.py: --prologue adaln applies to qkv_decode, ffn_decode and prefill_qkv", file=sys.stderr)
        return 2
    if not 1 <= args.step_rows <= 128:
        print("bench.py: --step-rows must be in 1..128", file=sys.stderr)
        return 2
    configs = [] if args.configs.strip() in ("", "none") else [c.strip() for c in args.configs.split(",")]
    bad = [c for c in configs if c not in CONFIG_CHOICES]
    if bad:
        print(f"bench.py: unknown config(s) {bad}; choose from {', '.join(CONFIG_CHOICES)}", file=sys.stderr)
        return 2

    # the headline: the workload named, with a one-thread CPU oracle figure
    head_args = argparse.Namespace(**vars(args))
    head_args.one_thread_s = min(5.0, args.cpu_seconds)
    head = measure(head_args, torch, fn, workloads)
    torch.cuda.empty_cache()
    sub = {}
    for name in configs:
        wl, weights = CONFIG_CHOICES[name]
        if (wl, weights) == (args.workload, args.weights) and not q8 and not adaln:
            continue    # the headline itself
        cargs = argparse.Namespace(**vars(args))
        cargs.workload, cargs.weights, cargs.output, cargs.prologue, cargs.hot = wl, weights, "native", "none", False
        cargs.steps, cargs.warmup = CONFIG_STEP_CAP.get(wl, (args.steps, args.warmup))
        cargs.steps, cargs.warmup = min(cargs.steps, args.steps), min(cargs.warmup, args.warmup)
        cargs.measured_peak = False
        if weights == "fp8":
            cargs.no_chain, cargs.no_cpu_baseline = True, True    # timing only; bf16 beside it in its own config
            cargs.parity_only = True                              # one untimed oracle call for the parity report
        sub[name] = measure(cargs, torch, fn, workloads)
        torch.cuda.empty_cache()

    out = {
        "metric": METRIC,
        "value": head["value"],
        "unit": head["unit"],
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": head["ms_per_step"],
        "higher_is_better": head["unit"] != "us/call",
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": head["dtype"],
        "data": "synthetic (seeded; random-init weights of the named shapes)",
        "config": head["config"],
        "roofline": head["roofline"],
    }
    if "cpu_baseline" in head:
        out["cpu_baseline"] = head["cpu_baseline"]
    for k, v in head.items():
        if k not in out and k not in ("config", "roofline", "cpu_baseline", "dtype"):
            out[k] = v
    if sub:
        out["configs"] = sub
    print(json.dumps(out), flush=True)
    return 0


if __name__ == "__main__":
    sys.exit(main())
