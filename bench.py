#!/usr/bin/env python3
"""Benchmark of the H-BitLinear forward (BitNet v2) on one MI355X.

A step is one pass of the whole layer over one batch: the fused RMSNorm +
Hadamard + quantisation kernel, then the ternary matmul with its dequant
epilogue (fp6 x fp4 matrix instruction for INT4 activations at prefill sizes,
int8 MFMA otherwise): the two kernels hbl_forward_int{8,4} launches.  Inputs are
seeded synthetic data already resident in device memory when timing starts.
Default workload: 7B-shaped FFN down projection, M=8192 tokens, K=16384,
N=4096, INT4 activations, bf16 in/out.

Prints one JSON line on stdout.  Extra context (INT8 path, decode shapes,
weight ternarisation) goes into extra keys of the same line.
"""
from __future__ import annotations

import argparse
import hashlib
import json
import os
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

METRIC = "H-BitLinear tokens/s + effective int TOPS & HBM GB/s vs roofline, 7B Wdown"
PEAK_INT8_TOPS = 5000.0      # MI355X dense int8 MFMA, TOP/s
PEAK_FP6_TFLOPS = 10100.0    # MI355X dense fp6 / fp4 MFMA, TFLOP/s
PEAK_HBM_GBS = 8000.0        # MI355X HBM3E, GB/s
PEAK_BF16_TFLOPS = 2500.0    # MI355X dense bf16 MFMA, TFLOP/s
TRAFFIC_FILE = os.path.join(ROOT, "profiles", "wdown_7b_int4_hbm_traffic.txt")
GEMM_SOURCES = [os.path.join(ROOT, "hadamard_rotated_ternary_amd", "csrc", f)
                for f in ("gemm.hip", "common.h", "mma.h", "copy_schedule.h")]


def log(*a):
    print(*a, file=sys.stderr, flush=True)


def gemm_source_sha() -> str:
    h = hashlib.sha256()
    for p in GEMM_SOURCES:
        with open(p, "rb") as f:
            h.update(f.read())
    return h.hexdigest()[:16]


def algorithmic_bytes(M, K, N, x_bytes=2, y_bytes=2):
    """What the layer itself must move: activations in, packed weights once, outputs out."""
    return M * K * x_bytes + N * K // 4 + M * N * y_bytes


def parse():
    ap = argparse.ArgumentParser(description=__doc__, formatter_class=argparse.RawDescriptionHelpFormatter)
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=50)
    ap.add_argument("--warmup", type=int, default=20)
    ap.add_argument("--workload", default="wdown_7b_int4")
    ap.add_argument("--no-extras", action="store_true", help="skip the INT8 and decode side measurements")
    ap.add_argument("--no-cpu", action="store_true", help="skip the CPU oracle baseline")
    ap.add_argument("--cpu-seconds", type=float, default=12.0, help="wall-clock budget of the CPU baseline")
    ap.add_argument("--extra", choices=["layers", "decode", "attention", "backward"], default=None,
                    help="run only this group of side measurements (for profiling one kernel family)")
    ap.add_argument("--copy-calibration", action="store_true",
                    help="also run a plain 1 GiB device copy (reference for HBM byte counters)")
    return ap.parse_args()


def main():
    args = parse()
    if args.gpus != 1:
        print(f"bench.py measures one GPU only (asked for --gpus {args.gpus}); the library has no "
              "multi-GPU sharding.", file=sys.stderr)
        sys.exit(2)
    import torch
    import hadamard_rotated_ternary_amd as hbl
    import synthetic

    assert torch.cuda.is_available(), "needs an MI355X"
    props = torch.cuda.get_device_properties(0)
    if "gfx950" not in props.gcnArchName:
        raise SystemExit(f"not a gfx950 device: {props.gcnArchName}")
    hbl.lib()

    w = synthetic.WORKLOADS[args.workload]
    M, K, N, bits = w.M, w.K, w.N, w.bits
    log(f"[bench] workload {w.name}: M={M} K={K} N={N} INT{bits} x={w.x_dtype}")
    x, xb, wl = synthetic.make_inputs(w)
    xd = torch.from_numpy(xb.view(np.int16)).cuda().view(torch.bfloat16) if xb is not None else torch.from_numpy(x).cuda()
    wd = torch.from_numpy(wl).cuda()

    # ---- offline weight ternarisation (not part of a step; reported for information)
    wp, a = hbl.quantize_weights(wd)
    torch.cuda.synchronize()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record()
    for _ in range(3):
        hbl.quantize_weights(wd)
    e1.record()
    torch.cuda.synchronize()
    wq_ms = e0.elapsed_time(e1) / 3
    # the weight + activation rotation variant: rows rotated, then ternarised
    hbl.quantize_weights(wd, rotate=True)
    torch.cuda.synchronize()
    e0.record()
    for _ in range(3):
        hbl.quantize_weights(wd, rotate=True)
    e1.record()
    torch.cuda.synchronize()
    wq_rot_ms = e0.elapsed_time(e1) / 3

    if args.copy_calibration:
        src = torch.empty(1 << 30, dtype=torch.uint8, device="cuda")
        dst = torch.empty_like(src)
        for _ in range(3):
            dst.copy_(src)
        torch.cuda.synchronize()
        del src, dst

    res = time_layer(torch, hbl, xd, wp, a, M, K, N, bits, args.steps, args.warmup)
    step_s = res["ms_per_step"] / 1e3
    gemm_s = res["gemm_ms"] / 1e3
    ops = 2.0 * M * N * K
    achieved = ops / gemm_s / 1e12
    traffic = stored_traffic(args.workload)
    fp6 = bits == 4 and M > 64
    kernel, peak = ("gemm_fp6_kernel", PEAK_FP6_TFLOPS) if fp6 else ("gemm_prefill_kernel", PEAK_INT8_TOPS)

    out = {
        "metric": METRIC,
        "value": M / step_s,
        "unit": "tokens/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": res["ms_per_step"],
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "fp6xfp4" if fp6 else "i8",
        "data": "synthetic",
        "config": {"workload": w.name, "M": M, "K": K, "N": N, "activation_bits": bits,
                   "x_dtype": w.x_dtype, "y_dtype": w.x_dtype, "parallelism": "single-gpu"},
        "effective_int_tops": ops / step_s / 1e12,
        "hbm_gbps_algorithmic": algorithmic_bytes(M, K, N) / step_s / 1e9,
        "roofline": {"kernel": kernel, "bound": "mfma", "achieved": achieved,
                     "peak": peak, "unit": "TFLOP/s", "frac": achieved / peak,
                     "traffic": traffic},
        "kernels": {
            "prep_ms": res["prep_ms"], "gemm_ms": res["gemm_ms"],
            "prep_gbps_impl": (M * K * 2 + M * hbl.codes_row_bytes(6 if fp6 else bits, K) + M * 4)
                              / (res["prep_ms"] / 1e3) / 1e9,
            "gemm_tops": achieved,
            "step_ms_median": res["step_ms_median"], "step_ms_min": res["step_ms_min"],
            "forward_entry_ms": res["forward_ms"], "forward_entry_calls": res["forward_calls"],
        },
        "inputs": res["rotation"],
        "weight_ternarise_ms": wq_ms,
        "weight_rotate_ternarise_ms": wq_rot_ms,
    }
    if not args.no_extras:
        out["extras"] = extras(torch, hbl, synthetic, args)
    if not args.no_cpu:
        out["cpu_baseline"] = cpu_baseline(x, wl, bits, args.cpu_seconds)
    print(json.dumps(out), flush=True)


def rotation_sets(torch, xd, wp, total_bytes=512 << 20):
    """Distinct input/weight copies cycled through by consecutive steps, so that
    the working set of a step sequence exceeds the 256 MB Infinity Cache
    (MALL): nothing is served from it across steps that a real layer stack
    would have evicted.  Returns (xs, ws) and a description."""
    per = xd.numel() * xd.element_size() + wp.numel()
    n = max(1, -(-total_bytes // per))
    xs = [xd] + [xd.clone() for _ in range(n - 1)]
    ws = [wp] + [wp.clone() for _ in range(n - 1)]
    return xs, ws, f"{n} activation/weight buffer sets rotated ({n * per / 2**20:.0f} MiB)"


def time_layer(torch, hbl, xd, wp, a, M, K, N, bits, steps, warmup, rotate=True):
    """Per-kernel times from the two stage calls with events between the
    kernels (their launch average is what the roofline uses); then `warmup`
    and `steps` single-call forwards, the latter timed back to back (wall
    clock between synchronisations).  The stage calls launch the same kernels as the
    single-call forward (the INT4 forward of more than 64 tokens keeps its
    codes in the fp6 operand layout, format 6).  Consecutive steps cycle through distinct activation and
    weight copies (rotation_sets)."""
    xs, wps, rot = rotation_sets(torch, xd, wp)
    sb = 6 if bits == 4 and M > 64 else bits
    codes = torch.empty(hbl.codes_shape(sb, M, K), dtype=torch.int8 if bits == 8 else torch.uint8, device="cuda")
    d = torch.empty(M + 4, dtype=torch.float32, device="cuda")[:M]
    y = torch.empty((M, N), dtype=xd.dtype, device="cuda")
    ws = torch.empty(max(hbl.workspace_bytes(hbl.OP_MATMUL, M, K, N), 16), dtype=torch.uint8, device="cuda")
    wsf = torch.empty(max(hbl.workspace_bytes(hbl.OP_FORWARD_INT8 if bits == 8 else hbl.OP_FORWARD_INT4, M, K, N), 16),
                      dtype=torch.uint8, device="cuda")

    def step(i, evs=None):
        if evs: evs[0].record()
        hbl.quantize_act(xs[i % len(xs)], sb, out=(codes, d), rotate=rotate)
        if evs: evs[1].record()
        hbl.matmul_dequant(codes, sb, d, wps[i % len(wps)], a, K, workspace=ws, out=y)
        if evs: evs[2].record()

    def forward(i):
        hbl.forward(xs[i % len(xs)], wps[i % len(wps)], a, bits, workspace=wsf, out=y, rotate=rotate)

    # per-kernel times first (untimed for the headline; it also brings the
    # clocks to their sustained state): the same kernels through the two
    # stage calls, events between them
    for i in range(max(50, warmup)):
        step(i)
    evs = [[torch.cuda.Event(enable_timing=True) for _ in range(3)] for _ in range(steps)]
    for i in range(steps):
        step(i, evs[i])
    torch.cuda.synchronize()
    prep = float(np.mean([e[0].elapsed_time(e[1]) for e in evs]))
    gemm = float(np.mean([e[1].elapsed_time(e[2]) for e in evs]))
    per_step = [e[0].elapsed_time(e[2]) for e in evs]
    # the timed region: `warmup` untimed calls, then exactly `steps` calls of the
    # public single-call forward (hbl_forward_int4 / _int8: both kernels
    # launched by one library call), back to back, nothing else on the stream
    for i in range(warmup):
        forward(i)
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for i in range(steps):
        forward(i)
    torch.cuda.synchronize()
    t1 = time.perf_counter()
    # >= 200 back-to-back single calls between two events
    calls = max(200, steps)
    f0, f1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    f0.record()
    for i in range(calls):
        forward(i)
    f1.record()
    torch.cuda.synchronize()
    return {"ms_per_step": (t1 - t0) * 1e3 / steps, "prep_ms": prep, "gemm_ms": gemm,
            "step_ms_median": float(np.median(per_step)), "step_ms_min": float(np.min(per_step)),
            "forward_ms": f0.elapsed_time(f1) / calls, "forward_calls": calls, "rotation": rot}


def stored_traffic(workload):
    """HBM bytes per matmul launch from the committed rocprofv3 counter runs
    (FETCH_SIZE and WRITE_SIZE, scaled by a 1 GiB copy), if they were taken on
    the current matmul source and this workload; otherwise None."""
    try:
        with open(TRAFFIC_FILE) as f:
            kv = dict(line.split(":", 1) for line in f if ":" in line and not line.startswith("#"))
    except OSError:
        return None
    kv = {k.strip(): v.strip() for k, v in kv.items()}
    if kv.get("source_sha") != gemm_source_sha() or kv.get("workload") != workload:
        return None
    return int(kv["bytes_per_launch"])


ATTN_PROFILE = os.path.join(ROOT, "profiles", "decode_attn_7b_kv3_rocprof.txt")


def attn_source_sha() -> str:
    h = hashlib.sha256()
    for f in ("attn.hip", "common.h", "fwht.h"):
        with open(os.path.join(ROOT, "hadamard_rotated_ternary_amd", "csrc", f), "rb") as fh:
            h.update(fh.read())
    return h.hexdigest()[:16]


def stored_attn_traffic():
    """HBM bytes per decode-attention launch from the committed counter runs,
    if they were taken on the current attention source; otherwise None."""
    try:
        with open(ATTN_PROFILE) as f:
            kv = dict(line.split(":", 1) for line in f if ":" in line and not line.startswith("#"))
    except OSError:
        return None
    kv = {k.strip(): v.strip() for k, v in kv.items()}
    if kv.get("source_sha") != attn_source_sha():
        return None
    return int(kv["attn_bytes_per_launch"])


def layer_config_extra(torch, hbl, synthetic, name, steps):
    """One prefill-shaped configuration end to end: tokens/s of the
    single-call forward, per-kernel times from the stage calls, effective int
    TOPS (2MNK per step), the matmul against its instruction's peak (fp6 x fp4
    10.1 P for INT4 beyond 64 tokens, int8 5.0 P otherwise) and prep against
    8 TB/s (its own bytes: activations in, codes and scales out)."""
    w = synthetic.WORKLOADS[name]
    x, xb, wl = synthetic.make_inputs(w)
    xd = torch.from_numpy(xb.view(np.int16)).cuda().view(torch.bfloat16) if xb is not None else torch.from_numpy(x).cuda()
    wp, a = hbl.quantize_weights(torch.from_numpy(wl).cuda())
    r = time_layer(torch, hbl, xd, wp, a, w.M, w.K, w.N, w.bits, steps, 5)
    ops = 2.0 * w.M * w.N * w.K
    fp6 = w.bits == 4 and w.M > 64
    peak = PEAK_FP6_TFLOPS if fp6 else PEAK_INT8_TOPS
    xb_ = xd.element_size()
    prep_bytes = w.M * w.K * xb_ + w.M * hbl.codes_row_bytes(6 if fp6 else w.bits, w.K) + w.M * 4
    gemm_tops = ops / (r["gemm_ms"] / 1e3) / 1e12
    res = {"M": w.M, "K": w.K, "N": w.N, "activation_bits": w.bits,
           "matmul": "fp6xfp4" if fp6 else "i8",
           "tokens_per_s": w.M / (r["ms_per_step"] / 1e3), "ms_per_step": r["ms_per_step"],
           "effective_int_tops": ops / (r["ms_per_step"] / 1e3) / 1e12,
           "hbm_gbps_algorithmic": algorithmic_bytes(w.M, w.K, w.N, xb_, xb_) / (r["ms_per_step"] / 1e3) / 1e9,
           "prep_ms": r["prep_ms"], "gemm_ms": r["gemm_ms"],
           "gemm_tops": gemm_tops, "gemm_peak_tops": peak, "gemm_frac": gemm_tops / peak,
           "prep_gbps": prep_bytes / (r["prep_ms"] / 1e3) / 1e9,
           "prep_hbm_frac": prep_bytes / (r["prep_ms"] / 1e3) / 1e9 / PEAK_HBM_GBS}
    del xd, wp
    return res


def int4_on_int8_extra(torch, hbl, synthetic, steps):
    """The 7B Wdown INT4 matmul on the int8 matrix instruction (INT4 nibble
    codes unpacked to int8 in registers, 2-bit weights expanded in
    registers): the stage call with format 4, against the 5.0 P dense int8
    peak.  The forward runs this shape on the fp6 x fp4 instruction instead
    (bit-identical results at twice the instruction rate)."""
    w = synthetic.WORKLOADS["wdown_7b_int4"]
    x, xb, wl = synthetic.make_inputs(w)
    xd = torch.from_numpy(xb.view(np.int16)).cuda().view(torch.bfloat16)
    wp, a = hbl.quantize_weights(torch.from_numpy(wl).cuda())
    codes, d = hbl.quantize_act(xd, 4)
    y = torch.empty((w.M, w.N), dtype=torch.bfloat16, device="cuda")
    ws = torch.empty(max(hbl.workspace_bytes(hbl.OP_MATMUL, w.M, w.K, w.N), 16), dtype=torch.uint8, device="cuda")
    wps = [wp, wp.clone()]
    for i in range(5):
        hbl.matmul_dequant(codes, 4, d, wps[i % 2], a, w.K, workspace=ws, out=y)
    torch.cuda.synchronize()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record()
    for i in range(steps):
        hbl.matmul_dequant(codes, 4, d, wps[i % 2], a, w.K, workspace=ws, out=y)
    e1.record()
    torch.cuda.synchronize()
    ms = e0.elapsed_time(e1) / steps
    tops = 2.0 * w.M * w.N * w.K / (ms / 1e3) / 1e12
    del xd, wp, wps, codes
    return {"M": w.M, "K": w.K, "N": w.N, "kernel": "gemm_prefill_kernel (INT4 codes, int8 MFMA)", "gemm_ms": ms,
            "gemm_tops": tops, "gemm_frac_int8_peak": tops / PEAK_INT8_TOPS}


def tiny_extra(torch, hbl, synthetic):
    """The smallest configuration (8 tokens, K = N = 256, fp32): per-call
    time of the single-call forward (latency; 1 us is a launch)."""
    w = synthetic.WORKLOADS["tiny_int8"]
    x, _, wl = synthetic.make_inputs(w)
    xd = torch.from_numpy(x).cuda()
    wp, a = hbl.quantize_weights(torch.from_numpy(wl).cuda())
    y = torch.empty((w.M, w.N), dtype=torch.float32, device="cuda")
    ws = torch.empty(max(hbl.workspace_bytes(hbl.OP_FORWARD_INT8, w.M, w.K, w.N), 16), dtype=torch.uint8, device="cuda")
    for _ in range(20):
        hbl.forward(xd, wp, a, 8, workspace=ws, out=y)
    torch.cuda.synchronize()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record()
    for _ in range(200):
        hbl.forward(xd, wp, a, 8, workspace=ws, out=y)
    e1.record()
    torch.cuda.synchronize()
    us = 1e3 * e0.elapsed_time(e1) / 200
    # the same calls replayed from a captured graph (device time, no host launch cost)
    s_ = torch.cuda.Stream()
    s_.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(s_):
        hbl.forward(xd, wp, a, 8, workspace=ws, out=y)
    torch.cuda.current_stream().wait_stream(s_)
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        for _ in range(40):
            hbl.forward(xd, wp, a, 8, workspace=ws, out=y)
    g.replay()
    torch.cuda.synchronize()
    e0.record()
    for _ in range(10):
        g.replay()
    e1.record()
    torch.cuda.synchronize()
    gus = 1e3 * e0.elapsed_time(e1) / 400
    return {"M": w.M, "K": w.K, "N": w.N, "forward_us": us, "tokens_per_s": w.M / (us / 1e6),
            "forward_us_graph": gus, "tokens_per_s_graph": w.M / (gus / 1e6),
            "timing": "events around 200 back-to-back calls (host launch rate included); graph: 40 calls "
                      "replayed 10 times"}


def extras(torch, hbl, synthetic, args):
    out = {}
    steps = max(10, args.steps // 2)

    def want(group):
        return args.extra in (None, group)
    if want("layers"):
        # every other configuration of the layer, end to end
        for name in ("wo_1p3b_int4", "wdown_3b_int4", "wo_7b_int8", "wo_7b_int4"):
            out[name] = layer_config_extra(torch, hbl, synthetic, name, steps)
        out["wdown_7b_int4_on_int8_mfma"] = int4_on_int8_extra(torch, hbl, synthetic, steps)
        out["tiny_int8"] = tiny_extra(torch, hbl, synthetic)
        # INT8 activations on the same 7B Wdown shape
        w8 = synthetic.WORKLOADS["wdown_7b_int8"]
        x, xb, wl = synthetic.make_inputs(w8)
        xd = torch.from_numpy(xb.view(np.int16)).cuda().view(torch.bfloat16)
        wp, a = hbl.quantize_weights(torch.from_numpy(wl).cuda())
        r = time_layer(torch, hbl, xd, wp, a, w8.M, w8.K, w8.N, 8, max(10, args.steps // 2), 5)
        ops = 2.0 * w8.M * w8.N * w8.K
        out["wdown_7b_int8"] = {"tokens_per_s": w8.M / (r["ms_per_step"] / 1e3), "ms_per_step": r["ms_per_step"],
                                "prep_ms": r["prep_ms"], "gemm_ms": r["gemm_ms"],
                                "gemm_tops": ops / (r["gemm_ms"] / 1e3) / 1e12,
                                "gemm_mfma_frac": ops / (r["gemm_ms"] / 1e3) / 1e12 / PEAK_INT8_TOPS}
        del xd, wp
        # BitLinear without the rotation on a 7B-scale FFN input projection
        wu = synthetic.WORKLOADS["up_7b_bitlinear_int4"]
        x, xb, wl = synthetic.make_inputs(wu)
        xd = torch.from_numpy(xb.view(np.int16)).cuda().view(torch.bfloat16)
        wp, a = hbl.quantize_weights(torch.from_numpy(wl).cuda())
        r = time_layer(torch, hbl, xd, wp, a, wu.M, wu.K, wu.N, 4, max(10, args.steps // 2), 5, rotate=False)
        ops = 2.0 * wu.M * wu.N * wu.K
        out[wu.name] = {"tokens_per_s": wu.M / (r["ms_per_step"] / 1e3), "ms_per_step": r["ms_per_step"],
                        "prep_ms": r["prep_ms"], "gemm_ms": r["gemm_ms"], "M": wu.M, "K": wu.K, "N": wu.N,
                        "gemm_tflops": ops / (r["gemm_ms"] / 1e3) / 1e12,
                        "gemm_frac_fp6": ops / (r["gemm_ms"] / 1e3) / 1e12 / PEAK_FP6_TFLOPS}
        del xd, wp
    if want("decode"):
        # decode shapes: weights rotated over enough copies to defeat the 256 MB
        # Infinity Cache; calls replayed from a captured graph so the timing is
        # not bound by host launch overhead.
        base = synthetic.WORKLOADS["decode_7b_m64"]
        x, xb, wl = synthetic.make_inputs(base)
        wp0, a = hbl.quantize_weights(torch.from_numpy(wl).cuda())
        R = 40
        wps = [wp0.clone() for _ in range(R)]
        xfull = torch.from_numpy(xb.view(np.int16)).cuda().view(torch.bfloat16)

        def graph_time(body):
            s_ = torch.cuda.Stream()
            s_.wait_stream(torch.cuda.current_stream())
            with torch.cuda.stream(s_):
                for i in range(3):
                    body(i)
            torch.cuda.current_stream().wait_stream(s_)
            g = torch.cuda.CUDAGraph()
            with torch.cuda.graph(g):
                for i in range(R):
                    body(i)
            g.replay()
            torch.cuda.synchronize()
            f0, f1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            f0.record()
            for _ in range(10):
                g.replay()
            f1.record()
            torch.cuda.synchronize()
            return 1e3 * f0.elapsed_time(f1) / (10 * R)

        for M in (1, 16, 64):
            xd = xfull[:M].contiguous()
            codes, d = hbl.quantize_act(xd, 4)
            ws = torch.empty(max(hbl.workspace_bytes(hbl.OP_MATMUL, M, base.K, base.N), 16), dtype=torch.uint8, device="cuda")
            wsf = torch.empty(hbl.workspace_bytes(hbl.OP_FORWARD_INT4, M, base.K, base.N), dtype=torch.uint8, device="cuda")
            y = torch.empty((M, base.N), dtype=torch.bfloat16, device="cuda")
            y_eager = hbl.matmul_dequant(codes, 4, d, wps[0], a, base.K, workspace=ws)
            f_eager = hbl.forward(xd, wps[0], a, 4, workspace=wsf)
            res = {}
            codes2, d2 = torch.empty_like(codes), torch.empty_like(d)
            for kind in ("gemm", "forward", "prep"):
                def body(i):
                    if kind == "gemm":
                        hbl.matmul_dequant(codes, 4, d, wps[i % R], a, base.K, workspace=ws, out=y)
                    elif kind == "forward":
                        hbl.forward(xd, wps[i % R], a, 4, workspace=wsf, out=y)
                    else:
                        hbl.quantize_act(xd, 4, out=(codes2, d2))
                s_ = torch.cuda.Stream()
                s_.wait_stream(torch.cuda.current_stream())
                with torch.cuda.stream(s_):
                    for i in range(3):
                        body(i)
                torch.cuda.current_stream().wait_stream(s_)
                g = torch.cuda.CUDAGraph()
                with torch.cuda.graph(g):
                    for i in range(R):
                        body(i)
                reps = 10
                g.replay()
                torch.cuda.synchronize()
                f0, f1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
                f0.record()
                for _ in range(reps):
                    g.replay()
                f1.record()
                torch.cuda.synchronize()
                res[kind] = 1e3 * f0.elapsed_time(f1) / (reps * R)
                # the last captured call used wps[R-1], a copy of wps[0]: same result as eager
                if kind != "prep":
                    ref = y_eager if kind == "gemm" else f_eager
                    assert torch.equal(y, ref), f"graph replay differs from eager ({kind}, M={M})"
            gbytes = base.N * base.K / 4 + M * base.K / 2 + M * base.N * 2 + M * 4
            # inside the forward, 5..64 tokens, the matmul reads its codes in the
            # decode-blocked layout (the stage call above reads row-major codes):
            # its time is the forward's less a prep stage call of the same tokens
            # (one token: the forward is a single fused kernel, no prep stage)
            out[f"decode_7b_m{M}"] = {"gemm_us": res["gemm"], "gemm_gbps": gbytes / (res["gemm"] / 1e6) / 1e9,
                                      "gemm_hbm_frac": gbytes / (res["gemm"] / 1e6) / 1e9 / PEAK_HBM_GBS,
                                      "forward_us": res["forward"], "tokens_per_s": M / (res["forward"] / 1e6),
                                      "timing": f"graph replay of {R} back-to-back calls over {R} weight copies"}
            if M >= 5:
                fg = res["forward"] - res["prep"]
                out[f"decode_7b_m{M}"].update({"prep_us": res["prep"], "forward_gemm_us": fg,
                                               "forward_gemm_hbm_frac": gbytes / (fg / 1e6) / 1e9 / PEAK_HBM_GBS})
                # every workgroup of the matmul reads all M tokens' codes
                # (M K / 2 bytes) from L2: the same bytes read by 256
                # workgroups, nothing else, in the same harness
                bdig = torch.empty((256,), dtype=torch.int32, device="cuda")
                cf = graph_time(lambda i: hbl.broadcast_read(codes, 256, bdig))
                out[f"decode_7b_m{M}"].update({"code_broadcast_read_us": cf,
                                               "code_broadcast_bytes_per_wg": codes.numel() * codes.element_size()})
        # a plain read of one 16 MiB weight copy per call in the same
        # graph-replay harness over the same 40 copies: the hand-written
        # streaming read (libhbl_calib.so: 64 KiB per workgroup, 1 KiB per wave
        # instruction, every load issued up front), and a torch row-wise
        # max-reduction (4096 rows of 4 KiB) as a library reference
        red = torch.empty((base.N,), dtype=torch.int64, device="cuda")
        dig = torch.empty((base.N * base.K // 4 // 65536,), dtype=torch.int32, device="cuda")

        read_us = graph_time(lambda i: hbl.stream_read(wps[i % R], dig))
        lib_us = graph_time(lambda i: torch.amax(wps[i % R].view(torch.int64), dim=1, out=red))
        wbytes = base.N * base.K / 4
        out["plain_read_16mib"] = {"us": read_us, "gbps": wbytes / (read_us / 1e6) / 1e9,
                                   "hbm_frac": wbytes / (read_us / 1e6) / 1e9 / PEAK_HBM_GBS,
                                   "library_read_us": lib_us,
                                   "timing": f"graph replay of {R} streaming reads (hbl_calib_stream_read), one "
                                             f"{R}-way rotated weight copy each; library_read_us: torch row-wise "
                                             "max-reductions of the same copies"}
        for M in (1, 16, 64):
            e = out[f"decode_7b_m{M}"]
            e["gemm_over_plain_read"] = e["gemm_us"] / read_us
            # the matmul's floor: the weight stream (plain read) or the code
            # stream through L2 (broadcast read), whichever is longer
            e["gemm_floor_us"] = max(read_us, e.get("code_broadcast_read_us", 0.0))
            e["forward_gemm_over_floor"] = e.get("forward_gemm_us", e["gemm_us"]) / e["gemm_floor_us"]
    if want("attention"):
        out["decode_attn_7b_kv3"] = attention_extra(torch, hbl, synthetic, args)
    if want("backward"):
        out["backward_wdown_7b_int4"] = backward_extra(torch, hbl, synthetic, args)
    return out


def backward_extra(torch, hbl, synthetic, args):
    """Straight-through backward of the same 7B-shaped Wdown layer (INT4):
    input gradient (bf16 product, transform, RMSNorm backward), gain gradient
    and latent-weight gradient, from the forward's codes."""
    w = synthetic.WORKLOADS["wdown_7b_int4"]
    x, xb, wl = synthetic.make_inputs(w)
    xd = torch.from_numpy(xb.view(np.int16)).cuda().view(torch.bfloat16)
    wp, a = hbl.quantize_weights(torch.from_numpy(wl).cuda())
    wbt = hbl.backward_weights(wp, w.K)
    codes, d = hbl.quantize_act(xd, 4)
    rng = np.random.Generator(np.random.PCG64(w.seed + 77))
    dyb = synthetic.f32_to_bf16_bits(rng.normal(0.0, 1.0, (w.M, w.N)).astype(np.float32))
    dy = torch.from_numpy(dyb.view(np.int16)).cuda().view(torch.bfloat16)
    g = torch.from_numpy(synthetic.make_gain(w.K, w.seed)).cuda()
    ws = torch.empty(hbl.workspace_bytes(hbl.OP_BACKWARD, w.M, w.K, w.N), dtype=torch.uint8, device="cuda")
    for _ in range(3):
        hbl.backward(xd, g, codes, 4, d, wbt, a, dy, workspace=ws)
    torch.cuda.synchronize()
    n = max(5, args.steps // 5)
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record()
    for _ in range(n):
        hbl.backward(xd, g, codes, 4, d, wbt, a, dy, workspace=ws)
    e1.record()
    torch.cuda.synchronize()
    ms = e0.elapsed_time(e1) / n
    flops = 2 * 2.0 * w.M * w.N * w.K            # two products of 2MNK each
    # context, not part of the path: the input-gradient product dy . W_t
    # through the library GEMM (torch.mm, hipBLASLt) on the same operands
    wt = wbt.t().contiguous()                     # [N][K] bf16
    lib = {}
    for name, fn in (("bf16_out", lambda: torch.mm(dy, wt)),
                     ("fp32_out", lambda: torch.mm(dy, wt, out_dtype=torch.float32))):
        try:
            for _ in range(2):
                fn()
            torch.cuda.synchronize()
            e0.record()
            for _ in range(n):
                fn()
            e1.record()
            torch.cuda.synchronize()
            lib[name] = e0.elapsed_time(e1) / n
        except (TypeError, RuntimeError):
            lib[name] = None
    del wt
    return {"M": w.M, "K": w.K, "N": w.N, "ms_per_step": ms, "tokens_per_s": w.M / (ms / 1e3),
            "matmul_tflops_if_all_time": flops / (ms / 1e3) / 1e12,
            "library_dxh_product_ms": lib,
            "timing": "events around back-to-back hbl_backward calls (both products, transform, norm, gain and "
                      "weight gradients); per-kernel split in the rocprofv3 trace; library_dxh_product_ms: "
                      "torch.mm of the same dy and ternary weights, for comparison with one product's kernel time"}


def attention_extra(torch, hbl, synthetic, args):
    """Low-bit attention states: prefill of a 3-bit KV cache and one decode
    step of attention over it (7B-shaped heads)."""
    w = synthetic.ATTN_WORKLOADS["decode_attn_7b_kv3"]
    q, k, v = synthetic.make_heads(w)
    dev = lambda a: torch.from_numpy(a.view(np.int16)).cuda().view(torch.bfloat16)
    qd, kd, vd = dev(q), dev(k), dev(v)
    del k, v
    cache = hbl.KVCache(w.B, w.Hkv, w.T, w.d, w.kv_bits)
    lens = torch.full((w.B,), w.T, dtype=torch.int32, device="cuda")
    ws = torch.empty(max(hbl.attention_workspace_bytes(w.B, w.Hq, w.d, w.T), 16), dtype=torch.uint8,
                     device="cuda")
    out = torch.empty((w.B, w.Hq, w.d), dtype=torch.bfloat16, device="cuda")

    def timed(fn, n):
        for _ in range(3):
            fn()
        torch.cuda.synchronize()
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record()
        for _ in range(n):
            fn()
        e1.record()
        torch.cuda.synchronize()
        return 1e3 * e0.elapsed_time(e1) / n

    t_app = timed(lambda: cache.append(kd, vd), 10)
    t_dec = timed(lambda: hbl.attention_decode(qd, w.q_bits, cache.k_codes, cache.k_scale, cache.v_codes,
                                               cache.v_scale, w.kv_bits, lens, workspace=ws, out=out), 50)
    rows = w.B * w.Hkv * w.T
    row_bytes = w.d * w.kv_bits // 8 + 4
    cache_bytes = 2 * rows * row_bytes
    dec_bytes = cache_bytes + w.B * w.Hq * w.d * 4
    app_bytes = 2 * rows * w.d * 2 + cache_bytes
    res = {"B": w.B, "Hq": w.Hq, "Hkv": w.Hkv, "d": w.d, "T": w.T, "kv_bits": w.kv_bits, "q_bits": w.q_bits,
           "decode_us": t_dec, "decode_gbps": dec_bytes / (t_dec / 1e6) / 1e9,
           "decode_hbm_frac": dec_bytes / (t_dec / 1e6) / 1e9 / PEAK_HBM_GBS,
           "decode_traffic_bytes": stored_attn_traffic(),
           "bf16_cache_hbm_floor_us": (2 * rows * (w.d * 2)) / (PEAK_HBM_GBS * 1e9) * 1e6,
           "append_prefill_us": t_app, "append_gbps": app_bytes / (t_app / 1e6) / 1e9,
           "timing": "events around back-to-back calls; cache and lengths resident in HBM"}
    del cache, kd, vd, qd, ws, out
    res["prefill"] = prefill_extra(torch, hbl, synthetic, timed)
    return res


def prefill_extra(torch, hbl, synthetic, timed):
    """Causal prefill of whole prompts over the 3-bit cache they were appended
    to: integer query-key scores on the int8 matrix instruction, bf16 value
    product.  Causal work: B*Hq*T(T+1)/2 query-key pairs, 4*d flops each, half
    of them int8 (peak 5.0 P) and half bf16 (peak 2.5 P), so the mixed peak
    for the whole is 1 / (0.5/5.0 + 0.5/2.5) = 3.33 PFLOP/s."""
    w = synthetic.ATTN_WORKLOADS["prefill_attn_7b_kv3"]
    q, k, v = synthetic.make_prefill(w)
    dev = lambda a: torch.from_numpy(a.view(np.int16)).cuda().view(torch.bfloat16)
    qd, kd, vd = dev(q), dev(k), dev(v)
    del q, k, v
    cache = hbl.KVCache(w.B, w.Hkv, w.T, w.d, w.kv_bits)
    start = torch.zeros(w.B, dtype=torch.int32, device="cuda")
    t_app = timed(lambda: cache.append(kd, vd, start), 10)
    out = torch.empty((w.B, w.T, w.Hq, w.d), dtype=torch.bfloat16, device="cuda")
    t_pf = timed(lambda: hbl.attention_prefill(qd, w.q_bits, cache.k_codes, cache.k_scale, cache.v_codes,
                                               cache.v_scale, w.kv_bits, start, out=out), 20)
    flops = w.B * w.Hq * (w.T * (w.T + 1) / 2) * w.d * 4
    mixed_peak = 1.0 / (0.5 / PEAK_INT8_TOPS + 0.5 / PEAK_BF16_TFLOPS)
    return {"workload": w.name, "B": w.B, "T": w.T, "Hq": w.Hq, "Hkv": w.Hkv, "d": w.d, "kv_bits": w.kv_bits,
            "q_bits": w.q_bits, "prefill_us": t_pf, "prefill_tflops": flops / (t_pf / 1e6) / 1e12,
            "mixed_mfma_peak_tflops": mixed_peak, "prefill_mfma_frac": flops / (t_pf / 1e6) / 1e12 / mixed_peak,
            "append_us": t_app, "flops_counted": "B*Hq*T(T+1)/2 pairs x 4d (scores and values, causal half)"}


def cpu_baseline(x, wl, bits, budget_s):
    """The oracle as it stands, on the host cores, on the first tokens of the
    same workload (sample sized to about `budget_s` seconds)."""
    import oracle
    wt, alpha = oracle.quantize_weights(wl)
    threads = oracle.max_threads()
    n0 = max(1, threads)
    t0 = time.perf_counter()
    oracle.forward(x[:n0], wt, alpha, bits, keep=False)
    dt = time.perf_counter() - t0
    n = int(min(x.shape[0], max(n0, n0 * budget_s / max(dt, 1e-6))))
    n = max(n0, (n // n0) * n0)
    t0 = time.perf_counter()
    oracle.forward(x[:n], wt, alpha, bits, keep=False)
    dt = time.perf_counter() - t0
    return {"value": n / dt, "unit": "tokens/s", "cores": threads, "kind": "oracle",
            "sample": f"first {n} of {x.shape[0]} tokens of the same workload (INT{bits}), {dt:.1f} s wall",
            "cpu": cpu_model(), "single_thread": single_thread_baselines(oracle)}


def single_thread_baselines(oracle):
    """The oracle on one thread for the smallest configuration (8 tokens,
    K = N = 256, INT8, fp32) and one-token decode (K = 16384, N = 4096,
    INT4), each repeated to about half a second."""
    import synthetic
    out = {}
    for name in ("tiny_int8", "decode_7b_m1"):
        w = synthetic.WORKLOADS[name]
        x, _, wl = synthetic.make_inputs(w)
        wt, alpha = oracle.quantize_weights(wl)
        reps, dt = 0, 0.0
        t0 = time.perf_counter()
        while dt < 0.5 or reps < 2:
            oracle.forward(x, wt, alpha, w.bits, keep=False, nthreads=1)
            reps += 1
            dt = time.perf_counter() - t0
        out[name] = {"tokens_per_s": reps * w.M / dt, "ms_per_call": 1e3 * dt / reps, "calls": reps,
                     "M": w.M, "K": w.K, "N": w.N, "bits": w.bits, "threads": 1}
    return out


def cpu_model() -> str:
    try:
        with open("/proc/cpuinfo") as f:
            for line in f:
                if line.startswith("model name"):
                    return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return "unknown"


if __name__ == "__main__":
    main()
