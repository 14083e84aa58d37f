#!/usr/bin/env python3
"""Benchmark of BATQuant's online W4A4 linear-layer hot path on one MI355X.

One step is one pass of the whole online path over one batch of synthetic input: the fused
transform + clip + MXFP4 quantiser (K1) on the bf16 activations, then the MXFP4 x MXFP4
scaled-MFMA GEMM (K2) against weights prepared offline.  Default workload: the largest
layer configuration, the S=16384-token prefill through a down_proj-shaped layer (N=12288
in-features, out=4096; Qwen3-8B shape), seeded synthetic data; the q_proj-shaped layer
(S=2048, N=4096, out=4096) is timed beside it as a secondary record.

Inputs are resident in HBM before timing starts.  Every step uses the next of R buffer sets
(activations, codes, scales, prepared weights, output), with R chosen so the sets together
exceed the 256 MB Infinity Cache several times over; the measured rates are therefore HBM
rates, not cache rates.  Kernel durations come from HIP events recorded on the stream the
kernels are launched on: the timed steps run quantiser and GEMM in turn, and each kernel is
then timed alone over the same number of back-to-back launches, captured into a HIP graph
and replayed, so that its event interval holds nothing but its own executions (and not the
host's cost of enqueueing them).  The step time is wall clock around the timed steps.

With --kv mxfp4|mxfp8 it measures the KV-cache side instead (slot-mapped cache writes of K
and V rows, the query and attention-output transforms, the dequantisation of cache rows) on
the K/V projection shapes kv_prefill (default) or kv_decode.

Prints one JSON line.  --gpus above 1 is refused: this path runs on one GPU.
"""
from __future__ import annotations

import argparse
import json
import math
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

METRIC = "fused BAT+clip+MXFP4 quantize GB/s; W4A4 MXFP4 GEMM TFLOPS (% of peak)"
METRIC_W4A8 = "fused BAT+clip+MXFP8 quantize GB/s; W4A8 (MXFP4 x MXFP8) GEMM TFLOPS (% of peak)"
HBM_PEAK_GBS = 8000.0            # MI355X HBM3E
FP4_PEAK_TFLOPS = 10100.0        # MI355X dense MXFP4 MFMA
BF16_PEAK_TFLOPS = 2500.0        # MI355X dense bf16 MFMA (the W4A8 product runs on it)


FORMS = {"gpk": 0, "kronecker": 1, "full": 2}


def k1_bytes(S, N, code_bytes=0.5, form="gpk"):
    """Algorithmic bytes of one quantiser launch: bf16 in (2 B/elem), codes out (0.5 B/elem
    for MXFP4, 1 B for MXFP8), scales out (1 B per 32 elem), plus the parameters (GPK: A and
    B_i; Kronecker: A_i and B_i; full: P_i; two ratios per block)."""
    k = N // 32
    params = {"gpk": 256 + 64 * k, "kronecker": 256 * k + 64 * k, "full": 4096 * k}[form]
    return S * N * 2 + int(S * N * code_bytes) + S * k + params + 8 * k


def k2_flops(S, N, out):
    return 2 * S * N * out


def k2_bytes(S, N, out, act_code_bytes=0.5, epilogue="f32"):
    """Compulsory bytes of one GEMM launch: both operands once (activation codes 0.5 or
    1 B/elem, weight codes 0.5 B/elem, one scale byte per 32), the output once (fp32 4 B or
    bf16 2 B per element) and, with a residual, the bf16 residual once."""
    out_b = {"f32": 4, "bf16": 2, "bf16_residual": 4}[epilogue]
    return (int(S * N * act_code_bytes) + S * (N // 32) + out * (N // 2 + N // 32)
            + out_b * S * out)


def measured_traffic(kernel: str, workload: str):
    """HBM bytes per launch of `kernel` on `workload` from the committed rocprofv3 FETCH_SIZE /
    WRITE_SIZE summary (calibrated on a plain copy), or None when there is no summary or the
    kernel's source has changed since the counters were taken."""
    import hashlib
    path = os.path.join(ROOT, "profiles", f"{kernel}_{workload}_hbm_traffic.txt")
    if not os.path.exists(path):
        return None
    fields = dict(l.split(": ", 1) for l in open(path).read().splitlines() if ": " in l)
    try:
        src = open(os.path.join(ROOT, fields["source_file"].strip()), "rb").read()
        if hashlib.sha256(src).hexdigest() != fields["source_sha256"].strip():
            return None
        return int(fields["traffic_bytes_per_launch"])
    except (KeyError, OSError, ValueError):
        return None


def host_cpu():
    """The host's CPU model and logical core count, and the cores this process may use."""
    model = "unknown"
    try:
        for line in open("/proc/cpuinfo"):
            if line.startswith("model name"):
                model = line.split(":", 1)[1].strip()
                break
    except OSError:
        pass
    usable = len(os.sched_getaffinity(0)) if hasattr(os, "sched_getaffinity") else os.cpu_count()
    return model, os.cpu_count() or 1, max(1, usable or 1)


def cpu_baseline(L, seconds, w4a8=False, runs=3):
    """The oracle as it stands (plain C, OpenMP over token rows) on every core this process
    may use, on a bounded sample of token rows of the same layer: quantise the sampled rows
    and compute every output of those rows.  The sample is sized by a short probe so that
    one run takes about `seconds`; the median of `runs` runs is reported."""
    import numpy as np
    from oracle import oracle

    model, nproc, threads = host_cpu()
    S, N, out = L.cfg.S, L.cfg.N, L.cfg.out
    r1, r2 = oracle.clip_ratio(L.alpha_min), oracle.clip_ratio(L.alpha_max)
    wq, we = oracle.prepare_weight(L.W, L.A, L.B, nthreads=threads)   # offline, untimed

    def run(rows):
        idx = np.linspace(0, S - 1, rows).astype(np.int64)
        t0 = time.perf_counter()
        quant = oracle.quantize_act_fp8 if w4a8 else oracle.quantize_act
        xq, xe = quant(L.x_bits[idx], L.A, L.B, r1, r2, nthreads=threads)
        t1 = time.perf_counter()
        (oracle.gemm_w4a8 if w4a8 else oracle.gemm)(xq, xe, wq, we, nthreads=threads)
        t2 = time.perf_counter()
        return t1 - t0, t2 - t1

    probe = min(S, threads)
    tq, tg = run(probe)
    rows = int(min(S, max(probe, probe * seconds / max(tq + tg, 1e-6))))
    times = sorted((run(rows) for _ in range(runs)), key=lambda t: t[0] + t[1])
    tq, tg = times[len(times) // 2]
    return {
        "value": round(k1_bytes(rows, N, 1.0 if w4a8 else 0.5) / tq / 1e9, 4),
        "unit": "GB/s",
        "gemm_value": round(k2_flops(rows, N, out) / tg / 1e12, 6),
        "gemm_unit": "TFLOP/s",
        "seconds": round(tq + tg, 2),
        "runs": runs,
        "cores": threads,
        "host_logical_cores": nproc,
        "cpu_model": model,
        "kind": "oracle",
        "sample": f"{rows} of {S} token rows (evenly spaced): quantise them and compute all "
                  f"{out} outputs of each; plain C oracle, OpenMP over rows on {threads} "
                  f"threads; median of {runs} runs",
    }


def time_launches(stream, fn, first, K, R):
    """K launches of fn on the rotated sets (fn(j) for set j = (first + i) % R), back to back
    on one stream; returns the event-measured GPU time per launch and the wall time per
    launch (seconds).  The events are recorded on the stream the kernels are launched on."""
    import torch
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    e0.record(stream)
    for i in range(K):
        if fn((first + i) % R):
            raise RuntimeError("library call failed")
    e1.record(stream)
    torch.cuda.synchronize()
    t1 = time.perf_counter()
    return e0.elapsed_time(e1) * 1e-3 / K, (t1 - t0) / K


def time_graph(stream, fn, first, K, R, reps=3):
    """K launches of fn (fn(j, stream_handle) for set j = (first + i) % R) captured into one
    HIP graph, replayed `reps` times on `stream`; returns the event-measured GPU time per
    launch (seconds).  Replay takes the host's launch cost out of the interval, so small
    kernels are timed by the GPU rather than by the Python loop that enqueues them."""
    import torch
    g = torch.cuda.CUDAGraph()
    cs = torch.cuda.Stream()
    torch.cuda.synchronize()
    with torch.cuda.graph(g, stream=cs):
        h = torch.cuda.current_stream().cuda_stream
        for i in range(K):
            if fn((first + i) % R, h):
                raise RuntimeError("library call failed")
    torch.cuda.synchronize()
    with torch.cuda.stream(stream):
        g.replay()                                   # untimed first replay
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record(stream)
        for _ in range(reps):
            g.replay()
        e1.record(stream)
    torch.cuda.synchronize()
    del g
    return e0.elapsed_time(e1) * 1e-3 / (K * reps)


def measure(name, args):
    """Time one layer configuration; returns (record, layer)."""
    import numpy as np
    import torch

    import w4a4_batq_quantize_amd as bq
    import workloads as wl

    L = wl.make_layer(name)
    S, N, out = L.cfg.S, L.cfg.N, L.cfg.out
    k = N // 32
    w4a8 = args.precision == "w4a8"
    form = getattr(args, "form", "gpk")
    epilogue = getattr(args, "epilogue", "f32")
    rms = getattr(args, "rmsnorm", False)
    if rms and (w4a8 or form != "gpk"):
        raise SystemExit("bench.py: --rmsnorm applies to the W4A4 GPK quantiser")
    if w4a8 and form != "gpk":
        raise SystemExit("bench.py: --form applies to the W4A4 path")
    cb = 1.0 if w4a8 else 0.5                 # activation code bytes per element
    peak = BF16_PEAK_TFLOPS if w4a8 else FP4_PEAK_TFLOPS
    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)

    A = torch.from_numpy(L.A).to(dev)
    B = torch.from_numpy(L.B).to(dev)
    rmin = torch.from_numpy(bq.clip_ratios(L.alpha_min)).to(dev)
    rmax = torch.from_numpy(bq.clip_ratios(L.alpha_max)).to(dev)
    W = torch.from_numpy(L.W).to(dev)
    layout = bq.SCALES_MFMA_TILED
    if form == "gpk":
        wq0, we0 = bq.prepare_weight(W, L.A, L.B, layout=layout)
    else:
        # seeded near-identity factors of the chosen form (thelatestinai listing, Table 1)
        F0h, F1h = wl.form_factors(FORMS[form], k, seed=(61, FORMS[form], N))
        wq0, we0 = bq.prepare_weight_form(W, FORMS[form], F0h, F1h, layout=layout)
        A = torch.from_numpy(F0h).to(dev)
        B = torch.from_numpy(F1h).to(dev) if F1h is not None else None
    del W
    x0 = torch.from_numpy(L.x_bits.view(np.int16)).to(dev).view(torch.bfloat16)

    per_set = S * N * 2 + S * (int(N * cb) + k) + out * (N // 2 + k) + 4 * S * out
    R = min(1024, max(2, math.ceil(args.rotate_bytes / per_set)))
    xs = [x0.clone() for _ in range(R)]
    wqs = [wq0.clone() for _ in range(R)]
    wes = [we0.clone() for _ in range(R)]
    xqs = [torch.empty((S, int(N * cb)), dtype=torch.uint8, device=dev) for _ in range(R)]
    xes = [torch.empty((bq.scale_bytes(S, N, layout),), dtype=torch.uint8, device=dev)
           for _ in range(R)]
    ydt = torch.float32 if epilogue == "f32" else torch.bfloat16
    ys = [torch.empty((S, out), dtype=ydt, device=dev) for _ in range(R)]
    resid = (torch.randn((S, out), device=dev).to(torch.bfloat16)
             if epilogue == "bf16_residual" else None)
    del x0, wq0, we0

    stream = torch.cuda.current_stream()
    sh = stream.cuda_stream
    pA, pr1, pr2 = A.data_ptr(), rmin.data_ptr(), rmax.data_ptr()
    pB = B.data_ptr() if B is not None else 0
    ptr = [(xs[j].data_ptr(), xqs[j].data_ptr(), xes[j].data_ptr(), wqs[j].data_ptr(),
            wes[j].data_ptr(), ys[j].data_ptr()) for j in range(R)]
    quant, gemm = ((bq.quantize_act_mxfp8_raw, bq.gemm_w4a8_raw) if w4a8 else
                   (bq.quantize_act_raw, bq.gemm_w4a4_raw))
    if rms:
        gamma = (1 + 0.1 * torch.randn(N, device=dev)).float().contiguous()
        pg = gamma.data_ptr()

        def quant(x, S_, N_, ldx, a, b, r1, r2, xq, xe, lay, st):
            return bq.quantize_act_rmsnorm_raw(x, S_, N_, ldx, pg, 1e-6, a, b, r1, r2, xq, xe,
                                               lay, st)
    if form != "gpk":
        fid = FORMS[form]

        def quant(x, S_, N_, ldx, a, b, r1, r2, xq, xe, lay, st):
            return bq.quantize_act_form_raw(x, S_, N_, ldx, fid, a, b, r1, r2, xq, xe, lay, st)

    def launch_k1(j, s=sh):
        x, xq, xe, _, _, _ = ptr[j]
        return quant(x, S, N, N, pA, pB, pr1, pr2, xq, xe, layout, s)

    if epilogue != "f32":
        gemm_out = bq.gemm_w4a8_out_raw if w4a8 else bq.gemm_w4a4_out_raw
        pres = resid.data_ptr() if resid is not None else 0

        def gemm(xq, xe, wq, we, S_, N_, out_, y, lay, st):
            return gemm_out(xq, xe, wq, we, S_, N_, out_, y, bq.OUT_BF16, pres, lay, st)

    def launch_k2(j, s=sh):
        _, xq, xe, wq, we, y = ptr[j]
        return gemm(xq, xe, wq, we, S, N, out, y, layout, s)

    def step(j):
        if launch_k1(j) | launch_k2(j):
            raise RuntimeError("library call failed")

    def timed(fn, first, K):
        return time_launches(stream, fn, first, K, R)

    # every set's activation codes and scales are written once before anything is timed, so
    # the GEMM-alone launches below never read buffers the quantiser has not filled
    for j in range(R):
        if launch_k1(j):
            raise RuntimeError("library call failed")
    for i in range(args.warmup):
        step(i % R)
    torch.cuda.synchronize()

    # the timed steps: quantise + GEMM per step
    K = args.steps
    t_step_ev, t_step_wall = timed(lambda j: step(j) or 0, args.warmup, K)
    ms_per_step = t_step_wall * 1e3
    # per-kernel durations: the same launches, each kernel alone back to back in a captured
    # graph, so that an event interval holds one kernel's executions and the dispatch gaps
    # between them only
    t_k1 = time_graph(stream, launch_k1, args.warmup + K, K, R)
    t_k2 = time_graph(stream, launch_k2, args.warmup + 2 * K, K, R)
    # at most four tokens the layer also runs as one kernel (batq_linear_w4a4): timed the
    # same way, for the record beside the two kernels (same outputs)
    t_lin = None
    if (form == "gpk" and not rms and epilogue == "f32" and S <= bq.LINEAR_FUSED_TOKENS
            and k % 8 == 0 and k <= 512 and (not w4a8 or S * k <= bq.LINEAR_W4A8_FUSED_BLOCKS)):
        lin = bq.linear_w4a8_raw if w4a8 else bq.linear_w4a4_raw

        def launch_lin(j, s=sh):
            x, _, _, wq, we, y = ptr[j]
            return lin(x, S, N, N, pA, pB, pr1, pr2, wq, we, out, y, 0, 0, layout, s)
        t_lin = time_graph(stream, launch_lin, args.warmup + 3 * K, K, R)

    if args.copy_calibration:
        # plain copy of known size, outside the timed region, for scaling HBM counters
        a = torch.empty(256 << 20, dtype=torch.uint8, device=dev)
        b = torch.empty_like(a)
        for _ in range(3):
            b.copy_(a)
        torch.cuda.synchronize()

    # keep the last step's output alive and finite (a cheap sanity check, untimed)
    last = ys[(args.warmup + 3 * K - 1) % R]
    assert bool(torch.isfinite(last).all().item()), "non-finite GEMM output"

    b1 = k1_bytes(S, N, cb, form) + (4 * N if rms else 0)
    b2 = k2_bytes(S, N, out, cb, epilogue)
    gbs = b1 / t_k1 / 1e9
    tflops = k2_flops(S, N, out) / t_k2 / 1e12
    k2_ai = k2_flops(S, N, out) / b2
    k2_roof = min(peak, k2_ai * HBM_PEAK_GBS / 1e3)
    k1_name = "quantize_kernel_mxfp8" if w4a8 else "quantize_kernel"
    big = (not w4a8 and epilogue == "f32" and k % 32 == 0
           and ((S + 255) // 256) * ((out + 255) // 256) >= 512)
    k2_name = ("gemm_skinny_kernel" if S <= 64 else
               "gemm_w4a8_kernel" if w4a8 else
               "gemm_big_kernel" if big else "gemm_pc_kernel")
    tr1 = measured_traffic(k1_name, L.cfg.name) if form == "gpk" and not rms else None
    tr2 = measured_traffic(k2_name, L.cfg.name) if epilogue == "f32" else None
    roof_k1 = {"kernel": f"{k1_name} (fused BAT+clip+{'MXFP8' if w4a8 else 'MXFP4'}"
                         + ("" if form == "gpk" else f", {form} transform")
                         + (", RMSNorm prologue" if rms else "") + ")",
               "bound": "hbm",
               "achieved": round(gbs, 1), "peak": HBM_PEAK_GBS, "unit": "GB/s",
               "frac": round(gbs / HBM_PEAK_GBS, 4), "traffic": tr1,
               "avg_us": round(t_k1 * 1e6, 3), "algorithmic_bytes": b1}
    hbm_bound = k2_roof < peak
    k2_gbs = b2 / t_k2 / 1e9
    roof_k2 = {"kernel": k2_name + (" (E2M1 x E4M3 dequantised to bf16, bf16 MFMA)" if w4a8
                                    else " (MXFP4 scaled MFMA)"),
               "bound": "hbm" if hbm_bound else "mfma",
               "achieved": round(k2_gbs if hbm_bound else tflops, 1),
               "peak": HBM_PEAK_GBS if hbm_bound else peak,
               "unit": "GB/s" if hbm_bound else "TFLOP/s",
               "frac": round(k2_gbs / HBM_PEAK_GBS if hbm_bound else tflops / peak, 4),
               "traffic": tr2, "tflops": round(tflops, 1),
               "algorithmic_bytes": b2,
               "avg_us": round(t_k2 * 1e6, 3), "algorithmic_flops": k2_flops(S, N, out),
               "roofline_tflops": round(k2_roof, 1), "frac_of_roofline": round(tflops / k2_roof, 4)}
    dominant = roof_k2 if t_k2 >= t_k1 else roof_k1

    rec = {
        "metric": METRIC_W4A8 if w4a8 else METRIC,
        "value": round(gbs, 1),
        "unit": "GB/s",
        "n_gpus": 1,
        "steps": K,
        "warmup": args.warmup,
        "ms_per_step": round(ms_per_step, 5),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "mxfp8/mxfp4" if w4a8 else "mxfp4",
        "dtype_detail": ("K1: bf16 in, fp32 transform/clip, E4M3+E8M0 out; K2: E2M1 weights and "
                         "E4M3 activations dequantised exactly to bf16, bf16 MFMA, fp32 "
                         "accumulate and output" if w4a8 else
                         "K1: bf16 in, fp32 transform/clip, E2M1+E8M0 out; "
                         "K2: E2M1 x E2M1 scaled MFMA, fp32 accumulate and output"),
        "data": "synthetic",
        "config": {"workload": f"{L.cfg.name}: S={S} N={N} out={out} (Qwen3-8B-shaped linear "
                               f"layer, seeded synthetic bf16 activations and fp32 weights)",
                   "S": S, "N": N, "out": out, "rotated_buffer_sets": R,
                   "scale_layout": "mfma_tiled", "transform": form,
                   "gemm_output": epilogue, "rmsnorm_prologue": rms},
        "gemm": {"value": round(tflops, 1), "unit": "TFLOP/s",
                 "pct_of_peak": round(100 * tflops / peak, 2)},
        "step_gpu_us": round(t_step_ev * 1e6, 3),
        "kernel_us": {"quantize": round(t_k1 * 1e6, 3), "gemm": round(t_k2 * 1e6, 3)},
        "roofline": dominant,
        "roofline_kernels": {"quantize": roof_k1, "gemm": roof_k2},
    }
    if t_lin is not None:
        # compulsory bytes of the one-kernel layer: bf16 rows in, weights and their scales,
        # fp32 outputs (the factors and ratios are a few KB)
        b_lin = S * N * 2 + out * (N // 2 + k) + 4 * S * out
        rec["linear_one_kernel"] = {
            "kernel": "gemm_linear16_kernel (transform + clip + "
                      + ("MXFP8" if w4a8 else "MXFP4") + " of the token rows inside the "
                      "few-token GEMM)",
            "avg_us": round(t_lin * 1e6, 3), "two_kernels_us": round((t_k1 + t_k2) * 1e6, 3),
            "bound": "hbm", "achieved": round(b_lin / t_lin / 1e9, 1), "peak": HBM_PEAK_GBS,
            "unit": "GB/s", "frac": round(b_lin / t_lin / 1e9 / HBM_PEAK_GBS, 4),
            "algorithmic_bytes": b_lin}
    return rec, L


def measure_data_dependence(name, args):
    """Each kernel of the W4A4 path alone on one layer shape with three operand contents.
    GEMM: the layer's own codes (quantised activations, prepared weights), uniformly random
    code bytes, and all-zero codes, every one with the layer's scale bytes.  Quantiser: the
    layer's bf16 activations, N(0,1) activations, and all-zero activations.  Same kernels,
    same launches, same bytes moved; only the values differ.  Returns one record with the
    graph-timed durations."""
    import numpy as np
    import torch

    import w4a4_batq_quantize_amd as bq
    import workloads as wl

    L = wl.make_layer(name)
    S, N, out = L.cfg.S, L.cfg.N, L.cfg.out
    k = N // 32
    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    layout = bq.SCALES_MFMA_TILED
    A = torch.from_numpy(L.A).to(dev)
    B = torch.from_numpy(L.B).to(dev)
    rmin = torch.from_numpy(bq.clip_ratios(L.alpha_min)).to(dev)
    rmax = torch.from_numpy(bq.clip_ratios(L.alpha_max)).to(dev)
    wq0, we0 = bq.prepare_weight(torch.from_numpy(L.W).to(dev), L.A, L.B, layout=layout)
    x0 = torch.from_numpy(L.x_bits.view(np.int16)).to(dev).view(torch.bfloat16)
    xq0, xe0 = bq.quantize_act(x0, A, B, rmin, rmax, layout=layout)
    torch.cuda.synchronize()
    per_set = S * (N // 2 + k) + out * (N // 2 + k) + 4 * S * out
    R = min(64, max(2, math.ceil(args.rotate_bytes / per_set)))
    g = torch.Generator(device=dev)
    g.manual_seed(7)

    def codes(kind, like):
        if kind == "layer":
            return like.clone()
        if kind == "zero":
            return torch.zeros_like(like)
        return torch.randint(0, 256, like.shape, dtype=torch.int32, device=dev,
                             generator=g).to(torch.uint8)

    stream = torch.cuda.current_stream()
    times = {}
    for kind in ("layer", "random", "zero"):
        sets = [(codes(kind, xq0), xe0.clone(), codes(kind, wq0), we0.clone(),
                 torch.empty((S, out), dtype=torch.float32, device=dev)) for _ in range(R)]

        def launch(j, st, sets=sets):
            xq, xe, wq, we, y = sets[j]
            return bq.gemm_w4a4_raw(xq.data_ptr(), xe.data_ptr(), wq.data_ptr(), we.data_ptr(),
                                    S, N, out, y.data_ptr(), layout, st)
        for j in range(R):                      # warm-up, untimed
            if launch(j, stream.cuda_stream):
                raise RuntimeError("library call failed")
        torch.cuda.synchronize()
        times[kind] = time_graph(stream, launch, 0, args.steps, R)
        del sets
        torch.cuda.empty_cache()
    # the quantiser on the layer's activations, N(0,1) activations and zeros
    R1 = min(64, max(2, math.ceil(args.rotate_bytes / (S * N * 2 + S * (N // 2 + k)))))
    qtimes = {}
    for kind in ("layer", "random", "zero"):
        if kind == "layer":
            xs = [x0.clone() for _ in range(R1)]
        elif kind == "random":
            xs = [torch.randn((S, N), device=dev, generator=g).to(torch.bfloat16)
                  for _ in range(R1)]
        else:
            xs = [torch.zeros((S, N), dtype=torch.bfloat16, device=dev) for _ in range(R1)]
        qs = [(torch.empty_like(xq0), torch.empty_like(xe0)) for _ in range(R1)]

        def launch_q(j, st, xs=xs, qs=qs):
            return bq.quantize_act_raw(xs[j].data_ptr(), S, N, N, A.data_ptr(), B.data_ptr(),
                                       rmin.data_ptr(), rmax.data_ptr(), qs[j][0].data_ptr(),
                                       qs[j][1].data_ptr(), layout, st)
        for j in range(R1):
            if launch_q(j, stream.cuda_stream):
                raise RuntimeError("library call failed")
        torch.cuda.synchronize()
        qtimes[kind] = time_graph(stream, launch_q, 0, args.steps, R1)
        del xs, qs
        torch.cuda.empty_cache()
    flops = k2_flops(S, N, out)
    return {
        "metric": "W4A4 path kernel times by operand contents (same kernels, shapes and bytes)",
        "unit": "us",
        "config": {"workload": f"{name}: S={S} N={N} out={out}", "S": S, "N": N, "out": out,
                   "rotated_buffer_sets": R, "scale_layout": "mfma_tiled",
                   "operands": {"layer": "the layer's quantised activations and prepared "
                                         "weights",
                                "random": "uniformly random code bytes, the layer's scales",
                                "zero": "all-zero code bytes, the layer's scales"}},
        "steps": args.steps,
        "gemm_us": {kd: round(t * 1e6, 3) for kd, t in times.items()},
        "gemm_tflops": {kd: round(flops / t / 1e12, 1) for kd, t in times.items()},
        "peak_tflops": FP4_PEAK_TFLOPS,
        "quantize_us": {kd: round(t * 1e6, 3) for kd, t in qtimes.items()},
        "quantize_gbs": {kd: round(k1_bytes(S, N) / t / 1e9, 1) for kd, t in qtimes.items()},
        "quantize_operands": {"layer": "the layer's bf16 activations",
                              "random": "N(0,1) bf16 activations", "zero": "all-zero activations"},
    }


# KV-cache side of attention with a transformed, quantised cache (W4A8KV8 / W4A8KV4), on the
# evaluated 8B model's attention shape: 8 kv heads x head dim 128, 32 query heads (GQA 4).
KV_HEADS, HEAD_DIM, GQA_GROUP = 8, 128, 4
METRIC_KV = "KV-cache write: fused BAT+clip+{fmt} into slot-mapped cache rows GB/s"


def kv_write_bytes(T, N, code_bytes):
    """Algorithmic bytes of one cache write: bf16 rows in, codes and scales out, the slot map
    (8 B per token), GPK factors and two ratios per block."""
    k = N // 32
    return T * N * 2 + int(T * N * code_bytes) + T * k + 8 * T + 256 + 64 * k + 8 * k


def transform_bytes(rows, N, in_b=2, out_b=2):
    return rows * N * (in_b + out_b) + 256 + 64 * (N // 32)


def dequant_bytes(rows, N, code_bytes, out_b=2):
    return rows * (int(N * code_bytes) + N // 32 + 8) + rows * N * out_b


def cpu_baseline_kv(L, fmt, seconds):
    """The oracle's slot-mapped cache write (single-threaded C) over the whole workload,
    repeated for about `seconds`."""
    import numpy as np
    from oracle import oracle
    import workloads as wl
    T, N = L.x_bits.shape
    r1, r2 = oracle.clip_ratio(L.alpha_min), oracle.clip_ratio(L.alpha_max)
    slots = wl.kv_slots(T, 2 * T, seed=(67,))
    cq = np.zeros((2 * T, N // 2 if fmt == 4 else N), dtype=np.uint8)
    ce = np.zeros((2 * T, N // 32), dtype=np.uint8)
    n, t0 = 0, time.perf_counter()
    while True:
        oracle.quantize_kv(L.x_bits, slots, fmt, L.A, L.B, r1, r2, cq, ce)
        n += 1
        if time.perf_counter() - t0 >= seconds:
            break
    dt = time.perf_counter() - t0
    return {"value": round(n * kv_write_bytes(T, N, 0.5 if fmt == 4 else 1.0) / dt / 1e9, 4),
            "unit": "GB/s", "seconds": round(dt, 2), "cores": 1, "kind": "oracle",
            "sample": f"{n} full passes over the {T} token rows (plain C oracle, one thread)"}


def measure_kv(name, args):
    """Time the KV path on one configuration: cache writes of K and V rows, the query
    transform (P^-T per kv head) and the attention-output transform (P^-1), and the
    dequantisation of the written cache rows."""
    import numpy as np
    import torch

    import w4a4_batq_quantize_amd as bq
    import workloads as wl

    fmt = bq.KV_MXFP4 if args.kv == "mxfp4" else bq.KV_MXFP8
    cb = 0.5 if fmt == bq.KV_MXFP4 else 1.0
    L = wl.make_layer(name, with_weight=False)
    T, N = L.x_bits.shape
    assert N == KV_HEADS * HEAD_DIM
    k = N // 32
    Nq = N * GQA_GROUP
    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    f32 = lambda a: torch.from_numpy(np.ascontiguousarray(a, dtype=np.float32)).to(dev)

    # factors: K rows use the layer's (A, B), V rows their own; queries take P_K^-T of the kv
    # head they attend to, attention outputs P_V^-1
    Av, Bv = wl.form_factors(0, k, seed=(68, N))
    Aki, Bki = bq.weight_factors(L.A, L.B)
    Avi, Bvi = bq.weight_factors(Av, Bv)
    kd = HEAD_DIM // 32
    per_q = lambda Bx: np.concatenate([Bx[(h // GQA_GROUP) * kd:(h // GQA_GROUP + 1) * kd]
                                       for h in range(KV_HEADS * GQA_GROUP)])
    Aq, Bq = Aki, per_q(Bki)
    Ao, Bo = Avi.T, per_q(np.transpose(Bvi, (0, 2, 1)))
    dA, dB, dAv, dBv = f32(L.A), f32(L.B), f32(Av), f32(Bv)
    dAq, dBq, dAo, dBo = f32(Aq), f32(Bq), f32(Ao), f32(Bo)
    rmin = f32(bq.clip_ratios(L.alpha_min))
    rmax = f32(bq.clip_ratios(L.alpha_max))

    per_set = (2 * T * N * 2 + 4 * T * Nq * 2 + 2 * T * (int(N * cb) + k) + 8 * T
               + T * N * 2)
    R = min(1024, max(2, math.ceil(args.rotate_bytes / per_set)))
    num_slots = R * T
    perm = torch.from_numpy(wl.kv_slots(num_slots, num_slots, seed=(69, T))).to(dev)
    slots = [perm[j * T:(j + 1) * T].contiguous() for j in range(R)]
    xk0 = torch.from_numpy(L.x_bits.view(np.int16)).to(dev).view(torch.bfloat16)
    xks = [xk0.clone() for _ in range(R)]
    xvs = [xk0.flip(0).contiguous() for _ in range(R)]
    qs = [torch.randn((T, Nq), device=dev).to(torch.bfloat16) for _ in range(R)]
    os_ = [torch.randn((T, Nq), device=dev).to(torch.bfloat16) for _ in range(R)]
    qts = [torch.empty((T, Nq), dtype=torch.bfloat16, device=dev) for _ in range(R)]
    ots = [torch.empty((T, Nq), dtype=torch.bfloat16, device=dev) for _ in range(R)]
    cols = int(N * cb)
    kq = torch.zeros((num_slots, cols), dtype=torch.uint8, device=dev)
    ke = torch.zeros((num_slots, k), dtype=torch.uint8, device=dev)
    vq = torch.zeros_like(kq)
    ve = torch.zeros_like(ke)
    deq = [torch.empty((T, N), dtype=torch.bfloat16, device=dev) for _ in range(R)]
    del xk0

    stream = torch.cuda.current_stream()
    sh = stream.cuda_stream
    BF = bq.OUT_BF16

    def write_k(j, s=sh):
        return bq.quantize_kv_raw(xks[j].data_ptr(), T, N, N, slots[j].data_ptr(), num_slots,
                                  fmt, dA.data_ptr(), dB.data_ptr(), rmin.data_ptr(),
                                  rmax.data_ptr(), kq.data_ptr(), ke.data_ptr(), s)

    def write_v(j, s=sh):
        return bq.quantize_kv_raw(xvs[j].data_ptr(), T, N, N, slots[j].data_ptr(), num_slots,
                                  fmt, dAv.data_ptr(), dBv.data_ptr(), rmin.data_ptr(),
                                  rmax.data_ptr(), vq.data_ptr(), ve.data_ptr(), s)

    def tq(j, s=sh):
        return bq.transform_rows_raw(qs[j].data_ptr(), BF, T, Nq, Nq, dAq.data_ptr(),
                                     dBq.data_ptr(), qts[j].data_ptr(), BF, s)

    def to(j, s=sh):
        return bq.transform_rows_raw(os_[j].data_ptr(), BF, T, Nq, Nq, dAo.data_ptr(),
                                     dBo.data_ptr(), ots[j].data_ptr(), BF, s)

    def dq(j, s=sh):
        return bq.dequantize_rows_raw(kq.data_ptr(), ke.data_ptr(), num_slots, N, fmt,
                                      slots[j].data_ptr(), T, deq[j].data_ptr(), BF, s)

    def step(j):
        return write_k(j) | write_v(j) | tq(j) | to(j)

    for j in range(R):
        if write_k(j) | write_v(j):
            raise RuntimeError("library call failed")
    for i in range(args.warmup):
        if step(i % R):
            raise RuntimeError("library call failed")
    torch.cuda.synchronize()
    K = args.steps
    t_step_ev, t_step_wall = time_launches(stream, step, args.warmup, K, R)
    t_kv = time_graph(stream, write_k, args.warmup + K, K, R)
    t_tr = time_graph(stream, tq, args.warmup + 2 * K, K, R)
    t_dq = time_graph(stream, dq, args.warmup + 3 * K, K, R)
    assert bool(torch.isfinite(deq[0].float()).all().item()), "non-finite dequantised rows"

    def roof(kernel, b, t):
        a = b / t / 1e9
        return {"kernel": kernel, "bound": "hbm", "achieved": round(a, 1),
                "peak": HBM_PEAK_GBS, "unit": "GB/s", "frac": round(a / HBM_PEAK_GBS, 4),
                "traffic": None, "avg_us": round(t * 1e6, 3), "algorithmic_bytes": b}

    b_kv = kv_write_bytes(T, N, cb)
    fname = "MXFP4" if fmt == bq.KV_MXFP4 else "MXFP8"
    r_kv = roof(f"quantize_kv_kernel (slot-mapped BAT+clip+{fname} cache write)", b_kv, t_kv)
    r_tr = roof("transform_rows_kernel (query transform, bf16 in and out)",
                transform_bytes(T, Nq), t_tr)
    r_dq = roof(f"dequantize_rows_kernel ({fname} cache rows by slot -> bf16)",
                dequant_bytes(T, N, cb), t_dq)
    dominant = max((r_kv, r_tr), key=lambda r: r["avg_us"])
    return {
        "metric": METRIC_KV.format(fmt=fname),
        "value": r_kv["achieved"],
        "unit": "GB/s",
        "n_gpus": 1, "steps": K, "warmup": args.warmup,
        "ms_per_step": round(t_step_wall * 1e3, 5),
        "higher_is_better": True, "scaling": "weak", "vs_baseline": None,
        "dtype": fname.lower(),
        "dtype_detail": f"bf16 K/V rows in, fp32 transform/clip, {fname} codes + E8M0 "
                        "scales out; transforms bf16 in/out with fp32 arithmetic",
        "data": "synthetic",
        "config": {"workload": f"{name}: T={T} tokens, K/V rows N={N} ({KV_HEADS} kv heads x "
                               f"{HEAD_DIM}), {KV_HEADS * GQA_GROUP} query heads, scattered "
                               f"cache slots, seeded synthetic bf16 data",
                   "T": T, "N": N, "query_N": Nq, "num_slots": num_slots,
                   "rotated_buffer_sets": R, "kv_format": fname},
        "step": "cache write of K and V rows + query transform + attention-output transform",
        "step_gpu_us": round(t_step_ev * 1e6, 3),
        "kernel_us": {"quantize_kv": r_kv["avg_us"], "transform_rows": r_tr["avg_us"],
                      "dequantize_rows": r_dq["avg_us"]},
        "roofline": dominant,
        "roofline_kernels": {"quantize_kv": r_kv, "transform_rows": r_tr,
                             "dequantize_rows": r_dq},
    }, L, fmt


def main():
    ap = argparse.ArgumentParser(description=__doc__.split("\n")[0])
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=200)
    ap.add_argument("--warmup", type=int, default=20)
    ap.add_argument("--config", default="sweep_s16384_n12288",
                    help="layer configuration (default: the S=16384 prefill, N=12288 -> 4096)")
    ap.add_argument("--also", default="q_proj",
                    help="a second configuration timed after the first and reported under "
                         "'secondary' (kernel times and rooflines only); 'none' to skip")
    ap.add_argument("--rotate-bytes", type=float, default=2.0e9,
                    help="total bytes of the rotated buffer sets")
    ap.add_argument("--cpu-seconds", type=float, default=6.0,
                    help="target length of one CPU-baseline run (three runs are made)")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--copy-calibration", action="store_true",
                    help="also run a plain device copy of known size (for counter scaling)")
    ap.add_argument("--precision", choices=("w4a4", "w4a8"), default="w4a4",
                    help="w4a8: MXFP8 activations against the MXFP4 weights")
    ap.add_argument("--form", choices=tuple(FORMS), default="gpk",
                    help="transform form of the quantiser (thelatestinai listing, Table 1): "
                         "gpk (the method), kronecker (private A_i), full (32x32 P_i)")
    ap.add_argument("--epilogue", choices=("f32", "bf16", "bf16_residual"), default="f32",
                    help="GEMM output: fp32 (the defined output), bf16, or bf16 plus a bf16 "
                         "residual")
    ap.add_argument("--rmsnorm", action="store_true",
                    help="quantise through the RMSNorm-fused quantiser (gamma [N], eps 1e-6)")
    ap.add_argument("--kv", choices=("mxfp4", "mxfp8"), default=None,
                    help="measure the KV-cache path instead (cache format; --config kv_prefill "
                         "or kv_decode)")
    ap.add_argument("--all", action="store_true",
                    help="measure every layer configuration, one JSON line each (no CPU baseline)")
    ap.add_argument("--data-dependence", action="store_true",
                    help="time the quantiser and the W4A4 GEMM alone on the layer's operands, "
                         "random operands and all-zero operands (the dependence of their speed "
                         "on the values)")
    args = ap.parse_args()
    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) != 1:
        print("bench.py: the path runs on one GPU; --gpus must be 1",
              file=sys.stderr)
        sys.exit(2)

    if args.kv:
        import workloads as wl
        name = args.config if args.config in wl.KV_CONFIGS else "kv_prefill"
        rec, L, fmt = measure_kv(name, args)
        if not args.no_cpu_baseline:
            rec["cpu_baseline"] = cpu_baseline_kv(L, fmt, args.cpu_seconds)
        print(json.dumps(rec), flush=True)
        return
    if args.data_dependence:
        print(json.dumps(measure_data_dependence(args.config, args)), flush=True)
        return
    if args.all:
        import workloads as wl
        for name in wl.CONFIGS:
            rec, _ = measure(name, args)
            print(json.dumps(rec), flush=True)
        return
    rec, L = measure(args.config, args)
    if args.also and args.also != "none" and args.also != args.config:
        rec2, _ = measure(args.also, args)
        rec["secondary"] = {k: rec2[k] for k in ("config", "kernel_us", "step_gpu_us",
                                                 "gemm", "roofline_kernels")}
        rec["secondary"]["value"] = rec2["value"]
        rec["secondary"]["unit"] = rec2["unit"]
    if not args.no_cpu_baseline:
        if args.form == "gpk" and not args.rmsnorm:
            rec["cpu_baseline"] = cpu_baseline(L, args.cpu_seconds, args.precision == "w4a8")
    print(json.dumps(rec), flush=True)


if __name__ == "__main__":
    main()
