#!/usr/bin/env python3
"""Benchmark of the fused W4A16 dequantize-GEMM on one MI355X.

One step = one w4a16_gemm call (the whole hot path: weight stream, unpack,
group dequant, MFMA, reduction, epilogue) on a seeded synthetic workload.
Inputs are resident in HBM before the timed region.  Every weight set fits
in the 256 MB Infinity Cache, so the benchmark rotates over enough
independent copies of the packed weights (>= 1 GiB in total) that each call
reads its weights from HBM, as a decode step does when the other layers'
weights have passed through the cache in between.

Prints one JSON line (rank 0): metric, value, roofline, cpu_baseline, ...
"""
import argparse
import json
import math
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

import numpy as np  # noqa: E402

import w4a16_synth as synth  # noqa: E402

HBM_PEAK_GBS = 8000.0        # MI355X HBM3E, 8 TB/s
MFMA_PEAK_TFLOPS = 2500.0    # MI355X dense fp16/bf16 MFMA, 2.5 PFLOP/s
INT8_PEAK_TOPS = 5000.0      # MI355X dense int8 MFMA, 5.0 POP/s
FP8_PEAK_TFLOPS = 5000.0     # MI355X dense fp8 MFMA, 5.0 PFLOP/s (the MXFP4 route's A operand is fp8)
DEFAULT_WORKLOAD = "decode_m1_k8192_n28672_fp16_asym_g128_outliers"
METRIC = "W4A16 GEMM achieved HBM GB/s"


_SLEEP_CYCLES_PER_MS = None


def hold_gpu(ms):
    """Enqueue a GPU spin of about `ms` milliseconds on the current stream.
    Launches queued behind it then run back to back, so per-launch events
    time the kernels and not the host's launch overhead."""
    import torch

    global _SLEEP_CYCLES_PER_MS
    if _SLEEP_CYCLES_PER_MS is None:
        a = torch.cuda.Event(enable_timing=True)
        b = torch.cuda.Event(enable_timing=True)
        torch.cuda.synchronize()
        a.record()
        torch.cuda._sleep(2_000_000)
        b.record()
        torch.cuda.synchronize()
        _SLEEP_CYCLES_PER_MS = 2_000_000 / max(a.elapsed_time(b), 1e-3)
    torch.cuda._sleep(int(ms * _SLEEP_CYCLES_PER_MS))


def algorithmic_bytes(cfg):
    M, K, N, G = cfg["M"], cfg["K"], cfg["N"], cfg["G"]
    b = K * N // 2 + (K // G) * N * 2 + M * K * 2 + M * N * 2
    if not cfg["sym"]:
        b += (K // G) * N // 2
    return b


def algorithmic_flops(cfg):
    return 2 * cfg["M"] * cfg["N"] * cfg["K"]


def bound_of(cfg):
    # ridge of the MI355X roofline: 2.5e15 / 8e12 = 312.5 flop/byte
    return "mfma" if algorithmic_flops(cfg) / algorithmic_bytes(cfg) > 312.5 else "hbm"


def cpu_baseline(name, cfg, budget_s=12.0):
    """The oracle as it stands, on this host's cores, on a slice of output
    columns of the same workload; the rate is extrapolated to the whole N."""
    import oracle

    oracle.build()
    # this process's CPU share (at most 16 threads, one GPU's share of its host)
    try:
        threads = len(os.sched_getaffinity(0))
    except (AttributeError, OSError):
        threads = os.cpu_count() or 1
    threads = max(1, min(threads, 16))
    cpu_model = "unknown CPU"
    try:
        with open("/proc/cpuinfo") as fh:
            for line in fh:
                if line.startswith("model name"):
                    cpu_model = line.split(":", 1)[1].strip()
                    break
    except OSError:
        pass
    p = synth.make_problem(seed=0, **cfg)
    M, K, N, G = cfg["M"], cfg["K"], cfg["N"], cfg["G"]
    rows = min(M, 64)

    def run(ncol):
        qw = np.ascontiguousarray(p.qweight[:, :ncol])
        sc = np.ascontiguousarray(p.scales[:, :ncol])
        zr = None if p.zeros is None else np.ascontiguousarray(p.zeros[:, :ncol])
        t0 = time.perf_counter()
        oracle.gemm(p.X[:rows], qw, sc, zr, rows, ncol, K, G, cfg["dtype"], cfg["sym"],
                    nthreads=threads)
        return time.perf_counter() - t0

    probe = min(N, max(threads, 64))
    t_probe = run(probe)
    ncol = int(min(N, max(probe, probe * budget_s / max(t_probe, 1e-6))))
    # repeat the sample until about budget_s of CPU time has been spent
    times = [run(ncol)]
    while sum(times) < budget_s and len(times) < 64:
        times.append(run(ncol))
    t = float(np.mean(times))
    t_full = t * (N / ncol) * (M / rows)
    return {
        "value": round(algorithmic_bytes(cfg) / t_full / 1e9, 4),
        "unit": "GB/s",
        "cores": threads,
        "kind": "oracle",
        "sample": f"{rows} of {M} rows x {ncol} of {N} columns (K={K}) of the same workload, "
                  f"{len(times)} runs, {t:.2f} s each on {threads} threads of {cpu_model} (the C oracle: "
                  f"per-element dequant with its own RNE, fp64 dot products); rate "
                  f"extrapolated linearly to the full {M}x{N} output ({t_full:.2f} s)",
    }


KERNEL_SOURCES = ("w4a16_gemm.hip", "w4a16_decode.hip", "w4a16_wide.hip", "w4a16_device.h",
                  "w4a16_epilogue.h",
                  "w4a16_layout.h", "w4a16_internal.h", "w4a16_api.cpp")
KERNEL_SOURCES_W4A8 = ("w4a8_gemm.hip", "w4a8_device.h", "w4a8_internal.h", "w4a8_api.cpp")
KERNEL_SOURCES_MXFP4 = ("mx_gemm.hip", "mx_internal.h", "mx_api.cpp")
# Reported beside the headline workload (same protocol, no CPU baseline or
# comparators): the prefill and the batched shapes of the same layer.
EXTRA_WORKLOADS = ("prefill_m4096_k8192_n28672_bf16_asym_g128",
                   "batch_m64_k8192_n28672_fp16_asym_g64")


def kernel_source_hash(sources=KERNEL_SOURCES):
    import hashlib

    h = hashlib.sha256()
    for f in sources:
        with open(os.path.join(ROOT, "w4a16_dequant_gemm_amd", "csrc", f), "rb") as fh:
            h.update(fh.read())
    return h.hexdigest()[:16]


def measured_traffic(name, sources=KERNEL_SOURCES):
    """HBM bytes per launch from the committed rocprofv3 FETCH_SIZE/WRITE_SIZE
    record of this workload, or None if there is none or the kernel sources
    changed since it was taken."""
    path = os.path.join(ROOT, "profiles", "traffic.json")
    if not os.path.exists(path):
        return None
    with open(path) as fh:
        rec = json.load(fh).get(name)
    if not rec or rec.get("source_hash") != kernel_source_hash(sources):
        return None
    return int(rec["traffic_bytes"])


def run_workload(name, steps, warmup, rotate_bytes=1 << 30, with_cpu=True, comparators=True,
                 plan=None, rows=None):
    import torch

    import w4a16_dequant_gemm_amd as w4

    w4.load_library()
    cfg = dict(synth.WORKLOADS[name])
    if rows is not None:          # the workload's weights with another number of rows
        cfg["M"] = rows
    dev = torch.device("cuda:0")
    p = synth.make_problem(seed=0, **cfg)
    flags = w4.flags_of(p.dtype, p.sym)
    X, qw, sc, zr = w4.to_device(p, dev)
    base = w4.w4a16_repack(qw, sc, zr, p.K, p.N, p.G, flags)
    del qw, sc, zr
    copies = max(2, min(16, math.ceil(rotate_bytes / base.data.numel())))
    blobs = [base] + [w4.PackedW4(base.data.clone(), base.K, base.N, base.group_size, base.flags,
                                  base.layout_version) for _ in range(copies - 1)]
    Y = torch.empty((p.M, p.N), dtype=X.dtype, device=dev)
    ws_bytes = w4.w4a16_workspace_bytes(p.M, p.N, p.K, p.G, flags | w4.plan_flags(plan))
    ws = None if ws_bytes == 0 else torch.zeros(ws_bytes, dtype=torch.uint8, device=dev)
    stream = torch.cuda.current_stream()

    def step(i):
        # the current stream: the default one, or the capture stream below
        w4.w4a16_gemm(X, blobs[i % copies], Y=Y, workspace=ws, plan=plan)

    for i in range(warmup):
        step(i)
    torch.cuda.synchronize()
    # host time to queue one step (Python + launch), to size the GPU holds below
    h0 = time.perf_counter()
    for i in range(10):
        step(i)
    host_ms = (time.perf_counter() - h0) * 1e3 / 10
    torch.cuda.synchronize()
    # Timed region: exactly `steps` calls, captured once into a HIP graph and
    # replayed between two events, so the GPU runs them back to back without
    # the host's per-call launch cost (the graph is built outside the region).
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        for i in range(steps):
            step(i)
    torch.cuda.synchronize()
    graph.replay()               # one untimed replay
    torch.cuda.synchronize()
    t0 = torch.cuda.Event(enable_timing=True)
    t1 = torch.cuda.Event(enable_timing=True)
    t0.record(stream)
    graph.replay()
    t1.record(stream)
    torch.cuda.synchronize()
    ms_total = t0.elapsed_time(t1)
    ms_step = ms_total / steps
    del graph
    # Per-launch durations for the roofline: a second pass with an event pair
    # around every call (the pairs themselves add a little GPU time).
    ev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
          for _ in range(steps)]
    torch.cuda.synchronize()
    hold_gpu(5.0 + 3.0 * host_ms * steps)
    for i in range(steps):
        ev[i][0].record(stream)
        step(i)
        ev[i][1].record(stream)
    torch.cuda.synchronize()
    per_launch = np.array([a.elapsed_time(b) for a, b in ev])
    kern_ms = float(np.mean(per_launch))

    # Practical read ceiling on the same bytes: the weight blobs read with the
    # split-K kernel's load pattern and no compute (w4a16_read_probe), timed the
    # same way (one graph of 50 calls over the rotating copies).
    read_gbs = None
    try:
        pbytes = base.data.numel() // 1024 * 1024
        pout = torch.empty(w4.w4a16_read_probe_out_bytes(), dtype=torch.uint8, device=dev)
        for i in range(5):
            w4.w4a16_read_probe(blobs[i % copies].data, pbytes, out=pout)
        torch.cuda.synchronize()
        pg = torch.cuda.CUDAGraph()
        with torch.cuda.graph(pg):
            for i in range(50):
                w4.w4a16_read_probe(blobs[i % copies].data, pbytes, out=pout)
        torch.cuda.synchronize()
        pg.replay()
        torch.cuda.synchronize()
        t0.record(stream)
        pg.replay()
        t1.record(stream)
        torch.cuda.synchronize()
        read_gbs = pbytes / (t0.elapsed_time(t1) / 50 * 1e-3) / 1e9
        del pg, pout
    except RuntimeError as e:
        read_gbs = None
        print(f"read probe skipped: {str(e)[:120]}", file=sys.stderr)

    nbytes = algorithmic_bytes(cfg)
    flops = algorithmic_flops(cfg)
    bound = bound_of(cfg)
    # the timed region holds nothing but back-to-back launches of the kernel,
    # so its average per step is the kernel's average launch duration
    if bound == "hbm":
        achieved = nbytes / (ms_step * 1e-3) / 1e9
        roof = {"bound": "hbm", "achieved": round(achieved, 1), "peak": HBM_PEAK_GBS,
                "unit": "GB/s", "frac": round(achieved / HBM_PEAK_GBS, 4),
                "traffic": measured_traffic(name)}
    else:
        achieved = flops / (ms_step * 1e-3) / 1e12
        roof = {"bound": "mfma", "achieved": round(achieved, 1), "peak": MFMA_PEAK_TFLOPS,
                "unit": "TFLOP/s", "frac": round(achieved / MFMA_PEAK_TFLOPS, 4),
                "traffic": measured_traffic(name)}
    out = {
        "metric": METRIC,
        "value": round(nbytes / (ms_step * 1e-3) / 1e9, 1),
        "unit": "GB/s",
        "n_gpus": 1,
        "steps": steps,
        "warmup": warmup,
        "ms_per_step": round(ms_step, 5),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "f16" if p.dtype == "fp16" else "bf16",
        "data": "synthetic",
        "config": {"workload": name, "M": p.M, "K": p.K, "N": p.N, "group_size": p.G,
                   "plan": plan,
                   "act_dtype": p.dtype, "quant": "sym" if p.sym else "asym",
                   "outlier_cols": cfg.get("outlier_frac", 0.0), "parallelism": "none (1 GPU)",
                   "cold_weight_copies": copies, "launch": "hip_graph_replay"},
        "kernel_us": round(ms_step * 1e3, 3),
        "host_us_per_call": round(host_ms * 1e3, 2),
        "kernel_us_event_pairs_mean_p10_p50_p90": [round(kern_ms * 1e3, 3)] + [
            round(float(np.percentile(per_launch, q)) * 1e3, 3) for q in (10, 50, 90)],
        "tflops": round(flops / (ms_step * 1e-3) / 1e12, 2),
        "algorithmic_bytes": nbytes,
        "kernel_source_hash": kernel_source_hash(),
        "weight_only_gbs": round((p.K * p.N // 2) / (ms_step * 1e-3) / 1e9, 1),
        "read_probe_gbs": None if read_gbs is None else round(read_gbs, 1),
        "frac_of_read_probe": None if read_gbs is None else round(
            nbytes / (ms_step * 1e-3) / 1e9 / read_gbs, 4),
        "roofline": roof,
    }
    if comparators:
        out["comparators"] = comparator_times(p, X, blobs, copies, stream)
    if with_cpu:
        out["cpu_baseline"] = cpu_baseline(name, cfg)
    return out


def time_steps(step, steps, warmup):
    """(ms per step over `steps` calls in one HIP graph between two events,
    per-launch durations in ms from event pairs around each call)."""
    import torch

    stream = torch.cuda.current_stream()
    for i in range(warmup):
        step(i)
    torch.cuda.synchronize()
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        for i in range(steps):
            step(i)
    torch.cuda.synchronize()
    graph.replay()
    torch.cuda.synchronize()
    t0 = torch.cuda.Event(enable_timing=True)
    t1 = torch.cuda.Event(enable_timing=True)
    t0.record(stream)
    graph.replay()
    t1.record(stream)
    torch.cuda.synchronize()
    ms_step = t0.elapsed_time(t1) / steps
    del graph
    ev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
          for _ in range(steps)]
    hold_gpu(5.0 + 0.1 * steps)
    for i in range(steps):
        ev[i][0].record(stream)
        step(i)
        ev[i][1].record(stream)
    torch.cuda.synchronize()
    return ms_step, np.array([a.elapsed_time(b) for a, b in ev])


def w8_bytes(cfg):
    """Algorithmic bytes of one W4A8 call: the blob (codes, group constants,
    column scales), the int8 activations and their row scales, the fp16 output."""
    M, K, N, G = cfg["M"], cfg["K"], cfg["N"], cfg["G"]
    return K * N // 2 + (K // G) * N * 2 + N * 4 + M * K + M * 4 + M * N * 2


def run_workload_w8(name, steps, warmup, rotate_bytes=1 << 30):
    """One W4A8 workload (w4a8_gemm, fp16 output) with the protocol of
    run_workload: cold weight copies, `steps` calls in one HIP graph between
    two events, then per-launch event pairs."""
    import torch

    import w4a16_dequant_gemm_amd as w4
    from w4a16_dequant_gemm_amd import w4a8 as w8

    w4.load_library()
    cfg = dict(synth.W4A8_WORKLOADS[name])
    M, K, N, G = cfg["M"], cfg["K"], cfg["N"], cfg["G"]
    dev = torch.device("cuda:0")
    p = synth.make_w4a8_problem(seed=0, **cfg)
    xq = torch.from_numpy(p.xq).to(dev)
    sx = torch.from_numpy(p.sx).to(dev)
    base = w8.w4a8_repack(torch.from_numpy(p.qweight.view(np.int32)).to(dev),
                          torch.from_numpy(p.s8).to(dev), torch.from_numpy(p.a).to(dev),
                          torch.from_numpy(p.sw).to(dev), K, N, G)
    copies = max(2, min(16, math.ceil(rotate_bytes / base.data.numel())))
    blobs = [base] + [w8.PackedW8(base.data.clone(), K, N, G) for _ in range(copies - 1)]
    Y = torch.empty((M, N), dtype=torch.float16, device=dev)

    def step(i):
        w8.w4a8_gemm(xq, sx, blobs[i % copies], out="fp16", Y=Y)

    ms_step, per_launch = time_steps(step, steps, warmup)
    nbytes = w8_bytes(cfg)
    ops = 2 * M * N * K
    gbs = nbytes / (ms_step * 1e-3) / 1e9
    tops = ops / (ms_step * 1e-3) / 1e12
    # ridge of the int8 roofline: 5.0e15 / 8e12 = 625 op/byte
    if ops / nbytes > INT8_PEAK_TOPS / HBM_PEAK_GBS * 1e3:
        roof = {"bound": "mfma", "achieved": round(tops, 1), "peak": INT8_PEAK_TOPS,
                "unit": "TOP/s (int8)", "frac": round(tops / INT8_PEAK_TOPS, 4)}
    else:
        roof = {"bound": "hbm", "achieved": round(gbs, 1), "peak": HBM_PEAK_GBS, "unit": "GB/s",
                "frac": round(gbs / HBM_PEAK_GBS, 4)}
    roof["traffic"] = measured_traffic(name, KERNEL_SOURCES_W4A8)
    return {
        "ms_per_step": round(ms_step, 5), "steps": steps, "kernel_us": round(ms_step * 1e3, 3),
        "kernel_us_event_pairs_mean_p50": [round(float(np.mean(per_launch)) * 1e3, 3),
                                           round(float(np.median(per_launch)) * 1e3, 3)],
        "gbs": round(gbs, 1), "tops_int8": round(tops, 1), "algorithmic_bytes": nbytes,
        "roofline": roof, "kernel_source_hash": kernel_source_hash(KERNEL_SOURCES_W4A8),
        "config": {"workload": name, "M": M, "K": K, "N": N, "group_size": G,
                   "act": "int8 per row", "out": "fp16", "cold_weight_copies": copies,
                   "launch": "hip_graph_replay"},
    }


def mx_bytes(cfg):
    """Algorithmic bytes of one MXFP4 call: the blob (E2M1 codes and E8M0
    block scales), the E4M3 activations and their block scales, the fp16 output."""
    M, K, N = cfg["M"], cfg["K"], cfg["N"]
    return K * N // 2 + K * N // 32 + M * K + M * K // 32 + M * N * 2


def run_workload_mx(name, steps, warmup, rotate_bytes=1 << 30):
    """One MXFP4 workload (mxfp4_gemm, fp16 output), protocol of run_workload_w8."""
    import torch

    import w4a16_dequant_gemm_amd as w4
    from w4a16_dequant_gemm_amd import mxfp4 as mx

    w4.load_library()
    cfg = dict(synth.MXFP4_WORKLOADS[name])
    M, K, N = cfg["M"], cfg["K"], cfg["N"]
    dev = torch.device("cuda:0")
    p = synth.make_mxfp4_problem(seed=0, **cfg)
    xq = torch.from_numpy(p.xq).to(dev)
    xs = torch.from_numpy(p.xs).to(dev)
    base = mx.mxfp4_repack(torch.from_numpy(p.qweight.view(np.int32)).to(dev),
                           torch.from_numpy(p.ws).to(dev), K, N)
    copies = max(2, min(16, math.ceil(rotate_bytes / base.data.numel())))
    blobs = [base] + [mx.PackedMX(base.data.clone(), K, N) for _ in range(copies - 1)]
    Y = torch.empty((M, N), dtype=torch.float16, device=dev)

    def step(i):
        mx.mxfp4_gemm(xq, xs, blobs[i % copies], out="fp16", Y=Y)

    ms_step, per_launch = time_steps(step, steps, warmup)
    nbytes = mx_bytes(cfg)
    flops = 2 * M * N * K
    gbs = nbytes / (ms_step * 1e-3) / 1e9
    tf = flops / (ms_step * 1e-3) / 1e12
    if flops / nbytes > FP8_PEAK_TFLOPS / HBM_PEAK_GBS * 1e3:
        roof = {"bound": "mfma", "achieved": round(tf, 1), "peak": FP8_PEAK_TFLOPS,
                "unit": "TFLOP/s (fp8 x fp4)", "frac": round(tf / FP8_PEAK_TFLOPS, 4)}
    else:
        roof = {"bound": "hbm", "achieved": round(gbs, 1), "peak": HBM_PEAK_GBS, "unit": "GB/s",
                "frac": round(gbs / HBM_PEAK_GBS, 4)}
    roof["traffic"] = measured_traffic(name, KERNEL_SOURCES_MXFP4)
    return {
        "ms_per_step": round(ms_step, 5), "steps": steps, "kernel_us": round(ms_step * 1e3, 3),
        "kernel_us_event_pairs_mean_p50": [round(float(np.mean(per_launch)) * 1e3, 3),
                                           round(float(np.median(per_launch)) * 1e3, 3)],
        "gbs": round(gbs, 1), "tflops": round(tf, 1), "algorithmic_bytes": nbytes,
        "roofline": roof, "kernel_source_hash": kernel_source_hash(KERNEL_SOURCES_MXFP4),
        "config": {"workload": name, "M": M, "K": K, "N": N, "block": 32,
                   "act": "E4M3 + E8M0 per 32", "weight": "E2M1 + E8M0 per 32", "out": "fp16",
                   "cold_weight_copies": copies, "launch": "hip_graph_replay"},
    }


def comparator_times(p, X, blobs, copies, stream, reps=20):
    """Context, not the metric: a dense fp16/bf16 torch.matmul (hipBLASLt) on the
    same shape, and the unfused route (dequantize to HBM, then torch.matmul)."""
    import torch

    import w4a16_dequant_gemm_amd as w4

    res = {}
    try:
        Wd = [w4.w4a16_dequant(blobs[i]) for i in range(min(copies, 4))]
        torch.cuda.synchronize()

        def timeit(fn):
            for i in range(3):
                fn(i)
            torch.cuda.synchronize()
            a = torch.cuda.Event(enable_timing=True)
            b = torch.cuda.Event(enable_timing=True)
            hold_gpu(5.0 + 0.15 * reps)
            a.record(stream)
            for i in range(reps):
                fn(i)
            b.record(stream)
            torch.cuda.synchronize()
            return a.elapsed_time(b) / reps * 1e3

        res["dense_matmul_us"] = round(timeit(lambda i: torch.matmul(X, Wd[i % len(Wd)])), 3)
        res["unfused_dequant_then_matmul_us"] = round(
            timeit(lambda i: torch.matmul(X, w4.w4a16_dequant(blobs[i % copies]))), 3)
        res["note"] = ("dense W held in HBM, rotated over %d copies; unfused writes the "
                       "dequantized W to HBM then multiplies" % len(Wd))
        del Wd
    except RuntimeError as e:   # e.g. out of memory for the dense copies
        res["error"] = str(e)[:200]
    return res


LAYER_PREFIX = "ffn_layer_"
LAYER_WORKLOADS = {f"ffn_layer_decode_m{m}_h8192_f28672_fp16_asym_g128": dict(M=m, H=8192, F=28672)
                   for m in (1, 8)}


def run_ffn_layer(name, steps, warmup, rotate_bytes=1 << 30):
    """A decoder FFN block of a 70B-class model on the W4A16 path, the three
    GEMMs with their epilogues fused and the launches captured in one HIP graph:
        G = silu(X Wg);  H = (X Wu) * G;  Y = H Wd + X  (residual)
    against the same GEMMs without epilogues followed by separate elementwise
    launches (silu, multiply, add).  Weights rotate over cold copies."""
    import torch

    import w4a16_dequant_gemm_amd as w4

    cfg = LAYER_WORKLOADS[name]
    M, H, F, G = cfg["M"], cfg["H"], cfg["F"], 128
    dev = torch.device("cuda:0")
    flags = w4.flags_of("fp16", False)

    def packed_of(K, N, seed):
        qw, sc, zr, _ = synth.make_weights(K, N, G, "fp16", False, seed=seed)
        t = w4.to_device(synth.Problem(1, K, N, G, "fp16", False, np.zeros((1, K), np.uint16),
                                       qw, sc, zr), dev)
        return w4.w4a16_repack(t[1], t[2], t[3], K, N, G, flags)

    base = [packed_of(H, F, 11), packed_of(H, F, 12), packed_of(F, H, 13)]
    layer_bytes = sum(b.data.numel() for b in base)
    copies = max(2, min(8, math.ceil(rotate_bytes / layer_bytes)))
    sets = [base] + [[w4.PackedW4(b.data.clone(), b.K, b.N, b.group_size, b.flags,
                                  b.layout_version) for b in base] for _ in range(copies - 1)]
    X = torch.from_numpy(synth.make_activations(M, H, "fp16", seed=0).view("int16")).view(
        torch.float16).to(dev)
    Gt = torch.empty((M, F), dtype=torch.float16, device=dev)
    Ht = torch.empty_like(Gt)
    Y = torch.empty((M, H), dtype=torch.float16, device=dev)
    U = torch.empty_like(Gt)
    ws = w4.workspace_for(max(w4.w4a16_workspace_bytes(M, F, H, G, flags),
                              w4.w4a16_workspace_bytes(M, H, F, G, flags)), dev)
    stream = torch.cuda.current_stream()

    def fused(i):
        wg, wu, wd = sets[i % copies]
        w4.w4a16_gemm_ex(X, wg, Y=Gt, workspace=ws, activation="silu")
        w4.w4a16_gemm_ex(X, wu, Y=Ht, workspace=ws, aux=Gt, aux_op="mul")
        w4.w4a16_gemm_ex(Ht, wd, Y=Y, workspace=ws, aux=X, aux_op="add")

    def unfused(i):
        wg, wu, wd = sets[i % copies]
        w4.w4a16_gemm(X, wg, Y=Gt, workspace=ws)
        torch.nn.functional.silu(Gt, inplace=True)
        w4.w4a16_gemm(X, wu, Y=U, workspace=ws)
        torch.mul(U, Gt, out=Ht)
        w4.w4a16_gemm(Ht, wd, Y=Y, workspace=ws)
        Y.add_(X)

    def graph_time(fn):
        for i in range(warmup):
            fn(i)
        torch.cuda.synchronize()
        g = torch.cuda.CUDAGraph()
        with torch.cuda.graph(g):
            for i in range(steps):
                fn(i)
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        a = torch.cuda.Event(enable_timing=True)
        b = torch.cuda.Event(enable_timing=True)
        a.record(stream)
        g.replay()
        b.record(stream)
        torch.cuda.synchronize()
        del g
        return a.elapsed_time(b) / steps

    ms_fused = graph_time(fused)
    Yf = Y.clone()
    ms_unfused = graph_time(unfused)
    torch.cuda.synchronize()
    diff = float((Yf.float() - Y.float()).abs().max())
    nbytes = layer_bytes + (M * H * 2) * 3 + (M * F * 2) * 3   # weights, X, Y, G, H traffic
    return {
        "metric": "W4A16 FFN layer (3 fused GEMMs, one HIP graph) achieved HBM GB/s",
        "value": round(nbytes / (ms_fused * 1e-3) / 1e9, 1), "unit": "GB/s", "n_gpus": 1,
        "steps": steps, "warmup": warmup, "ms_per_step": round(ms_fused, 5),
        "higher_is_better": True, "scaling": "weak", "vs_baseline": None, "dtype": "f16",
        "data": "synthetic",
        "config": {"workload": name, "M": M, "hidden": H, "ffn": F, "group_size": G,
                   "act_dtype": "fp16", "quant": "asym", "cold_weight_copies": copies,
                   "launch": "hip_graph_replay"},
        "layer_us_fused": round(ms_fused * 1e3, 3),
        "layer_us_unfused_six_launches": round(ms_unfused * 1e3, 3),
        "launches_fused": 3, "launches_unfused": 6,
        "algorithmic_bytes": nbytes,
        "max_abs_diff_fused_vs_unfused": diff,
    }


def main():
    ap = argparse.ArgumentParser(description=__doc__.split("\n")[0])
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=200)
    ap.add_argument("--warmup", type=int, default=20)
    ap.add_argument("--workload", default=DEFAULT_WORKLOAD,
                    help="a name from w4a16_synth.WORKLOADS, W4A8_WORKLOADS or MXFP4_WORKLOADS, "
                         "'all' (one "
                         "line each), or "
                         "one of " + ", ".join(LAYER_WORKLOADS) + " (fused FFN block)")
    ap.add_argument("--no-cpu", action="store_true", help="skip the CPU oracle baseline")
    ap.add_argument("--no-comparators", action="store_true")
    ap.add_argument("--m", type=int, default=None,
                    help="run the workload's weights with this many activation rows instead "
                         "(for sweeps of the kernel choice over M)")
    ap.add_argument("--no-extra", action="store_true",
                    help="skip the extra workloads reported beside a single workload")
    ap.add_argument("--plan", default=None,
                    help="kernel hint, e.g. decode, decode:2, splitk, tiled:4 (default: the "
                         "library's own choice)")
    ap.add_argument("--calibration-copy-mib", type=int, default=0,
                    help="before the workload, run a plain device copy of this many MiB (a "
                         "known-size kernel for scaling rocprofv3 FETCH_SIZE/WRITE_SIZE)")
    args = ap.parse_args()
    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) != 1:
        print(json.dumps({"error": "this benchmark runs on exactly one GPU; the W4A16 path "
                                   "has no multi-GPU mode (a caller shards N across GPUs)",
                          "n_gpus": args.gpus}), flush=True)
        sys.exit(2)
    if args.calibration_copy_mib > 0:
        import torch
        src = torch.ones(args.calibration_copy_mib << 20, dtype=torch.uint8, device="cuda:0")
        dst = torch.empty_like(src)
        torch.cuda.synchronize()
        dst.copy_(src)
        torch.cuda.synchronize()
        del src, dst
    if args.workload.startswith(LAYER_PREFIX):
        print(json.dumps(run_ffn_layer(args.workload, args.steps, args.warmup)), flush=True)
        return
    plan = None
    if args.plan:
        name_, _, param = args.plan.partition(":")
        plan = (name_, int(param or 0))
    names = list(synth.WORKLOADS) if args.workload == "all" else args.workload.split(",")
    if all(n in synth.W4A8_WORKLOADS or n in synth.MXFP4_WORKLOADS for n in names):
        for name in names:
            w8 = name in synth.W4A8_WORKLOADS
            out = (run_workload_w8 if w8 else run_workload_mx)(name, args.steps, args.warmup)
            out.update({"metric": ("W4A8" if w8 else "MXFP4") + " GEMM achieved " +
                        out["roofline"]["unit"],
                        "value": out["roofline"]["achieved"], "unit": out["roofline"]["unit"],
                        "n_gpus": 1, "warmup": args.warmup, "higher_is_better": True,
                        "scaling": "weak", "vs_baseline": None, "dtype": "i8" if w8 else "fp8xfp4",
                        "data": "synthetic"})
            print(json.dumps(out), flush=True)
        return
    for name in names:
        out = run_workload(name, args.steps, args.warmup,
                           with_cpu=not args.no_cpu and len(names) == 1,
                           comparators=not args.no_comparators, plan=plan, rows=args.m)
        if len(names) == 1 and not args.no_extra and plan is None and args.m is None:
            out["extra_workloads"] = extra_workloads(name, min(args.steps, 50), min(args.warmup, 5))
            out["w4a8_workloads"] = w4a8_workloads(min(args.steps, 50), min(args.warmup, 5))
            out["mxfp4_workloads"] = mxfp4_workloads(min(args.steps, 50), min(args.warmup, 5))
        print(json.dumps(out), flush=True)


def extra_workloads(headline, steps, warmup):
    """The roofline entries of EXTRA_WORKLOADS (those other than the headline),
    measured with the same protocol in the same process."""
    import torch

    res = {}
    for name in EXTRA_WORKLOADS:
        if name == headline:
            continue
        o = run_workload(name, steps, warmup, with_cpu=False, comparators=False)
        res[name] = {k: o[k] for k in ("kernel_us", "ms_per_step", "steps", "roofline",
                                       "read_probe_gbs", "tflops", "algorithmic_bytes")}
        res[name]["config"] = {k: o["config"][k] for k in ("M", "K", "N", "group_size",
                                                           "act_dtype", "quant")}
        torch.cuda.empty_cache()
    return res


def w4a8_workloads(steps, warmup):
    """The W4A8 route on its workloads (decode, batch 128, prefill), measured
    with the same protocol in the same process."""
    import torch

    res = {}
    for name in synth.W4A8_WORKLOADS:
        o = run_workload_w8(name, steps, warmup)
        res[name] = {k: o[k] for k in ("kernel_us", "ms_per_step", "steps", "roofline", "gbs",
                                       "tops_int8", "algorithmic_bytes")}
        torch.cuda.empty_cache()
    return res


def mxfp4_workloads(steps, warmup):
    """The MXFP4 route on its workloads, same protocol, same process."""
    import torch

    res = {}
    for name in synth.MXFP4_WORKLOADS:
        o = run_workload_mx(name, steps, warmup)
        res[name] = {k: o[k] for k in ("kernel_us", "ms_per_step", "steps", "roofline", "gbs",
                                       "tflops", "algorithmic_bytes")}
        torch.cuda.empty_cache()
    return res


if __name__ == "__main__":
    main()
