"""Benchmark of the batch-invariant router GEMM on one MI355X.

    python bench.py [--gpus 1] [--steps K] [--warmup W]

Workload (one "step"): the DeepSeek-V4-shaped fp32 router GateLinear,
X[M,4096] x W[256,4096]^T + b, called once for every decode batch size
M in {1,2,4,8,15,16,17,32,33,64,128}.  The weight is cold: each call reads
the next of 96 distinct copies of W (384 MiB in total, more than the 256 MB
Infinity Cache), so HBM claims are not cache hits.  Inputs are synthetic
(seeded normal draws, see workloads.py) and resident in HBM before timing.

Timing: every timed call runs inside a HIP graph (torch.cuda.CUDAGraph),
captured once after an eager pass, so neither the host's launch cost nor the
device cost of per-call events (about 4.4 us for an event pair alone) enters
the figures.  A step is one replay of a graph that holds the whole sweep;
eight such graphs cycle through the W copies.  HIP events bracket only the K
timed replays, queued behind a spin kernel on the same stream.  `value` is
whole-step throughput (algorithmic bytes of the step / step time); the
roofline object reports the decode call's average duration (step time / calls
per step) against the 8 TB/s HBM peak.  Per-M, prefill, bf16, MoE and top-k
figures are per-call averages over a replayed graph of many calls.
The prefill leg (M = 1024, 4096) reports TFLOP/s against the fp32 MFMA peak.
The CPU baseline times the fp64 oracle on the same decode sweep.

Prints exactly one JSON line.
"""
from __future__ import annotations

import argparse
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

HBM_PEAK_GBS = 8000.0
FP32_MFMA_PEAK_TFLOPS = 157.3
BF16_MFMA_PEAK_TFLOPS = 2500.0
N_COPIES = 96

# HBM bytes per launch of the dominant kernel (the XCD hand-over decode), averaged over the sweep's
# calls it serves (M = 1 .. 64), from two rocprofv3 PMC runs: FETCH_SIZE scaled x2.0 and WRITE_SIZE
# x1.0 by a 512 MiB copy of known size (see profiles/router_decode_hbm_bytes.md).  Valid only for the
# kernel sources with this digest; any later change to them reports traffic as null until the counters
# are taken again.
MEASURED_TRAFFIC = {"sources_sha256": "d8308b0fece7ecf0991085c0305957aa77e472a4eb45e60f1fb337bf96fff66d", "bytes_per_call": 7986534}
KERNEL_SOURCES = ("bi_device.h", "bi_launch.h", "bi_linear.hip", "bi_plan.cpp", "bi_plan.h", "bi_table.inc")


def kernel_sources_digest():
    import hashlib
    h = hashlib.sha256()
    for name in KERNEL_SOURCES:
        with open(os.path.join(ROOT, "deterministic_persistent_gemm_amd", "csrc", name), "rb") as f:
            h.update(name.encode() + b"\0" + f.read())
    return h.hexdigest()


def router_bytes(M, N=256, K=4096):
    """Algorithmic HBM bytes of one router call: W, X, bias read once, Y written once."""
    return 4 * (N * K + M * K + M * N + N)


def router_flops(M, N=256, K=4096):
    return 2 * M * N * K


def spin(torch, ms: float):
    """Queue a spin kernel of about `ms` milliseconds on the current stream."""
    torch.cuda._sleep(int(ms * spin.cycles_per_ms))


spin.cycles_per_ms = 1.0e6


def calibrate_spin(torch):
    s, e = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    s.record()
    torch.cuda._sleep(2_000_000)
    e.record()
    torch.cuda.synchronize()
    spin.cycles_per_ms = 2_000_000 / max(s.elapsed_time(e), 1e-3)


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=5)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-prefill", action="store_true")
    ap.add_argument("--no-bf16", action="store_true")
    ap.add_argument("--no-moe", action="store_true")
    ap.add_argument("--no-topk", action="store_true")
    ap.add_argument("--mode", choices=("step", "copy", "cpu-leg"), default="step",
                    help="copy: one 512 MiB device-to-device copy, the known-size kernel that "
                         "scales the PMC byte counters; cpu-leg: time the oracle (child process)")
    ap.add_argument("--seconds", type=float, default=10.0)
    args = ap.parse_args()
    if args.mode == "copy":
        return copy_calibration()
    if args.mode == "cpu-leg":
        return cpu_leg(args.seconds)
    if args.gpus != 1:
        print(json.dumps({"error": "this build runs on one GPU only; --gpus must be 1",
                          "n_gpus": args.gpus}))
        sys.exit(2)

    import numpy as np
    import torch

    import deterministic_persistent_gemm_amd as bi
    import workloads as wl

    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    calibrate_spin(torch)

    w = wl.router_weights(0)
    w_host = torch.from_numpy(w.w)
    copies = [w_host.to(dev) for _ in range(N_COPIES)]
    bias = torch.from_numpy(w.b).to(dev)
    sweep = list(wl.ROUTER_DECODE_M)
    xs = {M: torch.from_numpy(wl.router_batch(M, w).x).to(dev) for M in sweep}
    outs = {M: torch.empty((M, 256), dtype=torch.float32, device=dev) for M in sweep}
    bytes_step = sum(router_bytes(M) for M in sweep)
    calls_per_step = len(sweep)

    stream = torch.cuda.Stream(dev)
    n_graphs = 8

    def sweep_calls(j):
        calls = []
        for c, M in enumerate(sweep):
            wd = copies[(j * calls_per_step + c) % N_COPIES]
            calls.append(lambda M=M, wd=wd: bi.bi_linear_f32(xs[M], wd.t(), bias, out=outs[M]))
        return calls

    graphs = [capture(torch, sweep_calls(j), stream) for j in range(n_graphs)]

    K = args.steps
    with torch.cuda.stream(stream):
        for i in range(args.warmup):
            graphs[i % n_graphs].replay()
        torch.cuda.synchronize()
        t0, t1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        spin(torch, 2.0)
        t0.record()
        for k in range(K):
            graphs[k % n_graphs].replay()
        t1.record()
    torch.cuda.synchronize()
    total_ms = t0.elapsed_time(t1)
    ms_per_step = total_ms / K
    value = bytes_step / (ms_per_step * 1e-3) / 1e9
    del graphs

    per_m = {}
    for M in sweep:
        calls = [lambda M=M, wd=wd: bi.bi_linear_f32(xs[M], wd.t(), bias, out=outs[M]) for wd in copies]
        us = time_graph_calls(torch, calls, stream)
        t = us * 1e-6
        t_hbm = router_bytes(M) / (HBM_PEAK_GBS * 1e9)
        t_mfma = router_flops(M) / (FP32_MFMA_PEAK_TFLOPS * 1e12)
        per_m[str(M)] = {
            "us": round(us, 3),
            "GBps": round(router_bytes(M) / t / 1e9, 1),
            "TFLOPs": round(router_flops(M) / t / 1e12, 2),
            "hbm_frac": round(router_bytes(M) / t / 1e9 / HBM_PEAK_GBS, 4),
            "mfma_frac": round(router_flops(M) / t / 1e12 / FP32_MFMA_PEAK_TFLOPS, 4),
            # which peak binds an ideal kernel at this M (fp32 MFMA from M = 64)
            "bound": "hbm" if t_hbm >= t_mfma else "mfma",
            "path": decode_path_name(bi, M),
        }
    achieved = bytes_step / (ms_per_step * 1e-3) / 1e9
    floors = floors_leg(torch, bi, dev)
    # the dominant kernel: the one-launch XCD hand-over decode, which serves
    # the sweep's small batches; algorithmic bytes per call over its average
    # per-call duration, both averaged over the calls it serves
    xcd_m = [M for M in sweep if per_m[str(M)]["path"] == "decode_xcd"]
    dom = None
    if xcd_m:
        dom_us = sum(per_m[str(M)]["us"] for M in xcd_m) / len(xcd_m)
        dom_bytes = sum(router_bytes(M) for M in xcd_m) / len(xcd_m)
        dom = {"kernel": "k_decode<F32,F32,4,1,HANDOFF> (XCD hand-over decode, one launch per call)",
               "M": xcd_m, "us": round(dom_us, 3), "bytes": int(dom_bytes),
               "GBps": round(dom_bytes / dom_us / 1e3, 1)}

    extra = {"decode_per_M": per_m, "weight": f"cold: {N_COPIES} rotating copies of W (384 MiB)",
             "timing": "HIP graph replay; events bracket only the timed replays",
             "event_pair_floor_us": round(event_pair_floor(torch, stream), 2),
             "floors": floors, "step_GBps": round(achieved, 1)}

    if not args.no_prefill:
        extra["prefill"] = prefill_leg(torch, np, bi, wl, w, copies, bias, dev)
    del copies
    if not args.no_bf16:
        extra["dense_bf16"] = dense_bf16_leg(torch, np, bi, wl, dev)
    if not args.no_moe:
        extra["moe"] = moe_leg(torch, np, bi, wl, dev, floors["cold_read_1GiB"]["GBps"])
    if not args.no_topk:
        extra["indexer_topk"] = topk_leg(torch, np, bi, wl, dev)

    cpu = None
    if not args.no_cpu_baseline:
        cpu = cpu_baseline(sweep)

    line = {
        "metric": "router GateLinear fp32 GEMM, decode sweep M=1..128: HBM GB/s (bit-invariant)",
        "value": round(value, 1),
        "unit": "GB/s",
        "n_gpus": 1,
        "steps": K,
        "warmup": args.warmup,
        "ms_per_step": round(ms_per_step, 5),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "f32",
        "data": "synthetic",
        "config": {"workload": "DSv4 router GateLinear fp32, X[M,4096] W[256,4096] (weight.t()) + bias, "
                               "decode sweep M in {1,2,4,8,15,16,17,32,33,64,128}",
                   "sweep": sweep, "N": 256, "K": 4096},
        "roofline": roofline_line(dom, achieved, floors),
        "cpu_baseline": cpu,
        "extra": extra,
    }
    print(json.dumps(line))


def prefill_leg(torch, np, bi, wl, w, copies, bias, dev):
    """The router at the prefill sizes (M = 1024, 4096) and, between decode
    and prefill, at M = 256 and 512 (the k-split ring tiles)."""
    res = {}
    stream = torch.cuda.Stream(dev)
    for M in (256, 512) + tuple(wl.ROUTER_PREFILL_M):
        x = torch.from_numpy(wl.router_batch(M, w).x).to(dev)
        out = torch.empty((M, 256), dtype=torch.float32, device=dev)
        calls = [lambda wd=wd: bi.bi_linear_f32(x, wd.t(), bias, out=out) for wd in copies[:24]]
        us = time_graph_calls(torch, calls, stream)
        tf = router_flops(M) / (us * 1e-6) / 1e12
        res[str(M)] = {"us": round(us, 2), "TFLOPs": round(tf, 2),
                       "mfma_frac": round(tf / FP32_MFMA_PEAK_TFLOPS, 4)}
    return res


def capture(torch, calls, stream):
    """One HIP graph of `calls`, captured on `stream` after an eager pass there
    (which also sizes the library workspace outside the graph)."""
    with torch.cuda.stream(stream):
        for c in calls:
            c()
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g, stream=stream):
        for c in calls:
            c()
    torch.cuda.synchronize()
    return g


def time_graph_calls(torch, calls, stream, reps=3):
    """Average device time of one call in microseconds: the calls are captured
    into one graph, which is replayed `reps` times back to back behind a spin
    kernel, with HIP events around the replays only."""
    g = capture(torch, calls, stream)
    with torch.cuda.stream(stream):
        g.replay()
        torch.cuda.synchronize()
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        spin(torch, 1.0)
        e0.record()
        for _ in range(reps):
            g.replay()
        e1.record()
    torch.cuda.synchronize()
    del g
    return e0.elapsed_time(e1) * 1e3 / (reps * len(calls))


def event_pair_floor(torch, stream, n=50):
    """Device time between two HIP events recorded back to back (us)."""
    import statistics
    with torch.cuda.stream(stream):
        ev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in range(n)]
        spin(torch, 1.0)
        for a, b in ev:
            a.record()
            b.record()
    torch.cuda.synchronize()
    return statistics.median(a.elapsed_time(b) * 1e3 for a, b in ev)


def time_calls(torch, np, fn, n):
    """Average device time of fn(i) in microseconds over i = 0..n-1, from a
    replayed graph of the n calls."""
    stream = torch.cuda.Stream()
    return time_graph_calls(torch, [lambda i=i: fn(i) for i in range(n)], stream)


def dense_bf16_leg(torch, np, bi, wl, dev):
    """bf16 dense X[M,4096] W[4096,4096] -> bf16, cold W (12 rotating copies, 384 MiB)."""
    w = wl.dense_bf16_weights(0)
    wt = torch.from_numpy(w.w.view(np.int16)).view(torch.bfloat16).to(dev)
    copies = [wt] + [wt.clone() for _ in range(11)]
    res = {}
    for M in wl.DENSE_M_SWEEP:
        x = torch.from_numpy(wl.dense_bf16_batch(M, w).x.view(np.int16)).view(torch.bfloat16).to(dev)
        out = torch.empty((M, 4096), dtype=torch.bfloat16, device=dev)
        us = time_calls(torch, np, lambda i: bi.bi_linear_bf16(x, copies[i % 12].t(), None, out=out),
                        10 if M >= 1024 else 30)
        nbytes = 2 * (4096 * 4096 + M * 4096 + M * 4096)
        flops = 2 * M * 4096 * 4096
        res[str(M)] = {"us": round(us, 2), "GBps": round(nbytes / us / 1e3, 1),
                       "TFLOPs": round(flops / us / 1e6, 1),
                       "hbm_frac": round(nbytes / us / 1e3 / HBM_PEAK_GBS, 4),
                       "mfma_frac": round(flops / us / 1e6 / BF16_MFMA_PEAK_TFLOPS, 4)}
    return res


def moe_leg(torch, np, bi, wl, dev, stream_gbs=None):
    """Qwen3-30B-A3B-shaped MoE layer; algorithmic bytes count each distinct
    expert touched once (measured from the returned ids).  stream_frac: the
    rate against the long cold read of the same run (floors.cold_read_1GiB)."""
    w = wl.moe_weights(0)
    wr = torch.from_numpy(w.w_router).to(dev)
    w13 = torch.from_numpy(w.w13.view(np.int16)).view(torch.bfloat16).to(dev)
    w2 = torch.from_numpy(w.w2.view(np.int16)).view(torch.bfloat16).to(dev)
    H, E, I, k = wl.MOE_H, wl.MOE_E, wl.MOE_I, wl.MOE_TOPK
    res = {}
    for M in wl.MOE_M_SWEEP:
        x = torch.from_numpy(wl.moe_batch(M, w).x.view(np.int16)).view(torch.bfloat16).to(dev)
        _, ids, _ = bi.bi_moe_grouped_gemm(x, wr, None, w13, w2, k)
        distinct = int(torch.unique(ids).numel())
        us = time_calls(torch, np, lambda i: bi.bi_moe_grouped_gemm(x, wr, None, w13, w2, k), 20)
        nbytes = (E * H * 4 + M * H * 2 + distinct * 3 * I * H * 2 + M * H * 4 + M * k * 8)
        flops = 2 * M * E * H + 2 * M * k * 3 * I * H
        res[str(M)] = {"us": round(us, 2), "distinct_experts": distinct,
                       "GBps": round(nbytes / us / 1e3, 1), "TFLOPs": round(flops / us / 1e6, 2),
                       "hbm_frac": round(nbytes / us / 1e3 / HBM_PEAK_GBS, 4)}
        if stream_gbs:
            res[str(M)]["stream_frac"] = round(nbytes / us / 1e3 / stream_gbs, 4)
    # squared-ReLU experts (w1 = the gate half), weights applied in an fp32 top-k sum
    w1 = w13[:, :I, :].contiguous()
    for M in (16, 256):
        x = torch.from_numpy(wl.moe_batch(M, w).x.view(np.int16)).view(torch.bfloat16).to(dev)
        f = lambda i: bi.bi_moe_grouped_gemm_ex(x, wr, None, w1, w2, k, activation=bi.BI_ACT_SQRELU,
                                                probs_at_activation=False, apply_weights=True, acc_fp64=False)
        _, ids, _ = f(0)
        distinct = int(torch.unique(ids).numel())
        us = time_calls(torch, np, f, 20)
        nbytes = (E * H * 4 + M * H * 2 + distinct * 2 * I * H * 2 + M * H * 4 + M * k * 8)
        res[f"sqrelu_{M}"] = {"us": round(us, 2), "distinct_experts": distinct,
                              "GBps": round(nbytes / us / 1e3, 1),
                              "hbm_frac": round(nbytes / us / 1e3 / HBM_PEAK_GBS, 4)}
        if stream_gbs:
            res[f"sqrelu_{M}"]["stream_frac"] = round(nbytes / us / 1e3 / stream_gbs, 4)
    return res


def topk_leg(torch, np, bi, wl, dev):
    """Deterministic indexer top-k (8192 columns): decode batches of 1, 8 and
    64 rows and a 4096-row packed causal prefill, top-k 2048.  Algorithmic
    bytes: the in-window scores read once plus the int32 output written once;
    8 rotating copies of the scores keep them out of L2."""
    res = {}
    cases = [(f"decode_{n}", wl.indexer_decode(n)) for n in wl.INDEXER_DECODE_ROWS]
    cases.append((f"prefill_{wl.INDEXER_PREFILL_ROWS}", wl.indexer_prefill(wl.INDEXER_PREFILL_ROWS)))
    topk = 2048
    for name, b in cases:
        rows = b.scores.shape[0]
        s = torch.from_numpy(b.scores).to(dev)
        copies = [s] + [s.clone() for _ in range(7)]
        rs = torch.from_numpy(b.row_start).to(dev)
        re = torch.from_numpy(b.row_end).to(dev)
        out = torch.empty((rows, topk), dtype=torch.int32, device=dev)
        us = time_calls(torch, np, lambda i: bi.bi_indexer_topk(copies[i % 8], topk, rs, re, out=out),
                        10 if rows > 1024 else 30)
        win = np.clip(b.row_end, 0, b.scores.shape[1]) - np.clip(b.row_start, 0, b.scores.shape[1])
        nbytes = int(4 * np.maximum(win, 0).sum() + 4 * rows * topk + 16 * rows)
        res[name] = {"us": round(us, 2), "rows": rows, "GBps": round(nbytes / us / 1e3, 1),
                     "hbm_frac": round(nbytes / us / 1e3 / HBM_PEAK_GBS, 4)}
    return res


def copy_calibration():
    """One device-to-device copy of exactly 512 MiB (read 512 MiB, write 512 MiB)."""
    import torch
    dev = torch.device("cuda:0")
    n = 512 * 1024 * 1024 // 4
    a = torch.ones(n, dtype=torch.float32, device=dev)
    b = torch.empty_like(a)
    torch.cuda.synchronize()
    b.copy_(a)
    torch.cuda.synchronize()
    print(json.dumps({"copy_bytes": 4 * n, "ok": bool(b[-1].item() == 1.0)}))


def cpu_leg(seconds):
    """Child process: the fp64 oracle as it stands on the decode sweep for about
    `seconds` seconds, with whatever OMP_NUM_THREADS the parent set."""
    import oracle
    import workloads as wl
    w = wl.router_weights(0)
    sweep = list(wl.ROUTER_DECODE_M)
    batches = {M: wl.router_batch(M, w).x for M in sweep}
    reps = 0
    t0 = time.perf_counter()
    while True:
        for M in sweep:
            oracle.linear_f32(batches[M], w.w, w.b)
        reps += 1
        if time.perf_counter() - t0 > seconds:
            break
    dt = time.perf_counter() - t0
    print(json.dumps({"reps": reps, "seconds": dt, "threads": oracle.num_threads(),
                      "GBps": sum(router_bytes(M) for M in sweep) * reps / dt / 1e9}))


def cpu_model():
    try:
        with open("/proc/cpuinfo") as f:
            for line in f:
                if line.startswith("model name"):
                    return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return None


def cpu_baseline(sweep, seconds=10.0):
    """The fp64 oracle on the decode sweep, timed on the host cores in child
    processes: at OMP_NUM_THREADS=1 and at the thread count the environment
    sets (all host CPUs when it sets none)."""
    import subprocess
    runs = {}
    for label, threads in (("multi", os.environ.get("OMP_NUM_THREADS") or str(os.cpu_count())), ("one", "1")):
        env = dict(os.environ, OMP_NUM_THREADS=threads)
        out = subprocess.run([sys.executable, os.path.abspath(__file__), "--mode", "cpu-leg",
                              "--seconds", str(seconds)], env=env, capture_output=True, text=True, check=True)
        runs[label] = json.loads(out.stdout.strip().splitlines()[-1])
    m, o = runs["multi"], runs["one"]
    return {"value": round(m["GBps"], 3), "unit": "GB/s", "cores": m["threads"], "kind": "oracle",
            "sample": f"{m['reps']} passes of the decode sweep (M in {sweep}, N=256, K=4096), fp64 C oracle, "
                      f"{m['seconds']:.1f} s on {m['threads']} threads",
            "value_1_thread": round(o["GBps"], 3),
            "sample_1_thread": f"{o['reps']} passes, {o['seconds']:.1f} s on 1 thread",
            "host_cpus": os.cpu_count(), "cpu_model": cpu_model()}


def decode_path_name(bi, M, N=256, K=4096):
    """Which decode kernel the automatic plan picks for M rows of the router."""
    return {bi.BI_PATH_DECODE: "decode_two_launch", bi.BI_PATH_DECODE_XCD: "decode_xcd",
            bi.BI_PATH_PERSISTENT: "persistent", bi.BI_PATH_DECODE_WG: "decode_wg",
            bi.BI_PATH_DECODE_DMA: "decode_dma"}.get(bi.plan_path(bi.BI_F32, M, N, K), "?")


def floors_leg(torch, bi, dev):
    """What a launch and a cold read cost on this part, and the shader clock.
    Empty kernel: 512 workgroups, per launch in a replayed graph of 100
    launches (one or two per group).  Cold reads: 4 MiB (96 copies) and
    32 MiB (12 copies) read once each by a plain streaming kernel (256 and 512
    workgroups of 256 threads, the fastest measured), and 1 GiB (two copies,
    1024 workgroups) for the streaming rate of a long read.  L2 read: the rate
    at which the L2 delivers resident data to the compute units.  Clock: shader cycles
    (s_memtime) per 100 MHz wall tick over a dependent fp32 chain, with one
    wave per compute unit and with eight."""
    stream = torch.cuda.Stream(dev)
    res = {}
    one = time_graph_calls(torch, [lambda: bi.bi_lab_empty(512)] * 100, stream)
    two = time_graph_calls(torch, [lambda: (bi.bi_lab_empty(512), bi.bi_lab_empty(512))] * 50, stream)
    res["empty_kernel_us"] = round(one, 3)
    res["two_empty_kernels_us"] = round(two, 3)
    for mib, ncopy, grid in ((4, 96, 256), (32, 12, 512)):
        nb = mib << 20
        bufs = [torch.ones(nb // 4, dtype=torch.float32, device=dev) for _ in range(ncopy)]
        sink = torch.empty(grid, dtype=torch.int32, device=dev)
        us = time_graph_calls(torch, [lambda b=b: bi.bi_lab_stream_read(b, sink, grid) for b in bufs], stream)
        res[f"cold_read_{mib}MiB"] = {"us": round(us, 3), "GBps": round(nb / us / 1e3, 1), "workgroups": grid}
        del bufs
    # the streaming rate of a long read: what any kernel that reads a large
    # weight once can reach (two 1 GiB buffers, 1024 workgroups)
    nb = 1 << 30
    bufs = [torch.ones(nb // 4, dtype=torch.float32, device=dev) for _ in range(2)]
    sink = torch.empty(1024, dtype=torch.int32, device=dev)
    us = time_graph_calls(torch, [lambda b=b: bi.bi_lab_stream_read(b, sink, 1024) for b in bufs], stream)
    res["cold_read_1GiB"] = {"us": round(us, 1), "GBps": round(nb / us / 1e3, 1), "workgroups": 1024}
    del bufs
    # L2 to compute units: 512 workgroups each read the same 1 MiB (held in
    # every XCD's L2 after the first pass) four times
    src = torch.ones(1 << 18, dtype=torch.float32, device=dev)
    sink = torch.empty(512, dtype=torch.int32, device=dev)
    us = time_graph_calls(torch, [lambda: bi.bi_lab_l2_read(src, sink, 512, 4)] * 4, stream)
    gbs = 512 * 4 * (1 << 20) / us / 1e3
    res["l2_read"] = {"GBps": round(gbs, 1), "GBps_per_CU": round(gbs / 256, 1), "workgroups": 512,
                      "probe": "every workgroup reads the same L2-resident 1 MiB, 16-byte loads, 8 in flight"}
    out = torch.zeros((2048, 3), dtype=torch.int64, device=dev)
    for grid, name in ((256, "sclk_MHz_one_wave_per_CU"), (2048, "sclk_MHz_eight_waves_per_CU")):
        with torch.cuda.stream(stream):
            bi.bi_lab_clock(out, grid, 2000)
        torch.cuda.synchronize()
        o = out[:grid].cpu().numpy().astype("float64")
        res[name] = round(float(sorted(o[:, 0] / o[:, 1])[grid // 2] * 100.0), 1)
    res.update(ceilings_leg(torch, bi, dev))
    return res


def ceilings_leg(torch, bi, dev):
    """What a compute unit sustains with nothing else in the way: LDS read
    bytes per shader clock (one 16-wave workgroup per CU reading 64 KiB of LDS
    with conflict-free 16-byte loads) and the issue interval of the recipe's
    MFMA instructions on register operands (eight waves per CU, two per SIMD,
    eight independent chains each, and one, two or four).  Cycles and clock come from the probes'
    own shader-cycle and wall-tick counters (median over the workgroups)."""
    grid = 256
    out = torch.zeros((grid, 3), dtype=torch.int64, device=dev)

    def run(launch):
        launch()                      # warm-up
        torch.cuda.synchronize()
        launch()
        torch.cuda.synchronize()
        o = out.cpu().numpy().astype("float64")
        cyc = float(sorted(o[:, 0])[grid // 2])
        mhz = float(sorted(o[:, 0] / o[:, 1])[grid // 2] * 100.0)
        return cyc, mhz

    res = {}
    iters = 1000
    cyc, mhz = run(lambda: bi.bi_lab_lds_read(out, grid, iters))
    res["lds_read"] = {"B_per_clk_per_CU": round(iters * 65536 / cyc, 1), "MHz": round(mhz, 1),
                       "probe": "16 waves per CU, ds_read_b128, conflict-free"}
    for name, dtype, iters, flop, peak in (("mfma_bf16_16x16x32", bi.BI_BF16, 2000, 16384, 2500.0),
                                           ("mfma_f32_16x16x4", bi.BI_F32, 1000, 2048, FP32_MFMA_PEAK_TFLOPS)):
        cyc, mhz = run(lambda d=dtype, n=iters: bi.bi_lab_mfma_rate(out, d, grid, n))
        per = cyc / (iters * 8 * 2)            # two waves per SIMD, eight MFMAs per round
        tf = 256 * 4 * mhz * 1e6 / per * flop / 1e12
        res[name] = {"cycles_per_instr_per_SIMD": round(per, 2), "MHz": round(mhz, 1),
                     "TFLOPs": round(tf, 1), "frac_of_peak": round(tf / peak, 3),
                     "probe": "register operands, 8 waves per CU, 8 independent chains per wave"}
        # the same with fewer accumulators per wave: each MFMA depends on the
        # one `chains` before it, as the recipe's tile partials do
        res[name]["cycles_per_instr_per_SIMD_by_chains"] = {
            str(ch): round(run(lambda d=dtype, n=iters, c=ch: bi.bi_lab_mfma_rate(out, d, grid, n, c))[0]
                           / (iters * 8 * 2), 2)
            for ch in (1, 2, 4)}
    return res


def roofline_line(dom, step_gbps, floors):
    """The roofline object for the dominant kernel: algorithmic bytes per call
    of the one-launch decode over its average duration, against the 8 TB/s
    HBM peak and, for context, against what a plain kernel reading the same
    4 MiB cold achieves here."""
    cold = floors["cold_read_4MiB"]["GBps"]
    traffic = (MEASURED_TRAFFIC["bytes_per_call"]
               if kernel_sources_digest() == MEASURED_TRAFFIC["sources_sha256"] else None)
    if dom is None:
        return {"bound": "hbm", "achieved": round(step_gbps, 1), "peak": HBM_PEAK_GBS, "unit": "GB/s",
                "frac": round(step_gbps / HBM_PEAK_GBS, 4), "traffic": traffic,
                "kernel": "decode calls, average over the sweep"}
    return {"bound": "hbm", "achieved": dom["GBps"], "peak": HBM_PEAK_GBS, "unit": "GB/s",
            "frac": round(dom["GBps"] / HBM_PEAK_GBS, 4), "traffic": traffic,
            "kernel": dom["kernel"], "calls": dom["M"], "us_per_call": dom["us"],
            "algorithmic_bytes_per_call": dom["bytes"],
            "frac_vs_cold_read_4MiB": round(dom["GBps"] / cold, 4),
            "launch_floor_us": floors["empty_kernel_us"]}


if __name__ == "__main__":
    main()
