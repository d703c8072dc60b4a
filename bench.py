"""Throughput of the MBOK linear layer on one MI355X.

    python bench.py [--gpus 1] [--steps K] [--warmup W] [--config 2]

A step is one pass of the hot path over one batch of synthetic input: for the
default workload (LLaMA-7B attention projection 4096x4096, K=2 Boolean
kernels, group 128, fp16 scales, bf16 activations, one token) that is one
decode product y = sum_k (alpha_k (.) B_k) x.  The packed layer (signs and
scales) is quantized and packed on the device by the library beforehand
(untimed setup), then copied into a rotating pool of at least 1 GiB so that
every step streams cold weights from HBM rather than from the 256 MB
Infinity Cache.  Inputs are resident in HBM when the timed region starts.

Printed: one JSON line with the metric (weight GB/s), the roofline of the
dominant kernel (algorithmic bytes per launch / mean launch duration from HIP
events on the launch stream, against the 8 TB/s HBM peak) and the CPU oracle
timed on the host cores on a bounded sample of the same workload.
"""
from __future__ import annotations

import argparse
import json
import os
import sys
import time

import numpy as np

HBM_PEAK_GBPS = 8000.0
BF16_MFMA_PEAK_TFLOPS = 2500.0


def parse():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=2000)
    ap.add_argument("--warmup", type=int, default=300)
    ap.add_argument("--config", type=int, default=2, choices=[1, 2, 3, 4, 5])
    ap.add_argument("--K", type=int, default=None, help="override the workload's K")
    ap.add_argument("--T", type=int, default=None, help="tokens (workloads 3 and 5)")
    ap.add_argument("--no-graph", action="store_true", help="plain stream launches")
    ap.add_argument("--rotate-bytes", type=float, default=float(2 ** 30))
    ap.add_argument("--cpu-seconds", type=float, default=12.0)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    return ap.parse_args()


def weight_bytes(m, n, K, alpha_bytes):
    return K * m * n / 8 + K * m * (n // 128) * alpha_bytes


def main():
    args = parse()
    if args.gpus != 1:
        print(f"bench.py runs on one GPU only (asked for --gpus {args.gpus}); the layer "
              "is measured on one GPU's shard at its full shape.", file=sys.stderr)
        sys.exit(2)

    import torch

    import boolean_weight_amd as bw
    import mbok_synth as syn

    if not torch.cuda.is_available():
        print("no GPU visible", file=sys.stderr)
        sys.exit(1)
    bw.load_library()
    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)

    cfg = syn.WORKLOADS[args.config]
    K = args.K or cfg["K"]
    adt = bw.MBOK_F16 if cfg["alpha_dtype"] == "f16" else bw.MBOK_F32
    abytes = 2 if cfg["alpha_dtype"] == "f16" else 4
    xdt = torch.bfloat16 if cfg["x_dtype"] == "bf16" else torch.float32
    T = args.T or cfg["T"][0]
    linears = cfg["linears"]
    if args.config == 4:
        # q|k|v and gate|up share their input: one fused launch each
        linears = [("qkv_proj", 3 * 5120, 5120), ("o_proj", 5120, 5120),
                   ("gate_up_proj", 2 * 13824, 5120), ("down_proj", 5120, 13824)]
    if args.config == 3:
        linears = linears[:1] if T == 1 else linears

    # ---- setup: quantize + pack on the device, build the rotating pool
    layers = []
    per_step_wbytes = 0.0
    per_step_bytes = 0.0
    per_step_flops = 0.0
    for li, (name, m, n) in enumerate(linears):
        W = torch.from_numpy(syn.weight(m, n, syn.weight_seed(args.config, li))).to(dev)
        d, packed, signs, alpha = bw.quantize_and_pack(W, K, adt)
        del W, signs, alpha
        layers.append((name, d, packed))
        wb = weight_bytes(m, n, K, abytes)
        per_step_wbytes += wb
        per_step_bytes += wb + T * n * (2 if xdt == torch.bfloat16 else 4) + T * m * 4
        per_step_flops += 2.0 * m * n * T
    torch.cuda.empty_cache()
    ncopy = max(2, int(np.ceil(args.rotate_bytes / per_step_wbytes)))
    pools = []
    for name, d, packed in layers:
        pools.append(packed.repeat(ncopy).view(ncopy, -1))
        del packed
    torch.cuda.empty_cache()
    xs, ys = [], []
    for li, (name, d, _) in enumerate(layers):
        x = torch.from_numpy(syn.activations(T, d.n, syn.act_seed(args.config, li),
                                             cfg["x_dtype"])).to(dev).to(xdt)
        xs.append(x if T > 1 else x[0].contiguous())
        ys.append(torch.empty((T, d.m) if T > 1 else (d.m,), dtype=torch.float32, device=dev))

    def step(i):
        c = i % ncopy
        for li, (name, d, _) in enumerate(layers):
            if T == 1:
                bw.mbok_gemv(d, pools[li][c], xs[li], ys[li])
            else:
                bw.mbok_gemm(d, pools[li][c], xs[li], ys[li])

    # A HIP graph of one pass over the whole pool (>= 1 GiB of distinct
    # weights): replays stream cold weights and save per-launch CPU work.
    use_graph = not args.no_graph and ncopy * len(layers) <= 2048
    graph = None
    if use_graph:
        s = torch.cuda.Stream()
        s.wait_stream(torch.cuda.current_stream())
        with torch.cuda.stream(s):
            step(0)
        torch.cuda.current_stream().wait_stream(s)
        torch.cuda.synchronize()
        graph = torch.cuda.CUDAGraph()
        with torch.cuda.graph(graph):
            for i in range(ncopy):
                step(i)

    def run(nsteps):
        """Exactly nsteps steps: whole graph replays, then single launches."""
        i = 0
        if use_graph:
            for _ in range(nsteps // ncopy):
                graph.replay()
            i = (nsteps // ncopy) * ncopy
        while i < nsteps:
            step(i)
            i += 1
        return nsteps

    # ---- warmup, then the timed region
    run(args.warmup)
    torch.cuda.synchronize()
    stream = torch.cuda.current_stream()
    t0 = torch.cuda.Event(enable_timing=True)
    t1 = torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    wall0 = time.perf_counter()
    t0.record(stream)
    done = run(args.steps)
    t1.record(stream)
    torch.cuda.synchronize()
    wall = time.perf_counter() - wall0
    ms = t0.elapsed_time(t1)
    ms_per_step = ms / done

    # ---- per-launch durations of the dominant kernel (HIP events on the
    # launch stream, one pair per launch, plain stream launches)
    dom = max(range(len(layers)), key=lambda li: layers[li][1].m * layers[li][1].n)
    name, d, _ = layers[dom]
    nk = min(400, ncopy * 2)
    evs = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
           for _ in range(nk)]
    for i in range(nk):
        c = i % ncopy
        evs[i][0].record(stream)
        if T == 1:
            bw.mbok_gemv(d, pools[dom][c], xs[dom], ys[dom])
        else:
            bw.mbok_gemm(d, pools[dom][c], xs[dom], ys[dom])
        evs[i][1].record(stream)
    torch.cuda.synchronize()
    launch_us = float(np.mean([a.elapsed_time(b) for a, b in evs[nk // 4:]]) * 1e3)
    m, n = d.m, d.n
    alg_bytes = weight_bytes(m, n, K, abytes) + T * n * (2 if xdt == torch.bfloat16 else 4) + T * m * 4
    if T > 16:
        roof = {"bound": "mfma", "achieved": 2.0 * m * n * T / (launch_us * 1e-6) / 1e12,
                "peak": BF16_MFMA_PEAK_TFLOPS, "unit": "TFLOP/s"}
    else:
        roof = {"bound": "hbm", "achieved": alg_bytes / (launch_us * 1e-6) / 1e9,
                "peak": HBM_PEAK_GBPS, "unit": "GB/s"}
    roof["frac"] = roof["achieved"] / roof["peak"]
    roof["traffic"] = None
    roof["kernel"] = name
    roof["launch_us"] = launch_us

    if T > 16:
        metric, unit = "prefill TFLOP/s", "TFLOP/s"
        value = per_step_flops / (ms_per_step * 1e-3) / 1e12
    else:
        metric, unit = "weight GB/s", "GB/s"
        value = per_step_wbytes / (ms_per_step * 1e-3) / 1e9

    line = {
        "metric": metric, "value": value, "unit": unit, "n_gpus": 1, "steps": done,
        "warmup": args.warmup, "ms_per_step": ms_per_step, "higher_is_better": True,
        "scaling": "weak", "vs_baseline": None, "dtype": "f32",
        "data": "synthetic (seeded N(0,0.02) weights via greedy residual binarization, N(0,1) activations)",
        "config": {"workload": cfg["name"], "linears": [[nm, dd.m, dd.n] for nm, dd, _ in layers],
                   "K": K, "group": 128, "T": T, "alpha_dtype": cfg["alpha_dtype"],
                   "x_dtype": cfg["x_dtype"], "rotating_pool_MB": round(ncopy * per_step_wbytes / 2**20),
                   "launch": "hip graph" if use_graph else "stream",
                   "pct_hbm_peak_of_value": round(100 * value / HBM_PEAK_GBPS, 1) if unit == "GB/s" else None,
                   "wall_s": round(wall, 3)},
        "roofline": roof,
    }
    if not args.no_cpu_baseline:
        line["cpu_baseline"] = cpu_baseline(args, cfg, linears[dom], K, T, unit)
    print(json.dumps(line), flush=True)


def cpu_baseline(args, cfg, lin, K, T, unit):
    """The oracle as it stands (float64 NumPy) on the host cores, on a bounded
    sample of the same workload: repeated products of the dominant layer."""
    import threadpoolctl

    import mbok_synth as syn
    import oracle

    name, m, n = lin
    cores = len(os.sched_getaffinity(0))
    with threadpoolctl.threadpool_limits(cores):
        W = syn.weight(m, n, syn.weight_seed(args.config, 0))
        rows = m if T == 1 else min(m, 512)
        S, A, _ = oracle.residual_binarize(W[:rows], K, alpha_dtype=cfg["alpha_dtype"])
        X = syn.activations(T, n, syn.act_seed(args.config, 0), cfg["x_dtype"])
        t0 = time.perf_counter()
        reps = 0
        while True:
            oracle.product(S, A, X if T > 1 else X[0])
            reps += 1
            if time.perf_counter() - t0 > args.cpu_seconds:
                break
        dt = time.perf_counter() - t0
    wbytes = weight_bytes(rows, n, K, 2 if cfg["alpha_dtype"] == "f16" else 4)
    if unit == "GB/s":
        value = wbytes * reps / dt / 1e9
    else:
        value = 2.0 * rows * n * T * reps / dt / 1e12
    return {"value": value, "unit": unit, "cores": cores, "kind": "oracle",
            "sample": f"{reps} oracle products (fp64 dequantize + matmul) of {name} "
                      f"rows 0..{rows - 1} x {n}, K={K}, T={T}, in {dt:.1f} s"}


if __name__ == "__main__":
    main()
