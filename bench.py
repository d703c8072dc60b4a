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
    ap.add_argument("--steps", type=int, default=None,
                    help="timed steps (default 2000; with --quantizer, timed calls per "
                         "kernel, default 5)")
    ap.add_argument("--warmup", type=int, default=300)
    ap.add_argument("--config", type=int, default=2, choices=[1, 2, 3, 4, 5])
    ap.add_argument("--K", type=int, default=None, help="override the workload's K")
    ap.add_argument("--T", type=int, default=None, help="tokens (workloads 3 and 5)")
    ap.add_argument("--no-graph", action="store_true", help="plain stream launches")
    ap.add_argument("--rotate-bytes", type=float, default=float(2 ** 30))
    ap.add_argument("--cpu-seconds", type=float, default=12.0)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--calibrate-copy", action="store_true",
                    help="after the timed region, one 256 MiB device-to-device copy: the "
                         "kernel of known size that scales the byte counters")
    ap.add_argument("--summarize", nargs=3, metavar=("STATS_DIR", "FETCH_DIR", "WRITE_DIR"),
                    help="no GPU work: turn a rocprofv3 --kernel-trace --stats output and two "
                         "--pmc outputs (FETCH_SIZE, WRITE_SIZE) of this script into the "
                         "profile record of the workload given by --config/--K/--T")
    ap.add_argument("--command", default="", help="with --summarize: the commands that made "
                                                  "the rocprofv3 outputs, for the record")
    ap.add_argument("--quantizer", action="store_true",
                    help="time the setup kernels instead (greedy quantizer, refit, pack) on "
                         "every linear of the workload; prints one JSON line of its own")
    ap.add_argument("--refit-rounds", type=int, default=2)
    ap.add_argument("--svid", action="store_true",
                    help="one token: the SVID scale variant (successive SVID decomposition, "
                         "then y = sum_k s_out^k (.) (B_k (s_in^k (.) x)))")
    ap.add_argument("--svid-iters", type=int, default=32)
    ap.add_argument("--transposed", action="store_true",
                    help="one token: time the transposed product dx = W_hat^T g instead")
    ap.add_argument("--avg-k", type=float, default=None,
                    help="LLaMA-13B-shaped layer only: allocate K per linear (1..4) from the "
                         "residual energies for this average number of kernels per weight")
    ap.add_argument("--library-gemm", action="store_true",
                    help="time the vendor library's plain bf16 GEMM (torch.matmul) at the "
                         "workload's product shape, as a yardstick for the prefill kernel")
    ap.add_argument("--extra", nargs="*", default=[],
                    help="with --summarize: more --pmc output dirs of --calibrate-copy runs; "
                         "every counter in them is reported per dominant call")
    return ap.parse_args()


def weight_bytes(m, n, K, alpha_bytes):
    return K * m * n / 8 + K * m * (n // 128) * alpha_bytes


HERE = os.path.dirname(os.path.abspath(__file__))
CSRC = os.path.join(HERE, "boolean_weight_amd", "csrc")
COPY_BYTES = 2 ** 28  # calibration copy: 256 MiB read and 256 MiB written
CAL_CALLS = 8         # dominant calls bracketed by the two calibration copies


def kernel_family(T):
    """Source file and kernel-name prefix of the kernel one call runs."""
    if T == 1:
        return "gemv.hip", "gemv_"
    if T <= 16:
        return "skinny.hip", "gemm_skinny"
    return "gemm.hip", "gemm_mfma"


def source_digest(T):
    import hashlib
    h = hashlib.sha256()
    for f in (kernel_family(T)[0], "mbok_device.h"):
        with open(os.path.join(CSRC, f), "rb") as fh:
            h.update(fh.read())
    return h.hexdigest()[:16]


def workload_key(config, K, T):
    return f"config{config}_K{K}_T{T}"


def profile_path(config, K, T):
    return os.path.join(HERE, "profiles", f"pmc_traffic_{kernel_family(T)[0][:-4]}_"
                        f"{workload_key(config, K, T)}.txt")


def stored_traffic(config, K, T):
    """HBM bytes per launch from the stored counter record of this workload,
    or None when there is none or the kernel source changed since."""
    path = profile_path(config, K, T)
    if not os.path.exists(path):
        return None
    rec = {}
    with open(path) as fh:
        for line in fh:
            if ":" in line and not line.startswith("#"):
                k, v = line.split(":", 1)
                rec[k.strip()] = v.strip()
    if rec.get("source_sha256") != source_digest(T):
        return None
    try:
        return float(rec["traffic_bytes_per_launch"])
    except (KeyError, ValueError):
        return None


def _csv_rows(d, suffix):
    import csv
    import glob
    rows = []
    for path in glob.glob(os.path.join(d, "**", "*" + suffix), recursive=True):
        with open(path) as fh:
            rows.extend(csv.DictReader(fh))
    return rows


def bracketed(dispatches, prefix):
    """dispatches: [(dispatch id, kernel name, value)].  The run ends with
    [calibration copy][CAL_CALLS calls of the dominant kernel(s)][calibration
    copy]; returns (values of the first copy's dispatches, values of the
    calls' dispatches), or None when the pattern is not there."""
    ds = sorted(dispatches, key=lambda t: t[0])
    is_copy = lambda nm: "copy" in nm.lower()
    j = len(ds)
    while j > 0 and is_copy(ds[j - 1][1]):  # second copy
        j -= 1
    end_calls = j
    while j > 0 and prefix in ds[j - 1][1]:
        j -= 1
    calls = [v for _, _, v in ds[j:end_calls]]
    end_copy = j
    while j > 0 and is_copy(ds[j - 1][1]):  # first copy
        j -= 1
    copy = [v for _, _, v in ds[j:end_copy]]
    if not calls or not copy or end_calls == len(ds):
        return None
    return copy, calls


def summarize(args):
    """Profile record of one workload from rocprofv3 outputs of bench.py."""
    import mbok_synth as syn

    cfg = syn.WORKLOADS[args.config]
    K = args.K or cfg["K"]
    T = args.T or cfg["T"][0]
    _, prefix = kernel_family(T)
    stats_dir, fetch_dir, write_dir = args.summarize
    lines = [f"# rocprofv3 summary, workload {workload_key(args.config, K, T)} "
             f"({cfg['name']})", f"# commands: {args.command}", ""]
    stats = _csv_rows(stats_dir, "kernel_stats.csv")
    lines.append("kernel-trace stats (top kernels by total time):")
    stats.sort(key=lambda r: -float(r.get("TotalDurationNs", 0)))
    for r in stats[:6]:
        lines.append(f"  {r['Name'][:110]} | calls {r['Calls']} | avg {float(r['AverageNs']) / 1e3:.3f} us"
                     f" | min {float(r['MinNs']) / 1e3:.3f} us | max {float(r['MaxNs']) / 1e3:.3f} us")
    trace = _csv_rows(stats_dir, "kernel_trace.csv")
    br = bracketed([(int(r["Dispatch_Id"]), r["Kernel_Name"],
                     float(r["End_Timestamp"]) - float(r["Start_Timestamp"])) for r in trace], prefix)
    if br:
        lines.append(f"dominant_call_kernel_us: {sum(br[1]) / CAL_CALLS / 1e3:.3f} "
                     f"(sum of kernel durations over {CAL_CALLS} bracketed calls / {CAL_CALLS})")
    lines.append("")
    out = {}
    for tag, d, counter, unit_scale in (("fetch", fetch_dir, "FETCH_SIZE", 1.0),
                                        ("write", write_dir, "WRITE_SIZE", 1.0)):
        rows = [r for r in _csv_rows(d, "counter_collection.csv") if r["Counter_Name"] == counter]
        br = bracketed([(int(r["Dispatch_Id"]), r["Kernel_Name"], float(r["Counter_Value"]))
                        for r in rows], prefix)
        if not br:
            lines.append(f"{counter}: calibration pattern not found")
            continue
        copy_kib, call_kib = sum(br[0]), sum(br[1])
        scale = COPY_BYTES / (copy_kib * 1024.0)
        per_call = call_kib * 1024.0 * scale / CAL_CALLS
        out[tag] = per_call
        lines += [f"{counter}_copy_kib: {copy_kib:.1f} over {len(br[0])} dispatches "
                  f"(256 MiB copied)",
                  f"{counter}_scale: {scale:.4f}",
                  f"{counter}_calls_kib: {call_kib:.1f} over {len(br[1])} dispatches",
                  f"{tag}_bytes_per_launch: {per_call:.0f}"]
    if len(out) == 2:
        lines.append(f"traffic_bytes_per_launch: {out['fetch'] + out['write']:.0f}")
    for d in args.extra:
        rows = _csv_rows(d, "counter_collection.csv")
        for counter in sorted({r["Counter_Name"] for r in rows}):
            br = bracketed([(int(r["Dispatch_Id"]), r["Kernel_Name"], float(r["Counter_Value"]))
                            for r in rows if r["Counter_Name"] == counter], prefix)
            if br:
                lines.append(f"{counter}_per_call: {sum(br[1]) / CAL_CALLS:.6g}")
    lines.append(f"source_sha256: {source_digest(T)}")
    print("\n".join(lines))


def main():
    args = parse()
    if args.steps is None:
        args.steps = 5 if args.quantizer else 2000
    if args.summarize:
        summarize(args)
        return
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
        linears = list(syn.LAYER_STREAM_13B)
    if args.config == 3:
        linears = linears[:1] if T == 1 else linears
    if args.svid and (T != 1 or args.transposed or args.avg_k is not None):
        print("--svid runs one token on its own", file=sys.stderr)
        sys.exit(2)
    if args.transposed and T != 1:
        print("--transposed runs one gradient vector (T = 1)", file=sys.stderr)
        sys.exit(2)
    if args.quantizer:
        quantizer_bench(args, cfg, cfg["linears"], K, adt, abytes)
        return
    if args.library_gemm:
        library_gemm_bench(args, cfg, linears, T)
        return

    # weights of each launch: (name, W on the device, K)
    allocation = None
    if args.avg_k is not None:
        if args.config != 4:
            print("--avg-k applies to the LLaMA-13B-shaped layer (--config 4)", file=sys.stderr)
            sys.exit(2)
        Ws = [torch.from_numpy(syn.weight(m, n, syn.weight_seed(4, li))).to(dev)
              for li, (name, m, n) in enumerate(cfg["linears"])]
        Ks, _ = bw.allocate_for_budget(Ws, args.avg_k, kmax=4, alpha_dtype=adt)
        allocation = {nm: k for (nm, _, _), k in zip(cfg["linears"], Ks)}
        names = [nm for nm, _, _ in cfg["linears"]]
        launches = []
        # q|k|v and gate|up share their input: fused when their K agree
        for group in (["q_proj", "k_proj", "v_proj"], ["o_proj"], ["gate_proj", "up_proj"],
                      ["down_proj"]):
            idx = [names.index(g) for g in group]
            if len({Ks[t] for t in idx}) == 1 and len(idx) > 1:
                launches.append(("|".join(group), torch.cat([Ws[t] for t in idx]), Ks[idx[0]]))
            else:
                launches.extend((names[t], Ws[t], Ks[t]) for t in idx)
        del Ws
        K = max(Ks)
    else:
        launches = [(name, None, K) for name, m, n in linears]

    # ---- setup: quantize + pack on the device, build the rotating pool
    layers = []
    svid_in = []  # s_in of each layer (SVID)
    per_step_wbytes = 0.0
    per_step_bytes = 0.0
    per_step_flops = 0.0
    for li, (name, Wl, Kl) in enumerate(launches):
        if Wl is None:
            _, m, n = linears[li]
            Wl = torch.from_numpy(syn.weight(m, n, syn.weight_seed(args.config, li))).to(dev)
        m, n = Wl.shape
        if args.svid:
            d = bw.mbok_desc_init(m, n, Kl, adt)
            at = bw.alpha_torch_dtype(adt)
            signs = torch.empty((Kl, m, n), dtype=torch.int8, device=dev)
            s_out = torch.empty((Kl, m), dtype=at, device=dev)
            s_in = torch.empty((Kl, n), dtype=at, device=dev)
            bw.mbok_svid_decompose(d, Wl, signs, s_out, s_in, args.svid_iters)
            packed = torch.empty(bw.mbok_packed_bytes(d), dtype=torch.uint8, device=dev)
            bw.mbok_svid_pack(d, signs, s_out, packed)
            svid_in.append(s_in)
            del signs, s_out
        else:
            d, packed, signs, alpha = bw.quantize_and_pack(Wl, Kl, adt)
            del signs, alpha
        del Wl
        layers.append((name, d, packed))
        wb = weight_bytes(m, n, Kl, abytes)
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
        if args.transposed:  # gradient g [m] in, dx [n] out
            x = torch.from_numpy(syn.activations(1, d.m, syn.act_seed(args.config, li) + 500,
                                                 cfg["x_dtype"])).to(dev).to(xdt)
            xs.append(x[0].contiguous())
            ys.append(torch.empty((d.n,), dtype=torch.float32, device=dev))
            continue
        x = torch.from_numpy(syn.activations(T, d.n, syn.act_seed(args.config, li),
                                             cfg["x_dtype"])).to(dev).to(xdt)
        xs.append(x if T > 1 else x[0].contiguous())
        ys.append(torch.empty((T, d.m) if T > 1 else (d.m,), dtype=torch.float32, device=dev))

    def call(li, c):
        d = layers[li][1]
        if args.svid:
            bw.mbok_svid_gemv(d, pools[li][c], svid_in[li], xs[li], ys[li])
        elif args.transposed:
            bw.mbok_gemvt(d, pools[li][c], xs[li], ys[li])
        elif T == 1:
            bw.mbok_gemv(d, pools[li][c], xs[li], ys[li])
        else:
            bw.mbok_gemm(d, pools[li][c], xs[li], ys[li])

    def step(i):
        c = i % ncopy
        for li in range(len(layers)):
            call(li, c)

    # A HIP graph of one pass over the whole pool (>= 1 GiB of distinct
    # weights), or of the timed steps when they are fewer: replays stream
    # cold weights and save per-launch CPU work (and the timed region never
    # mixes graph replays with plain launches when steps <= the pool).
    glen = min(ncopy, max(1, args.steps))
    use_graph = not args.no_graph and glen * len(layers) <= 2048
    graph = None
    if use_graph:
        s = torch.cuda.Stream()
        s.wait_stream(torch.cuda.current_stream())
        with torch.cuda.stream(s):
            step(0)
        torch.cuda.current_stream().wait_stream(s)
        torch.cuda.synchronize()
        def capture(count):
            g = torch.cuda.CUDAGraph()
            with torch.cuda.graph(g):
                for i in range(count):
                    step(i)
            g.replay()  # the first replay uploads the graph: keep it untimed
            torch.cuda.synchronize()
            return g

        graph = capture(glen)
        # the steps past the last whole replay (warm-up and timed counts) run
        # as graphs of their own too, captured here, outside the timed region
        rest = {r: capture(r) for r in {args.warmup % glen, args.steps % glen} if r}

    def run(nsteps):
        """Exactly nsteps steps: whole graph replays, then the remainder."""
        i = 0
        if use_graph:
            for _ in range(nsteps // glen):
                graph.replay()
            i = (nsteps // glen) * glen
            if nsteps > i:
                rest[nsteps - i].replay()
                i = nsteps
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

    # ---- mean duration of the dominant call: a HIP graph of that call alone
    # over the pool, replayed back to back and timed with HIP events on the
    # stream that launches it (graph launches leave no gaps between kernels,
    # so this is the kernel time rocprofv3 reports)
    dom = max(range(len(layers)), key=lambda li: layers[li][1].m * layers[li][1].n)
    name, d, _ = layers[dom]

    def dom_call(i):
        call(dom, i % ncopy)

    s2 = torch.cuda.Stream()
    s2.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(s2):
        dom_call(0)
    torch.cuda.current_stream().wait_stream(s2)
    torch.cuda.synchronize()
    nrep = max(1, min(200, 2000 // ncopy))
    if use_graph and ncopy <= 2048:
        g2 = torch.cuda.CUDAGraph()
        with torch.cuda.graph(g2):
            for i in range(ncopy):
                dom_call(i)
        g2.replay()
        torch.cuda.synchronize()
        e0 = torch.cuda.Event(enable_timing=True)
        e1 = torch.cuda.Event(enable_timing=True)
        e0.record(stream)
        for _ in range(nrep):
            g2.replay()
        e1.record(stream)
        torch.cuda.synchronize()
        launch_us = e0.elapsed_time(e1) * 1e3 / (nrep * ncopy)
        del g2
    else:
        e0 = torch.cuda.Event(enable_timing=True)
        e1 = torch.cuda.Event(enable_timing=True)
        e0.record(stream)
        for i in range(ncopy):
            dom_call(i)
        e1.record(stream)
        torch.cuda.synchronize()
        launch_us = e0.elapsed_time(e1) * 1e3 / ncopy
    if args.calibrate_copy:
        # [copy] [CAL_CALLS dominant calls on pool copies read longest ago] [copy]:
        # the profile summary finds this pattern at the end of the dispatch list
        a = torch.empty(COPY_BYTES // 4, dtype=torch.float32, device=dev)
        b = torch.empty_like(a)
        torch.cuda.synchronize()
        b.copy_(a)
        for i in range(CAL_CALLS):
            dom_call(i)
        b.copy_(a)
        torch.cuda.synchronize()
        del a, b
    m, n = d.m, d.n
    if args.svid:  # packed layer, s_in, x in; y out
        alg_bytes = (weight_bytes(m, n, d.K, abytes) + d.K * n * abytes
                     + n * (2 if xdt == torch.bfloat16 else 4) + m * 4)
    elif args.transposed:  # g in, dx out
        alg_bytes = weight_bytes(m, n, d.K, abytes) + m * (2 if xdt == torch.bfloat16 else 4) + n * 4
    else:
        alg_bytes = weight_bytes(m, n, d.K, abytes) + T * n * (2 if xdt == torch.bfloat16 else 4) + T * m * 4
    if T > 16:
        roof = {"bound": "mfma", "achieved": 2.0 * m * n * T / (launch_us * 1e-6) / 1e12,
                "peak": BF16_MFMA_PEAK_TFLOPS, "unit": "TFLOP/s"}
    else:
        roof = {"bound": "hbm", "achieved": alg_bytes / (launch_us * 1e-6) / 1e9,
                "peak": HBM_PEAK_GBPS, "unit": "GB/s"}
    roof["frac"] = roof["achieved"] / roof["peak"]
    roof["traffic"] = (stored_traffic(args.config, K, T)
                       if allocation is None and not args.transposed and not args.svid else None)
    roof["kernel"] = name
    roof["launch_us"] = launch_us
    roof["alg_bytes_per_launch"] = alg_bytes

    if args.svid:
        metric, unit = "svid weight GB/s", "GB/s"
        value = per_step_wbytes / (ms_per_step * 1e-3) / 1e9
    elif args.transposed:
        metric, unit = "transposed weight GB/s", "GB/s"
        value = per_step_wbytes / (ms_per_step * 1e-3) / 1e9
    elif T > 16:
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
                   "K": K if allocation is None else allocation, "group": 128, "T": T,
                   "alpha_dtype": cfg["alpha_dtype"],
                   "x_dtype": cfg["x_dtype"], "rotating_pool_MB": round(ncopy * per_step_wbytes / 2**20),
                   "launch": "hip graph" if use_graph else "stream",
                   "pct_hbm_peak_of_value": round(100 * value / HBM_PEAK_GBPS, 1) if unit == "GB/s" else None,
                   "wall_s": round(wall, 3)},
        "roofline": roof,
    }
    if args.transposed:
        line["config"]["product"] = "dx = W_hat^T g"
    if args.svid:
        line["config"]["product"] = "y = sum_k s_out^k (.) (B_k (s_in^k (.) x)) (successive SVID)"
        line["config"]["svid_iters"] = args.svid_iters
    if not args.no_cpu_baseline:
        dname, dd = layers[dom][0], layers[dom][1]
        line["cpu_baseline"] = cpu_baseline(args, cfg, (dname, dd.m, dd.n), dd.K, T, unit)
    print(json.dumps(line), flush=True)


def quantizer_bench(args, cfg, linears, K, adt, abytes):
    """Mean device time of the setup kernels per linear, from HIP events on
    the launch stream: greedy residual binarization, the alternating refit
    (--refit-rounds) and packing.  Algorithmic bytes: W fp32 read; signs int8
    written (greedy), read and written (refit), read (pack); scales likewise;
    the packed layer written (pack)."""
    import torch

    import boolean_weight_amd as bw
    import mbok_synth as syn

    dev = torch.device("cuda:0")
    stream = torch.cuda.current_stream()
    reps = max(1, args.steps)
    out = []

    def timed(fn):
        fn()
        torch.cuda.synchronize()
        e0 = torch.cuda.Event(enable_timing=True)
        e1 = torch.cuda.Event(enable_timing=True)
        e0.record(stream)
        for _ in range(reps):
            fn()
        e1.record(stream)
        torch.cuda.synchronize()
        return e0.elapsed_time(e1) * 1e3 / reps

    for li, (name, m, n) in enumerate(linears):
        W = torch.from_numpy(syn.weight(m, n, syn.weight_seed(args.config, li))).to(dev)
        d = bw.mbok_desc_init(m, n, K, adt)
        signs = torch.empty((K, m, n), dtype=torch.int8, device=dev)
        alpha = torch.empty((K, m, n // 128), dtype=bw.alpha_torch_dtype(adt), device=dev)
        packed = torch.empty(bw.mbok_packed_bytes(d), dtype=torch.uint8, device=dev)
        s0 = torch.empty_like(signs)
        a0 = torch.empty_like(alpha)
        bw.mbok_residual_binarize(d, W, s0, a0)
        us_greedy = timed(lambda: bw.mbok_residual_binarize(d, W, signs, alpha))

        def refit_once():
            # each timed call starts again from the greedy result (two copies
            # on the same stream, timed apart and subtracted)
            signs.copy_(s0)
            alpha.copy_(a0)
            bw.mbok_refit(d, W, signs, alpha, args.refit_rounds)

        def copies_only():
            signs.copy_(s0)
            alpha.copy_(a0)

        us_refit = timed(refit_once) - timed(copies_only)
        us_pack = timed(lambda: bw.mbok_pack(d, signs, alpha, packed))
        at = bw.alpha_torch_dtype(adt)
        so = torch.empty((K, m), dtype=at, device=dev)
        si = torch.empty((K, n), dtype=at, device=dev)
        svws = torch.empty(bw.mbok_svid_workspace_bytes(d), dtype=torch.uint8, device=dev)
        us_svid = timed(lambda: bw.mbok_svid_decompose(d, W, signs, so, si, args.svid_iters, svws))
        nw = m * n
        na = K * m * (n // 128) * abytes
        b_greedy = 4 * nw + K * nw + na
        b_refit = 4 * nw + 2 * K * nw + 2 * na
        b_pack = K * nw + na + bw.mbok_packed_bytes(d)
        # SVID: per kernel, per power-iteration round two passes over W and the
        # earlier kernels' signs, plus the sign pass
        b_svid = sum((2 * args.svid_iters + 1) * (4 * nw + kk * nw) + nw for kk in range(K))
        for kern, us, b in (("residual_binarize", us_greedy, b_greedy),
                            ("refit", us_refit, b_refit), ("pack", us_pack, b_pack),
                            ("svid_decompose", us_svid, b_svid)):
            out.append({"linear": name, "m": m, "n": n, "kernel": kern, "us": round(us, 2),
                        "alg_bytes": b, "GB/s": round(b / (us * 1e-6) / 1e9, 1),
                        "frac_hbm": round(b / (us * 1e-6) / 1e9 / HBM_PEAK_GBPS, 4)})
        del W, signs, alpha, packed, s0, a0
        torch.cuda.empty_cache()
        print(f"quantizer bench: {name} {m}x{n} done", file=sys.stderr, flush=True)
    print(json.dumps({"metric": "setup kernel time", "unit": "us", "workload": cfg["name"],
                      "K": K, "refit_rounds": args.refit_rounds, "reps": reps,
                      "alpha_dtype": cfg["alpha_dtype"], "kernels": out}), flush=True)


def library_gemm_bench(args, cfg, linears, T):
    """A yardstick, not the product: the vendor library's dense bf16 GEMM
    (torch.matmul, hipBLASLt on ROCm) at the first linear's shape, with
    weights already in bf16 (no unpacking) and a bf16 output.  Both operand
    orders are timed, each as a HIP graph of repeated calls."""
    import torch

    dev = torch.device("cuda:0")
    name, m, n = linears[0]
    X = torch.randn(T, n, device=dev, dtype=torch.bfloat16)
    W = torch.randn(m, n, device=dev, dtype=torch.bfloat16)
    reps = 50
    out = []
    for order, a, b in (("X W^T", X, W.t().contiguous()), ("W X^T", W, X.t().contiguous())):
        C = torch.empty(a.shape[0], b.shape[1], device=dev, dtype=torch.bfloat16)
        side = torch.cuda.Stream()
        side.wait_stream(torch.cuda.current_stream())
        with torch.cuda.stream(side):
            for _ in range(3):
                torch.matmul(a, b, out=C)
        torch.cuda.current_stream().wait_stream(side)
        torch.cuda.synchronize()
        g = torch.cuda.CUDAGraph()
        with torch.cuda.graph(g):
            for _ in range(reps):
                torch.matmul(a, b, out=C)
        g.replay()
        torch.cuda.synchronize()
        e0 = torch.cuda.Event(enable_timing=True)
        e1 = torch.cuda.Event(enable_timing=True)
        e0.record()
        g.replay()
        e1.record()
        torch.cuda.synchronize()
        us = e0.elapsed_time(e1) * 1e3 / reps
        tf = 2.0 * T * n * m / (us * 1e-6) / 1e12
        out.append({"order": order, "us": round(us, 1), "TFLOP/s": round(tf, 1),
                    "frac_bf16_peak": round(tf / BF16_MFMA_PEAK_TFLOPS, 4)})
        del C, g
    print(json.dumps({"metric": "library bf16 GEMM TFLOP/s", "kind": "comparison",
                      "library": "torch.matmul (hipBLASLt), bf16 in and out, weights pre-unpacked",
                      "workload": cfg["name"], "linear": [name, m, n], "T": T, "runs": out}),
          flush=True)


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
        Gr = syn.activations(1, rows, syn.act_seed(args.config, 0) + 500, cfg["x_dtype"])[0]
        t0 = time.perf_counter()
        reps = 0
        while True:
            if args.svid:
                oracle.svid_product(S, A[:, :, 0], np.ones((K, n)), X[0])
            elif args.transposed:
                oracle.product_transposed(S, A, Gr)
            else:
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
            "sample": f"{reps} oracle {'transposed ' if args.transposed else ''}products "
                      f"(fp64 dequantize + matmul) of {name} "
                      f"rows 0..{rows - 1} x {n}, K={K}, T={T}, in {dt:.1f} s"}


if __name__ == "__main__":
    main()
