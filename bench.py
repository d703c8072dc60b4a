"""Throughput of the MBOK linear layer on one MI355X.

    python bench.py [--gpus 1] [--steps K] [--warmup W] [--config 2]

A step is one pass of the hot path over one batch of synthetic input.  For
the default workload (LLaMA-7B attention projection 4096x4096, K=2 Boolean
kernels, group 128, fp16 scales, bf16 activations, one token) that is one
decode product y = sum_k (alpha_k (.) B_k) x.  The packed layer (signs and
scales) is quantized and packed on the device by the library beforehand
(untimed setup) and copied into a rotating pool of at least 1 GiB.  The
timed steps read pool copies that the graph upload and the warm-up did not
touch, and the rest of the pool is read in between, so every timed step
streams its weights from HBM, not from the 256 MB Infinity Cache.  Inputs are
resident in HBM when the timed region starts.

Printed: one JSON line with the metric (weight GB/s of the decode product),
tokens/s, the roofline of the dominant kernel (algorithmic bytes per launch
over its mean launch duration from HIP events on the launch stream, against
the 8 TB/s HBM nameplate and against the read ceiling this part measures),
the CPU oracle timed on the host cores on a bounded sample of the same
workload, and the same figures for the prefill product (11008x4096, K=3,
2048 tokens: TFLOP/s against the bf16 matrix-core nameplate and the measured
matrix-core rate), for the LLaMA-7B MLP decode shapes, and for the whole MLP
step (gate, up, down) at 4 and 16 tokens.
"""
from __future__ import annotations

import argparse
import json
import os
import statistics
import sys
import time

import numpy as np

HBM_PEAK_GBPS = 8000.0
BF16_MFMA_PEAK_TFLOPS = 2500.0


def parse(argv=None):
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=None,
                    help="timed steps (default 2000; with --quantizer, timed calls per "
                         "kernel, default 5)")
    ap.add_argument("--warmup", type=int, default=300)
    ap.add_argument("--config", type=int, default=None, choices=[1, 2, 3, 4, 5],
                    help="workload (default 2, with the prefill and LLaMA-7B MLP decode "
                         "figures added to the line)")
    ap.add_argument("--K", type=int, default=None, help="override the workload's K")
    ap.add_argument("--T", type=int, default=None, help="tokens (workloads 3 and 5)")
    ap.add_argument("--no-graph", action="store_true",
                    help="plain stream launches for the timed steps (the default when the "
                         "timed region holds at most 64 launches)")
    ap.add_argument("--graph", action="store_true",
                    help="a HIP graph of the timed steps whatever their count")
    ap.add_argument("--precise", action="store_true",
                    help="multi-token products through mbok_gemm_precise (two-term levels)")
    ap.add_argument("--rotate-bytes", type=float, default=float(2 ** 30))
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-extra", action="store_true",
                    help="default workload only: leave out the prefill and MLP decode figures")
    ap.add_argument("--calibrate-copy", action="store_true",
                    help="after the timed region, one 256 MiB device-to-device copy, "
                         "CAL_CALLS cold calls of the dominant kernel, and another copy: the "
                         "bracket that scales the byte counters")
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
    ap.add_argument("--ceilings", action="store_true",
                    help="only the part's own ceilings: launch floor, read stream by size, "
                         "matrix-core rates; prints one JSON line of its own")
    ap.add_argument("--extra", nargs="*", default=[],
                    help="with --summarize: more --pmc output dirs of --calibrate-copy runs; "
                         "every counter in them is reported per dominant call")
    args = ap.parse_args(argv)
    args.default_line = args.config is None
    if args.config is None:
        args.config = 2
    return args


def weight_bytes(m, n, K, alpha_bytes):
    return K * m * n / 8 + K * m * (n // 128) * alpha_bytes


HERE = os.path.dirname(os.path.abspath(__file__))
CSRC = os.path.join(HERE, "boolean_weight_amd", "csrc")
COPY_BYTES = 2 ** 28  # calibration copy: 256 MiB read and 256 MiB written
CAL_CALLS = 8         # dominant calls bracketed by the two calibration copies
MARKER = "region_marker_kernel"  # the ceilings library's marker brackets each timed region


def kernel_family(T, m=None, n=None, K=None, x_bf16=True):
    """Source file and kernel-name prefix of the kernel one call runs (the
    library's default choice)."""
    if T == 1:
        # the library's default choice (use_f4_for_gemv in csrc/gemv.hip)
        if x_bf16 and m is not None and (K * n >= 8192 or K * m * n >= (1 << 25) or K >= 4):
            return "gemv_f4.hip", "gemv_f4_kernel"
        return "gemv.hip", "gemv_stream_kernel"
    # the few-token choice (token_kernel in csrc/gemm.hip)
    v = os.environ.get("MBOK_SKINNY_VARIANT", "")
    if (T == 2 and v == "") or (T <= 4 and v == "f4"):
        return "gemv_f4.hip", "gemm_f4_kernel"
    big = m is not None and K * m * n >= (1 << 26)
    if (3 <= T <= 6 and v == "" and big) or (T <= 16 and v == "f4g"):
        return "gemv_f4.hip", "gemm_f4g_kernel"
    if T <= 16:
        return "skinny.hip", "gemm_skinny"
    return "gemm.hip", "gemm_mfma"


def code_text(src: str) -> str:
    """C++ source without comments and with whitespace collapsed, so that a
    comment edit leaves the digest of a kernel's code unchanged."""
    import re
    out, i, n = [], 0, len(src)
    while i < n:
        if src.startswith("//", i):
            j = src.find("\n", i)
            i = n if j < 0 else j
        elif src.startswith("/*", i):
            j = src.find("*/", i + 2)
            i = n if j < 0 else j + 2
            out.append(" ")
        elif src[i] in "\"'":
            q, j = src[i], i + 1
            while j < n and src[j] != q:
                j += 2 if src[j] == "\\" else 1
            out.append(src[i:j + 1])
            i = j + 1
        else:
            out.append(src[i])
            i += 1
    return re.sub(r"\s+", " ", "".join(out)).strip()


def source_digest(T, m=None, n=None, K=None):
    """Digest of the code (comments and layout aside) of the kernel source one
    call runs and of the shared device header."""
    import hashlib
    h = hashlib.sha256()
    for f in (kernel_family(T, m, n, K)[0], "mbok_device.h"):
        with open(os.path.join(CSRC, f), encoding="utf-8") as fh:
            h.update(code_text(fh.read()).encode())
    return h.hexdigest()[:16]


def workload_key(config, K, T):
    return f"config{config}_K{K}_T{T}"


def dominant_shape(config, K, T):
    """(m, n) of the workload's dominant launch."""
    import mbok_synth as syn
    if config == 4:
        return max(((m, n) for _, m, n in syn.LAYER_STREAM_13B), key=lambda s: s[0] * s[1])
    _, m, n = syn.WORKLOADS[config]["linears"][0]
    return m, n


def profile_path(config, K, T):
    m, n = dominant_shape(config, K, T)
    return os.path.join(HERE, "profiles", f"pmc_traffic_{kernel_family(T, m, n, K)[0][:-4]}_"
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
    m, n = dominant_shape(config, K, T)
    if rec.get("source_sha256") != source_digest(T, m, n, K):
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


def timed_regions(dispatches):
    """dispatches: [(dispatch id, kernel name, duration ns)].  Every timed
    region of the run is bracketed by two marker kernels; returns, per region
    in order, {kernel name: [durations]} of the dispatches between them."""
    ds = sorted(dispatches, key=lambda t: t[0])
    marks = [i for i, (_, nm, _) in enumerate(ds) if MARKER in nm]
    regions = []
    for a, b in zip(marks[0::2], marks[1::2]):
        reg = {}
        for _, nm, dur in ds[a + 1:b]:
            reg.setdefault(nm, []).append(dur)
        regions.append(reg)
    return regions


def summarize(args):
    """Profile record of one workload from rocprofv3 outputs of bench.py."""
    import mbok_synth as syn

    cfg = syn.WORKLOADS[args.config]
    K = args.K or cfg["K"]
    T = args.T or cfg["T"][0]
    m, n = dominant_shape(args.config, K, T)
    _, prefix = kernel_family(T, m, n, K)
    stats_dir, fetch_dir, write_dir = args.summarize
    lines = [f"# rocprofv3 summary, workload {workload_key(args.config, K, T)} "
             f"({cfg['name']}; dominant launch {m}x{n})", f"# commands: {args.command}", ""]
    trace = _csv_rows(stats_dir, "kernel_trace.csv")
    disp = [(int(r["Dispatch_Id"]), r["Kernel_Name"],
             float(r["End_Timestamp"]) - float(r["Start_Timestamp"])) for r in trace]
    regions = timed_regions(disp)
    if regions:
        lines.append("kernel-trace over the first timed region only (between the marker kernels):")
        for nm, durs in sorted(regions[0].items(), key=lambda kv: -sum(kv[1])):
            lines.append(f"  {nm[:110]} | calls {len(durs)} | avg {sum(durs) / len(durs) / 1e3:.3f} us"
                         f" | min {min(durs) / 1e3:.3f} us | max {max(durs) / 1e3:.3f} us")
        dom = [d for nm, ds_ in regions[0].items() if prefix in nm for d in ds_]
        if dom:
            lines.append(f"timed_region_dominant_kernel_us: {sum(dom) / len(dom) / 1e3:.3f} "
                         f"(mean over {len(dom)} dispatches in the timed region)")
    else:
        lines.append("timed region markers not found")
    stats = _csv_rows(stats_dir, "kernel_stats.csv")
    lines.append("kernel-trace stats over the whole run (setup and profiling calls included):")
    stats.sort(key=lambda r: -float(r.get("TotalDurationNs", 0)))
    for r in stats[:6]:
        lines.append(f"  {r['Name'][:110]} | calls {r['Calls']} | avg {float(r['AverageNs']) / 1e3:.3f} us"
                     f" | min {float(r['MinNs']) / 1e3:.3f} us | max {float(r['MaxNs']) / 1e3:.3f} us")
    br = bracketed(disp, prefix)
    if br:
        lines.append(f"dominant_call_kernel_us: {sum(br[1]) / CAL_CALLS / 1e3:.3f} "
                     f"(sum of kernel durations over {CAL_CALLS} bracketed cold calls / {CAL_CALLS})")
    lines.append("")
    out = {}
    for tag, d, counter in (("fetch", fetch_dir, "FETCH_SIZE"), ("write", write_dir, "WRITE_SIZE")):
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
                per_call = sum(br[1]) / CAL_CALLS
                lines.append(f"{counter}_per_call: {per_call:.6g}")
                if counter in ("SQ_INSTS_VALU", "SQ_INSTS_LDS", "SQ_INSTS_MFMA"):
                    # wavefront instructions x 64 lanes over the call's sign bits
                    lines.append(f"{counter}_lane_ops_per_sign_bit: "
                                 f"{per_call * 64 / (K * m * n):.4g}")
    lines.append(f"source_sha256: {source_digest(T, m, n, K)}")
    print("\n".join(lines))


# ------------------------------------------------------------------ GPU side

class Workload:
    """The launches of one workload: packed layers (quantized and packed on
    the device), a rotating pool of copies of them, inputs and outputs."""

    def __init__(self, args, config, K=None, T=None, launches=None):
        import torch

        import boolean_weight_amd as bw
        import mbok_synth as syn

        self.bw = bw
        dev = torch.device("cuda:0")
        cfg = syn.WORKLOADS[config]
        self.config, self.cfg = config, cfg
        self.K = K or cfg["K"]
        self.T = T or cfg["T"][0]
        self.adt = bw.MBOK_F16 if cfg["alpha_dtype"] == "f16" else bw.MBOK_F32
        self.abytes = 2 if cfg["alpha_dtype"] == "f16" else 4
        self.xdt = torch.bfloat16 if cfg["x_dtype"] == "bf16" else torch.float32
        self.xbytes = 2 if cfg["x_dtype"] == "bf16" else 4
        self.svid, self.transposed = args.svid, args.transposed
        self.precise = getattr(args, "precise", False)
        self.allocation = None
        if launches is None:
            linears = cfg["linears"]
            if config == 4:
                # q|k|v and gate|up share their input: one fused launch each
                linears = list(syn.LAYER_STREAM_13B)
            if config == 3 and self.T == 1:
                linears = linears[:1]
            launches = [(name, None, self.K, m, n) for name, m, n in linears]
        layers, svid_in = [], []
        for li, (name, Wl, Kl, m, n) in enumerate(launches):
            if Wl is None:
                Wl = torch.from_numpy(syn.weight(m, n, syn.weight_seed(config, li))).to(dev)
            if self.svid:
                d = bw.mbok_desc_init(m, n, Kl, self.adt)
                at = bw.alpha_torch_dtype(self.adt)
                signs = torch.empty((Kl, m, n), dtype=torch.int8, device=dev)
                s_out = torch.empty((Kl, m), dtype=at, device=dev)
                s_in = torch.empty((Kl, n), dtype=at, device=dev)
                bw.mbok_svid_decompose(d, Wl, signs, s_out, s_in, args.svid_iters)
                packed = torch.empty(bw.mbok_packed_bytes(d), dtype=torch.uint8, device=dev)
                bw.mbok_svid_pack(d, signs, s_out, packed)
                svid_in.append(s_in)
                del signs, s_out
            else:
                d, packed, signs, alpha = bw.quantize_and_pack(Wl, Kl, self.adt)
                del signs, alpha
            del Wl
            layers.append((name, d, packed))
        self.svid_in = svid_in
        self.wbytes = sum(weight_bytes(d.m, d.n, d.K, self.abytes) for _, d, _ in layers)
        self.flops = sum(2.0 * d.m * d.n * self.T for _, d, _ in layers)
        torch.cuda.empty_cache()
        self.ncopy = max(2, int(np.ceil(args.rotate_bytes / self.wbytes)))
        self.pools = [packed.repeat(self.ncopy).view(self.ncopy, -1) for _, _, packed in layers]
        self.layers = [(name, d) for name, d, _ in layers]
        del layers
        torch.cuda.empty_cache()
        self.xs, self.ys = [], []
        for li, (name, d) in enumerate(self.layers):
            if self.transposed:  # gradient g [m] in, dx [n] out
                g = syn.activations(1, d.m, syn.act_seed(config, li) + 500, cfg["x_dtype"])
                self.xs.append(torch.from_numpy(g).to(dev).to(self.xdt)[0].contiguous())
                self.ys.append(torch.empty((d.n,), dtype=torch.float32, device=dev))
                continue
            x = torch.from_numpy(syn.activations(self.T, d.n, syn.act_seed(config, li),
                                                 cfg["x_dtype"])).to(dev).to(self.xdt)
            self.xs.append(x if self.T > 1 else x[0].contiguous())
            self.ys.append(torch.empty((self.T, d.m) if self.T > 1 else (d.m,),
                                       dtype=torch.float32, device=dev))
        self.dom = max(range(len(self.layers)),
                       key=lambda li: self.layers[li][1].m * self.layers[li][1].n)

    def call(self, li, c):
        bw = self.bw
        d = self.layers[li][1]
        if self.svid:
            bw.mbok_svid_gemv(d, self.pools[li][c], self.svid_in[li], self.xs[li], self.ys[li])
        elif self.transposed:
            bw.mbok_gemvt(d, self.pools[li][c], self.xs[li], self.ys[li])
        elif self.T == 1:
            bw.mbok_gemv(d, self.pools[li][c], self.xs[li], self.ys[li])
        elif self.precise:
            bw.mbok_gemm_precise(d, self.pools[li][c], self.xs[li], self.ys[li])
        else:
            bw.mbok_gemm(d, self.pools[li][c], self.xs[li], self.ys[li])

    def step(self, c):
        for li in range(len(self.layers)):
            self.call(li, c % self.ncopy)

    def dom_alg_bytes(self):
        d = self.layers[self.dom][1]
        wb = weight_bytes(d.m, d.n, d.K, self.abytes)
        if self.svid:
            return wb + d.K * d.n * self.abytes + d.n * self.xbytes + d.m * 4
        if self.transposed:
            return wb + d.m * self.xbytes + d.n * 4
        return wb + self.T * d.n * self.xbytes + self.T * d.m * 4


def _capture(torch, fn):
    """Warm fn up on a side stream, record it into a HIP graph, and replay it
    once (the first replay uploads the graph)."""
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(s):
        fn()
    torch.cuda.current_stream().wait_stream(s)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        fn()
    g.replay()
    torch.cuda.synchronize()
    return g


def _marker(spin_us=0):
    """The ceilings library's empty kernel, enqueued just outside each timed
    region so that a kernel trace can find the region's dispatches; with
    spin_us, a spin kernel first keeps the stream busy while the host
    enqueues the region (so the start event fires with the region's work
    already queued behind it: host submission latency is not timed)."""
    import torch

    from boolean_weight_amd import ceilings
    lib = ceilings.load()
    st = torch.cuda.current_stream().cuda_stream
    if spin_us:
        out = torch.empty(1, dtype=torch.float32, device="cuda")
        if lib.mbok_ceiling_spin(spin_us, out.data_ptr(), st) != 0:
            raise RuntimeError("spin kernel failed")
    if lib.mbok_ceiling_marker(st) != 0:
        raise RuntimeError("marker kernel failed")


def _evict(wl, copies):
    """Read the given pool copies of every layer with the read-stream
    kernel, so that the timed copies leave the Infinity Cache."""
    import torch

    from boolean_weight_amd import ceilings
    lib = ceilings.load()
    out = torch.empty(1024, dtype=torch.float32, device="cuda")
    for c in copies:
        for pool in wl.pools:
            nb = pool[c].numel() // 16 * 16
            if lib.mbok_ceiling_read(pool[c].data_ptr(), nb, out.data_ptr(), 1024, 256,
                                     torch.cuda.current_stream().cuda_stream) != 0:
                raise RuntimeError("eviction read failed")


# A HIP graph replay costs ~10 us before its first kernel starts; over a
# short timed region (the 20 single-launch decode steps of a quick run: 4.07
# against 3.77 us per step measured) that is a tenth of the region.  Up to
# this many launches the timed decode and few-token steps are plain stream
# launches, all enqueued while a spin kernel holds the stream, so they too run
# back to back.  Prefill steps stay in a graph: as plain launches each 90 MB
# fp32 output costs more at the kernel boundary (210 against 196 us per step).
GRAPH_MIN_LAUNCHES = 64
SPIN_US_PER_LAUNCH = 30  # host enqueue time per launch that the spin covers


def timed_with_graph(args, launches, T):
    if args.graph:
        return True
    if args.no_graph:
        return False
    return T > 16 or launches > GRAPH_MIN_LAUNCHES


def measure_steps(wl, steps, warmup, use_graph=True):
    """Exactly `steps` steps in the timed region.  The timed steps use pool
    copies 0 .. glen-1 (glen = min(steps, pool copies)).  The other copies
    are read once after the graph upload, then the warm-up steps run on them,
    so each timed copy was last read at least (pool - glen) copies of other
    data earlier (every copy of the pool, cycled, when steps >= pool).
    Without a graph the steps are enqueued behind a spin kernel long enough
    to cover their host-side launch time.
    Returns ms per step, the wall time and the pool bookkeeping."""
    import torch
    glen = min(wl.ncopy, max(1, steps))
    use_graph = use_graph and glen * len(wl.layers) <= 4096
    graphs = {}
    if use_graph:
        graphs[glen] = _capture(torch, lambda: [wl.step(i) for i in range(glen)])
        rem = steps % glen
        if rem:
            graphs[rem] = _capture(torch, lambda: [wl.step(i) for i in range(rem)])
    read_before = 0
    if glen < wl.ncopy:
        _evict(wl, range(glen, wl.ncopy))
        read_before = (wl.ncopy - glen) * wl.wbytes
    # the warm-up right before the region, on copies the region does not read
    others = list(range(glen, wl.ncopy)) or list(range(wl.ncopy))
    for i in range(warmup):
        wl.step(others[i % len(others)])
    torch.cuda.synchronize()
    stream = torch.cuda.current_stream()
    t0 = torch.cuda.Event(enable_timing=True)
    t1 = torch.cuda.Event(enable_timing=True)
    _marker(spin_us=300 if use_graph else 300 + SPIN_US_PER_LAUNCH * steps * len(wl.layers))
    wall0 = time.perf_counter()
    t0.record(stream)
    if use_graph:
        for _ in range(steps // glen):
            graphs[glen].replay()
        if steps % glen:
            graphs[steps % glen].replay()
    else:
        for i in range(steps):
            wl.step(i % glen)
    t1.record(stream)
    _marker()
    torch.cuda.synchronize()
    wall = time.perf_counter() - wall0  # includes the spin kernel
    return {"ms_per_step": t0.elapsed_time(t1) / steps, "wall_s": wall, "graph": use_graph,
            "pool_copies": wl.ncopy, "timed_copies": glen,
            "timed_pool_MB": round(glen * wl.wbytes / 2 ** 20, 1),
            "read_before_timing_MB": round(read_before / 2 ** 20)}


def measure_dominant(wl, calibrate=False):
    """Mean duration of the dominant call: a HIP graph of that call over the
    whole pool, replayed back to back, timed with HIP events on the launching
    stream (graph launches leave no gaps between kernels, so this is the
    kernel time a trace reports)."""
    import torch
    ncopy = wl.ncopy
    g = _capture(torch, lambda: [wl.call(wl.dom, i) for i in range(ncopy)])
    nrep = max(1, min(50, 2000 // ncopy))
    e0 = torch.cuda.Event(enable_timing=True)
    e1 = torch.cuda.Event(enable_timing=True)
    e0.record()
    for _ in range(nrep):
        g.replay()
    e1.record()
    torch.cuda.synchronize()
    launch_us = e0.elapsed_time(e1) * 1e3 / (nrep * ncopy)
    del g
    if calibrate:
        # [copy] [CAL_CALLS dominant calls on pool copies read longest ago] [copy]:
        # the profile summary finds this pattern at the end of the dispatch list
        a = torch.empty(COPY_BYTES // 4, dtype=torch.float32, device="cuda")
        b = torch.empty_like(a)
        torch.cuda.synchronize()
        b.copy_(a)
        for i in range(CAL_CALLS):
            wl.call(wl.dom, i % ncopy)
        b.copy_(a)
        torch.cuda.synchronize()
        del a, b
    return launch_us


def measure_ceilings(read_sizes):
    """The part's own ceilings: launch floor, nontemporal read stream at the
    given sizes (bytes, each over a rotating pool of at least 1 GiB) and the
    bf16 matrix-core rate."""
    from boolean_weight_amd import ceilings
    out = {"launch_floor_us": round(ceilings.launch_floor_us(256, 512), 3), "read": {}}
    for nb in read_sizes:
        r = ceilings.read_bandwidth(int(nb), grid=1024, block=256)
        out["read"][str(int(nb) // 16 * 16)] = {"us": round(r["us"], 3),
                                                 "GB/s": round(r["GB/s"], 1)}
    r = ceilings.mfma_rate(ceilings.MFMA_BF16, iters=2000, grid=1024, block=256)
    out["mfma_bf16_TFLOP/s"] = round(r["TFLOP/s"], 1)
    return out


# --------------------------------------------------------------- CPU oracle

def _cpu_facts():
    model = "unknown"
    try:
        with open("/proc/cpuinfo") as fh:
            for line in fh:
                if line.startswith("model name"):
                    model = line.split(":", 1)[1].strip()
                    break
    except OSError:
        pass
    blas = "unknown"
    try:
        dep = np.show_config(mode="dicts")["Build Dependencies"]["blas"]
        blas = f"{dep.get('name')} {dep.get('version')}"
    except Exception:
        pass
    return model, blas


def cpu_baseline(config, K, T, rows, unit, runs=5):
    """The oracle as it stands (float64 NumPy) on the host cores, on a
    bounded sample of the same workload: the first `rows` output rows of the
    dominant layer.  O1 (the greedy quantizer) once on the sample, then the
    product (O2 dequantize + O3 matmul, oracle.product) and O2 alone: one
    warm-up and `runs` timed runs each, medians reported, with all cores and
    with one thread."""
    import threadpoolctl

    import mbok_synth as syn
    import oracle

    cfg = syn.WORKLOADS[config]
    m, n = dominant_shape(config, K, T)
    W = syn.weight(m, n, syn.weight_seed(config, 0))[:rows]
    X = syn.activations(T, n, syn.act_seed(config, 0), cfg["x_dtype"])
    Xa = X if T > 1 else X[0]
    cores = len(os.sched_getaffinity(0))
    t = time.perf_counter()
    S, A, _ = oracle.residual_binarize(W, K, alpha_dtype=cfg["alpha_dtype"])
    t_o1 = time.perf_counter() - t
    work = (weight_bytes(rows, n, K, 2 if cfg["alpha_dtype"] == "f16" else 4) if unit == "GB/s"
            else 2.0 * rows * n * T)
    res = {}
    X2 = np.asarray(Xa, dtype=np.float64).reshape(-1, n)
    for threads in (cores, 1):
        with threadpoolctl.threadpool_limits(threads):
            oracle.product(S, A, Xa)
            tp, td, tm = [], [], []
            for _ in range(runs):
                t = time.perf_counter()
                oracle.product(S, A, Xa)
                tp.append(time.perf_counter() - t)
                t = time.perf_counter()
                Wd = oracle.dequantize(S, A)
                td.append(time.perf_counter() - t)
                # O3 on its own: the oracle's matmul of the dequantized weights
                t = time.perf_counter()
                X2 @ Wd.T
                tm.append(time.perf_counter() - t)
        res[threads] = (statistics.median(tp), statistics.median(td), statistics.median(tm))
    scale = 1e9 if unit == "GB/s" else 1e12
    model, blas = _cpu_facts()
    tp, td, tm = res[cores]
    return {"value": work / tp / scale, "unit": unit, "cores": cores, "kind": "oracle",
            "value_1_thread": work / res[1][0] / scale,
            "sample": f"oracle.product (fp64 dequantize + matmul) of rows 0..{rows - 1} of the "
                      f"{m}x{n} layer, K={K}, T={T}; median of {runs} runs after 1 warm-up",
            "o2_dequantize_s": round(td, 5), "o3_matmul_s": round(tm, 5),
            "o1_quantize_s": round(t_o1, 3), "o1_rows": rows,
            "cpu_model": model, "blas": blas, "blas_threads": cores}


# ---------------------------------------------------------------- the line

def product_figures(args, wl, steps, warmup, ceil=None):
    """Timed steps and the dominant call's roofline for one workload."""
    timed = measure_steps(wl, steps, warmup,
                          use_graph=timed_with_graph(args, steps * len(wl.layers), wl.T))
    launch_us = measure_dominant(wl, calibrate=args.calibrate_copy)
    d = wl.layers[wl.dom][1]
    alg = wl.dom_alg_bytes()
    if wl.T > 16:
        achieved = 2.0 * d.m * d.n * wl.T / (launch_us * 1e-6) / 1e12
        roof = {"bound": "mfma", "achieved": achieved, "peak": BF16_MFMA_PEAK_TFLOPS,
                "unit": "TFLOP/s", "frac": achieved / BF16_MFMA_PEAK_TFLOPS}
        if ceil:
            roof["measured_ceiling"] = ceil["mfma_bf16_TFLOP/s"]
            roof["frac_of_measured_ceiling"] = achieved / ceil["mfma_bf16_TFLOP/s"]
    else:
        achieved = alg / (launch_us * 1e-6) / 1e9
        roof = {"bound": "hbm", "achieved": achieved, "peak": HBM_PEAK_GBPS, "unit": "GB/s",
                "frac": achieved / HBM_PEAK_GBPS}
        r = (ceil or {}).get("read", {}).get(str(int(alg) // 16 * 16))
        if r:
            roof["measured_ceiling"] = r["GB/s"]
            roof["frac_of_measured_ceiling"] = achieved / r["GB/s"]
            roof["read_ceiling_us"] = r["us"]
    roof["traffic"] = (stored_traffic(wl.config, wl.K, wl.T)
                       if wl.allocation is None and not wl.transposed and not wl.svid else None)
    roof["kernel"] = f"{wl.layers[wl.dom][0]} {d.m}x{d.n}"
    roof["launch_us"] = launch_us
    roof["alg_bytes_per_launch"] = alg
    if wl.T > 16:
        roof["alg_flops_per_launch"] = 2.0 * d.m * d.n * wl.T
    return timed, roof


def _pool(timed):
    return {k: timed[k] for k in ("pool_copies", "timed_copies", "timed_pool_MB",
                                  "read_before_timing_MB")}


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
    from boolean_weight_amd import ceilings

    if not torch.cuda.is_available():
        print("no GPU visible", file=sys.stderr)
        sys.exit(1)
    bw.load_library()
    ceilings.load()
    torch.cuda.set_device(0)

    def note(msg):
        print(f"bench: {msg}", file=sys.stderr, flush=True)

    cfg = syn.WORKLOADS[args.config]
    K = args.K or cfg["K"]
    T = args.T or cfg["T"][0]
    if args.ceilings:
        ceil = measure_ceilings([4743168, 19_070_000, 59_700_000, 268_435_456])
        for kind in (ceilings.MFMA_F4F8, ceilings.MFMA_F4F8_LANE_SCALES):
            ceil[f"mfma_kind{kind}_TFLOP/s"] = round(ceilings.mfma_rate(kind)["TFLOP/s"], 1)
        print(json.dumps({"metric": "ceilings", "kind": "measurement", **ceil}), flush=True)
        return
    if args.svid and (T != 1 or args.transposed or args.avg_k is not None):
        print("--svid runs one token on its own", file=sys.stderr)
        sys.exit(2)
    if args.transposed and T != 1:
        print("--transposed runs one gradient vector (T = 1)", file=sys.stderr)
        sys.exit(2)
    if args.quantizer:
        quantizer_bench(args, cfg, cfg["linears"], K,
                        bw.MBOK_F16 if cfg["alpha_dtype"] == "f16" else bw.MBOK_F32,
                        2 if cfg["alpha_dtype"] == "f16" else 4)
        return
    if args.library_gemm:
        library_gemm_bench(args, cfg, cfg["linears"], T)
        return

    launches, allocation = None, None
    if args.avg_k is not None:
        if args.config != 4:
            print("--avg-k applies to the LLaMA-13B-shaped layer (--config 4)", file=sys.stderr)
            sys.exit(2)
        adt = bw.MBOK_F16 if cfg["alpha_dtype"] == "f16" else bw.MBOK_F32
        Ws = [torch.from_numpy(syn.weight(m, n, syn.weight_seed(4, li))).to("cuda")
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
                Wc = torch.cat([Ws[t] for t in idx])
                launches.append(("|".join(group), Wc, Ks[idx[0]], Wc.shape[0], Wc.shape[1]))
            else:
                launches.extend((names[t], Ws[t], Ks[t], Ws[t].shape[0], Ws[t].shape[1])
                                for t in idx)
        del Ws
        K = max(Ks)

    note(f"setup: workload {args.config} ({cfg['name']}), K={K}, T={T}")
    wl = Workload(args, args.config, K, T, launches)
    wl.allocation = allocation
    note("ceilings")
    ceil = measure_ceilings([wl.dom_alg_bytes()])
    note(f"timed region: {args.steps} steps after {args.warmup} warm-up steps")
    timed, roof = product_figures(args, wl, args.steps, args.warmup, ceil)
    ms = timed["ms_per_step"]

    if args.svid:
        metric, unit, value = "svid weight GB/s", "GB/s", wl.wbytes / (ms * 1e-3) / 1e9
    elif args.transposed:
        metric, unit, value = "transposed weight GB/s", "GB/s", wl.wbytes / (ms * 1e-3) / 1e9
    elif T > 16:
        metric, unit, value = "prefill TFLOP/s", "TFLOP/s", wl.flops / (ms * 1e-3) / 1e12
    else:
        metric, unit, value = "weight GB/s", "GB/s", wl.wbytes / (ms * 1e-3) / 1e9
    if args.default_line:
        metric = ("weight GB/s (% HBM peak) for the sum_k alpha_k B_k x decode GEMV at "
                  "LLaMA-7B shapes; prefill TFLOP/s in 'prefill'")
    line = {
        "metric": metric, "value": value, "unit": unit, "n_gpus": 1, "steps": args.steps,
        "warmup": args.warmup, "ms_per_step": ms, "higher_is_better": True,
        "scaling": "weak", "vs_baseline": None,
        "dtype": f"{cfg['x_dtype']} x, {cfg['alpha_dtype']} alpha, f32 accumulate",
        "data": "synthetic (seeded N(0,0.02) weights via greedy residual binarization, "
                "N(0,1) activations)",
        "config": {"workload": cfg["name"],
                   "linears": [[nm, dd.m, dd.n] for nm, dd in wl.layers],
                   "K": K if allocation is None else allocation, "group": 128, "T": T,
                   "alpha_dtype": cfg["alpha_dtype"], "x_dtype": cfg["x_dtype"],
                   "launch": ("hip graph" if timed["graph"] else
                              "stream launches enqueued behind a spin kernel"),
                   "pool": _pool(timed), "wall_s": round(timed["wall_s"], 3)},
        "tokens_per_s": (T if args.config != 4 else 1) / (ms * 1e-3),
        "pct_hbm_peak_of_value": round(100 * value / HBM_PEAK_GBPS, 2) if unit == "GB/s" else None,
        "roofline": roof,
        "ceilings": ceil,
    }
    if args.config == 4:
        line["config"]["tokens_per_s_counts"] = "one token through one decoder layer"
    if args.transposed:
        line["config"]["product"] = "dx = W_hat^T g"
    if args.svid:
        line["config"]["product"] = "y = sum_k s_out^k (.) (B_k (s_in^k (.) x)) (successive SVID)"
        line["config"]["svid_iters"] = args.svid_iters
    del wl
    torch.cuda.empty_cache()

    extra = args.default_line and not args.no_extra and not (args.svid or args.transposed)
    if extra:
        # the other half of the metric: prefill TFLOP/s (11008x4096, K=3, 2048 tokens)
        note("prefill: setup")
        pw = Workload(args, 5)
        note(f"prefill: timed region: {args.steps} steps after {args.warmup} warm-up steps")
        ptimed, proof = product_figures(args, pw, args.steps, args.warmup, ceil)
        pms = ptimed["ms_per_step"]
        ptf = pw.flops / (pms * 1e-3) / 1e12
        line["prefill"] = {
            "workload": syn.WORKLOADS[5]["name"], "K": pw.K, "T": pw.T, "value": ptf,
            "unit": "TFLOP/s", "steps": args.steps, "warmup": args.warmup, "ms_per_step": pms,
            "tokens_per_s": pw.T / (pms * 1e-3),
            "pct_bf16_peak_of_value": round(100 * ptf / BF16_MFMA_PEAK_TFLOPS, 2),
            "dtype": "bf16 x and bf16 W_hat tiles, f16 alpha, f32 accumulate",
            "pool": _pool(ptimed), "roofline": proof}
        # the same workload through the two-term product (hi + lo bf16 levels)
        note("prefill: two-term product")
        pw.precise = True
        qsteps = max(1, args.steps // 4)
        qtimed = measure_steps(pw, qsteps, max(1, args.warmup // 4),
                               use_graph=timed_with_graph(args, qsteps * len(pw.layers), pw.T))
        qms = qtimed["ms_per_step"]
        line["prefill"]["precise"] = {
            "entry": "mbok_gemm_precise", "steps": qsteps, "ms_per_step": qms,
            "value": pw.flops / (qms * 1e-3) / 1e12, "unit": "TFLOP/s",
            "dtype": "bf16 x, two bf16 terms per W_hat level, f16 alpha, f32 accumulate",
            "pool": _pool(qtimed)}
        del pw
        torch.cuda.empty_cache()
        # the LLaMA-7B MLP decode shapes (gate/up 11008x4096, down 4096x11008, K=3)
        mlp = {}
        for name, m, n in syn.WORKLOADS[3]["linears"]:
            if name == "up_proj":
                continue  # the shape of gate_proj
            note(f"MLP decode: {name} {m}x{n}")
            li = [nm for nm, _, _ in syn.WORKLOADS[3]["linears"]].index(name)
            Wl = torch.from_numpy(syn.weight(m, n, syn.weight_seed(3, li))).to("cuda")
            mw = Workload(args, 3, 3, 1, [(name, Wl, 3, m, n)])
            del Wl
            mtimed, mroof = product_figures(args, mw, args.steps, args.warmup, None)
            mms = mtimed["ms_per_step"]
            gbs = mw.wbytes / (mms * 1e-3) / 1e9
            mlp[name] = {"shape": [m, n], "K": 3, "value": gbs, "unit": "GB/s",
                         "ms_per_step": mms, "pct_hbm_peak_of_value": round(100 * gbs / HBM_PEAK_GBPS, 2),
                         "kernel_launch_us": mroof["launch_us"], "pool": _pool(mtimed)}
            del mw
            torch.cuda.empty_cache()
        line["mlp_decode"] = mlp
        # the few-token product on the whole LLaMA-7B MLP step (gate, up, down)
        few = {}
        for Tq in (4, 16):
            note(f"MLP few-token step: {Tq} tokens")
            fw = Workload(args, 3, 3, Tq)
            ftimed, froof = product_figures(args, fw, args.steps, args.warmup, None)
            fms = ftimed["ms_per_step"]
            gbs = fw.wbytes / (fms * 1e-3) / 1e9
            fd = fw.layers[fw.dom][1]
            few[f"T{Tq}"] = {"linears": [[nm, m, n] for nm, m, n in syn.WORKLOADS[3]["linears"]],
                             "K": 3, "T": Tq, "value": gbs, "unit": "GB/s", "ms_per_step": fms,
                             "tokens_per_s": Tq / (fms * 1e-3),
                             "pct_hbm_peak_of_value": round(100 * gbs / HBM_PEAK_GBPS, 2),
                             "dominant_kernel": kernel_family(Tq, fd.m, fd.n, 3)[1],
                             "dominant_launch_us": froof["launch_us"], "pool": _pool(ftimed)}
            del fw
            torch.cuda.empty_cache()
        line["few_token"] = few

    if not args.no_cpu_baseline:
        note("cpu baseline")
        if args.transposed or args.svid:
            line["cpu_baseline"] = None
        else:
            rows = 512 if T > 1 else (1024 if args.config == 4 else dominant_shape(args.config, K, T)[0])
            line["cpu_baseline"] = cpu_baseline(args.config, K if allocation is None else 3,
                                                T, rows, unit)
            if "prefill" in line:
                line["prefill"]["cpu_baseline"] = cpu_baseline(5, 3, 2048, 512, "TFLOP/s")
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



if __name__ == "__main__":
    main()
