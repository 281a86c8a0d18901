"""Throughput of the quantized attention hot path on one MI355X.

python bench.py [--gpus 1] [--steps K] [--warmup W] [--workload NAME] [--no-cpu-baseline] [--two-pass]
                [--latency [--samples S]]

--workload takes any workload of quantized_attention_video_amd/workloads.py; a packed one
(varlen_h24_4seg) passes cu_seqlens.

A step is one pass of the whole path over one batch of synthetic input already resident
in HBM: sattn_quantize_qkv with the Q buffers absent (K statistics, mean-smoothed INT8 K
tiles, E4M3 V tiles) followed by sattn_fwd_fused (the attention kernel, which quantizes
each workgroup's Q rows to INT8 from the BF16 view before its key loop).  The default
workload is the H3-like video layer: B=1, H=32, L=37,810 packed tokens, D=128, Q/K/V
projection-strided slices of one fused [L, 3, H, D] BF16 tensor.  `value` is 4*Lq*Lk*D*H
per step over the measured step time (TOPS).  The attention kernel's own launches are
timed with HIP events on the stream it runs on; its algorithmic operation count over that
time, against the 5.0 POP/s dense INT8/FP8 MFMA peak, is the roofline entry.  The CPU
baseline times the FP64 oracle on a bounded sample of the same workload and extrapolates
linearly.

--latency (for the small shapes, e.g. --workload fixed_q128_kv192) reports the per-launch
time of sattn_fwd the way the pages time their fixed-shape kernel: samples of 20
back-to-back launches, the per-launch time being a sample's event interval over 20; the
launches are replayed from a captured HIP graph so that host enqueue time (Python and
ctypes) does not stretch the interval, with the eager figure beside it.  sattn_fwd gets
its forward workspace (--no-split withholds it), with which the query tiles of a short last
dispatch round split their keys between two workgroups on CUs of their own.  Its
CPU baseline is the whole oracle on the whole shape, on one host thread and on all of them.

--summarize-trace CSV (with the --steps/--warmup of the profiled run) reads a rocprofv3
kernel-trace CSV of a bench.py run and prints per-kernel launch statistics with the warm-up
launches and the timed ones apart; --summarize-counters CSV [CSV ...] prints the mean of
every counter of rocprofv3 --pmc runs per kernel over the timed launches.

--two-pass times the other form of the same path: sattn_quantize_qkv (Q as well) followed
by sattn_fwd (or sattn_fwd_varlen) over the INT8 Q tiles.  The outputs are bit-identical;
the fused form saves the Q pass (a BF16 read and an INT8 write of Q) and is the default.
"""
import argparse
import hashlib
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

PEAK_TOPS = 5000.0  # MI355X dense INT8 (and FP8) MFMA peak, TOP/s
HBM_PEAK_GBS = 8000.0
TRAFFIC_FILE = os.path.join(ROOT, "profiles", "attn_fwd_fused_h3_l37810_traffic.txt")
KERNEL_SRC = os.path.join(ROOT, "quantized_attention_video_amd", "csrc", "attn.hip")


def kernel_source_hash():
    return hashlib.sha256(open(KERNEL_SRC, "rb").read()).hexdigest()[:16]


def measured_traffic(workload):
    """HBM bytes per attention launch from the committed rocprofv3 counter summary, or None
    if there is none for this workload or the kernel source changed since it was taken."""
    if not os.path.exists(TRAFFIC_FILE):
        return None
    kv = {}
    for line in open(TRAFFIC_FILE):
        if "=" in line and not line.lstrip().startswith("#"):
            a, b = line.split("=", 1)
            kv[a.strip()] = b.strip()
    if kv.get("workload") != workload or kv.get("attn_hip_sha256_16") != kernel_source_hash():
        return None
    try:
        return float(kv["hbm_bytes_per_launch"])
    except (KeyError, ValueError):
        return None


def _head_slice(seg, n):
    """The first n heads of one segment of the oracle's quantized output."""
    return {k: (v[:, :n] if k in ("q8", "k8", "v8", "v8val") else v[:n] if hasattr(v, "shape") else v)
            for k, v in seg.items()}


def cpu_baseline(w, inp, att_heads=8, rows=1024):
    """Time the oracle on a bounded sample of the step: the quantization of all heads over
    all tokens, and attention for `rows` query rows (half from each end) of the first
    segment's first `att_heads` heads against all of its keys; the attention time is
    extrapolated linearly, by operation count, to every row, head and segment."""
    import numpy as np
    from threadpoolctl import threadpool_info

    from oracle import sattn as O
    from quantized_attention_video_amd import workloads as W

    q, k, v = (W.packed_float64(inp[n]) for n in "qkv")
    t0 = time.perf_counter()
    quant = O.quantize(q, k, v, inp["cu_q"], inp["cu_k"])
    t1 = time.perf_counter()
    L0, Lk0 = w.seqlens_q()[0], w.seqlens_k()[0]
    rows = min(rows, L0)
    att_heads = min(att_heads, w.H)
    sel = np.concatenate([np.arange(0, rows // 2), np.arange(L0 - (rows - rows // 2), L0)])
    O.attention([_head_slice(seg, att_heads) for seg in quant], w.sm_scale, rows={0: sel})
    t2 = time.perf_counter()
    est = (t1 - t0) + (t2 - t1) * w.ops() / (4 * 128 * att_heads * rows * Lk0)
    threads = max([p.get("num_threads", 1) for p in threadpool_info()] + [1])
    return {
        "value": w.ops() / est / 1e12,
        "unit": "TOPS",
        "cores": threads,
        "kind": "oracle",
        "sample": (f"FP64 oracle: quantization of all {w.H} heads over all tokens ({t1 - t0:.1f} s) + "
                   f"attention for {rows} query rows of {att_heads}/{w.H} heads of the first "
                   f"{'segment' if w.varlen else 'sequence'} against all its keys ({t2 - t1:.1f} s); "
                   f"attention extrapolated linearly by operation count to all rows, heads and "
                   f"sequences: full step = {est:.0f} s"),
        "cpu": _cpu_model(),
    }


def _data_recipe(w):
    parts = ["seeded N(0,1) BF16"]
    if w.k_bias_std:
        parts.append(f"per-channel K bias N(0,{w.k_bias_std:g})")
    if w.q_boost_frac:
        parts.append(f"{w.q_boost_frac:.0%} of Q rows x8")
    return "synthetic (" + ", ".join(parts) + ")"


def _pct(xs, p):
    """p-th percentile (linear interpolation) of a list."""
    xs = sorted(xs)
    r = (len(xs) - 1) * p / 100.0
    lo = int(r)
    hi = min(lo + 1, len(xs) - 1)
    return xs[lo] + (xs[hi] - xs[lo]) * (r - lo)


def _cv(xs):
    """Coefficient of variation (standard deviation over mean)."""
    m = sum(xs) / len(xs)
    return (sum((x - m) ** 2 for x in xs) / len(xs)) ** 0.5 / m if m else 0.0


def copy_gbs(torch, nbytes=1 << 30, reps=5):
    """HBM rate of a plain device copy (bytes read + written per second, GB/s): what a
    pure streaming kernel reaches on this part, beside the 8 TB/s nameplate."""
    src = torch.empty(nbytes, dtype=torch.uint8, device="cuda").fill_(1)
    dst = torch.empty_like(src)
    dst.copy_(src)
    a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    a.record()
    for _ in range(reps):
        dst.copy_(src)
    b.record()
    torch.cuda.synchronize()
    rate = 2 * nbytes * reps / (a.elapsed_time(b) * 1e-3) / 1e9
    del src, dst
    return rate


def _cpu_model():
    try:
        for line in open("/proc/cpuinfo"):
            if line.startswith("model name"):
                return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return "unknown"


# The pages' fixed-shape figure (B=1, H=1, Q=128, KV=192): VEA-B per-launch p50 over 500
# samples of 20 launches on GB10 ([Report] "Timing"); context for --latency, another chip.
PAGES_FIXED_SHAPE_US = 14.426


def cpu_oracle_full(w, inp):
    """The whole oracle (quantization + attention of every row and head) on the whole
    shape, timed on one host thread and on all of them (BLAS threads)."""
    from threadpoolctl import threadpool_info, threadpool_limits

    from oracle import sattn as O
    from quantized_attention_video_amd import workloads as W

    q, k, v = (W.packed_float64(inp[n]) for n in "qkv")

    def run():
        t0 = time.perf_counter()
        O.attention(O.quantize(q, k, v, inp["cu_q"], inp["cu_k"]), w.sm_scale)
        return time.perf_counter() - t0

    small = w.ops() <= 1e9
    if small:
        run()  # warm-up (imports, first-touch)
    reps = 3 if small else 1
    t_all = min(run() for _ in range(reps))
    with threadpool_limits(limits=1):
        t_one = min(run() for _ in range(reps))
    threads = max([p.get("num_threads", 1) for p in threadpool_info()] + [1])
    return {"value": t_all * 1e6, "unit": "us", "cores": threads, "kind": "oracle",
            "single_thread_us": t_one * 1e6,
            "sample": f"FP64 oracle, whole shape (quantize + attention), {'best of 3' if small else 'one run'}",
            "cpu": _cpu_model()}


def latency(args, w, torch, B):
    """Per-launch time of sattn_fwd on one dense shape (see the module docstring)."""
    from quantized_attention_video_amd import workloads as W

    inp = W.make_inputs(w)
    dev = W.to_device(inp)
    q, k, v = dev["q"], dev["k"], dev["v"]
    Bn, Lq, H = q.shape[:3]
    Lk = k.shape[1]
    quant = B.alloc_quantized(Bn, Bn * Lq, Bn * Lk, H)
    out = torch.empty((Bn, Lq, H, 128), dtype=torch.bfloat16, device="cuda")
    B.sattn_quantize_qkv(q, k, v, out=quant)
    per = 20
    ws = None if args.no_split else B.split_workspace(Bn, H, Lq, Lk)  # lets small grids split their keys

    def fwd():
        B.sattn_fwd(quant, Bn, H, Lq, Lk, w.sm_scale, out=out, workspace=ws)

    fwd()
    torch.cuda.synchronize()
    ref = out.clone()
    # the split leaves its partial results in the workspace (and its counters at zero); a
    # forward that does not split never writes it
    key_split = ws is not None and bool(ws.any())

    def sample_times(launch, n, count):
        """n event intervals around `launch()`, each covering `count` kernel launches (us per launch)."""
        for _ in range(args.warmup):
            launch()
        ev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in range(n)]
        stream = torch.cuda.current_stream()
        for a, b in ev:
            a.record(stream)
            launch()
            b.record(stream)
        torch.cuda.synchronize()
        return [a.elapsed_time(b) * 1e3 / count for a, b in ev]

    def eager20():
        for _ in range(per):
            fwd()

    eager = sample_times(eager20, args.samples, per)
    single = sample_times(fwd, 4 * args.samples, 1)
    # the same 20 launches captured once and replayed (no host work between kernels)
    g = torch.cuda.CUDAGraph()
    out.zero_()
    torch.cuda.synchronize()
    with torch.cuda.graph(g):
        eager20()
    graph = sample_times(g.replay, args.samples, per)
    replays_ok = True
    for _ in range(3):  # every replay, with eager work between, must reproduce the eager output
        out.zero_()
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        replays_ok &= bool(torch.equal(out, ref))
        fwd()
        torch.cuda.synchronize()

    def stats(xs):
        return {"p10": _pct(xs, 10), "p50": _pct(xs, 50), "p90": _pct(xs, 90), "cv": _cv(xs), "samples": len(xs)}

    value = _pct(graph, 50)
    line = {
        "metric": "sattn_fwd time per launch (20 back-to-back launches per sample)",
        "value": value,
        "unit": "us",
        "n_gpus": 1,
        "higher_is_better": False,
        "vs_baseline": value / PAGES_FIXED_SHAPE_US if w.name == "fixed_q128_kv192" else None,
        "dtype": "int8 (QK) + fp8 e4m3 (PV), fp32 softmax",
        "data": _data_recipe(w),
        "config": {"workload": w.name, "B": Bn, "H": H, "Lq": Lq, "Lk": Lk, "D": 128, "layout": w.layout,
                   "launches_per_sample": per, "forward_workspace": ws is not None, "key_split": key_split},
        "graph_replay_us": stats(graph),
        "eager_us": stats(eager),
        "single_launch_us": stats(single),
        "graph_replays_match_eager": replays_ok,
        "tops_at_p50": w.ops() / (value * 1e-6) / 1e12,
    }
    if w.name == "fixed_q128_kv192":
        line["context"] = (f"pages, GB10: {PAGES_FIXED_SHAPE_US} us per launch p50 (same shape, 500 x 20 "
                           f"launches); vs_baseline = value / that")
    if not args.no_cpu_baseline and w.ops() <= 1e11:  # larger shapes: the throughput mode's sampled baseline
        line["cpu_baseline"] = cpu_oracle_full(w, inp)
    print(json.dumps(line))
    if not replays_ok:
        raise SystemExit("graph replays differ from the eager output")


def _short(name):
    """A kernel's name without namespace and argument list (templates kept)."""
    n = name.split("(")[0]
    return n.replace("sattn::", "")


def summarize_trace(path, steps, warmup):
    """Per-kernel launch times of a rocprofv3 kernel trace of bench.py: the first `warmup`
    launches of each step kernel are the warm-up, the next `steps` the timed ones."""
    import csv
    rows = sorted(csv.DictReader(open(path)), key=lambda r: int(r["Start_Timestamp"]))
    by = {}
    for r in rows:
        by.setdefault(_short(r["Kernel_Name"]), []).append((int(r["End_Timestamp"]) - int(r["Start_Timestamp"])) / 1e3)
    print(f"{'kernel':44s} {'phase':7s} {'calls':>5s} {'avg_us':>10s} {'p50_us':>10s} {'min_us':>10s} {'max_us':>10s}")
    for k, us in by.items():
        parts = [("all", us)]
        if len(us) == steps + warmup:
            parts = [("warm-up", us[:warmup]), ("timed", us[warmup:])]
        for label, xs in parts:
            if xs:
                print(f"{k[:44]:44s} {label:7s} {len(xs):5d} {sum(xs) / len(xs):10.1f} {_pct(xs, 50):10.1f} "
                      f"{min(xs):10.1f} {max(xs):10.1f}")


def summarize_counters(paths, steps, warmup):
    """Mean of every rocprofv3 --pmc counter per kernel (summed over the dimensions a counter
    reports per dispatch), over the timed launches of the step kernels (the last `steps`)."""
    import csv
    per = {}  # (kernel, counter) -> {dispatch: value}
    for path in paths:
        for r in csv.DictReader(open(path)):
            key = (_short(r["Kernel_Name"]), r["Counter_Name"])
            d = per.setdefault(key, {})
            d[int(r["Dispatch_Id"])] = d.get(int(r["Dispatch_Id"]), 0.0) + float(r["Counter_Value"])
    for (k, cn), d in sorted(per.items()):
        vals = [d[i] for i in sorted(d)]
        if len(vals) == steps + warmup:
            vals = vals[warmup:]
        print(f"{k[:44]:44s} {cn:28s} n={len(vals):3d} mean={sum(vals) / len(vals):.6g}")


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=50)
    ap.add_argument("--warmup", type=int, default=20)
    ap.add_argument("--workload", default="h3_video_l37810")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--two-pass", action="store_true",
                    help="step = Q/K/V quantization + sattn_fwd over INT8 Q tiles (default: K/V quantization + "
                         "sattn_fwd_fused, which prepares Q inside the attention launch)")
    ap.add_argument("--latency", action="store_true",
                    help="per-launch time of sattn_fwd on a small dense shape (samples of 20 launches)")
    ap.add_argument("--samples", type=int, default=500, help="--latency: samples of 20 launches")
    ap.add_argument("--no-split", action="store_true",
                    help="--latency: no forward workspace (small grids do not split their keys)")
    ap.add_argument("--copy-calib", type=int, default=0,
                    help="only run N plain 1 GiB device copies (counter calibration) and exit")
    ap.add_argument("--summarize-trace", metavar="CSV", help="print launch statistics of a rocprofv3 kernel trace")
    ap.add_argument("--summarize-counters", metavar="CSV", nargs="+", help="print per-kernel counter means")
    args = ap.parse_args()
    if args.summarize_trace:
        summarize_trace(args.summarize_trace, args.steps, args.warmup)
        return
    if args.summarize_counters:
        summarize_counters(args.summarize_counters, args.steps, args.warmup)
        return
    if args.gpus != 1:
        print(f"bench.py runs on exactly one GPU: this build has no multi-GPU path "
              f"(asked for --gpus {args.gpus}).", file=sys.stderr)
        sys.exit(2)

    import torch

    if args.copy_calib:
        src = torch.empty(1 << 30, dtype=torch.uint8, device="cuda").fill_(1)
        dst = torch.empty_like(src)
        for _ in range(args.copy_calib):
            dst.copy_(src)
        torch.cuda.synchronize()
        print(json.dumps({"copy_bytes_each": 1 << 30, "copies": args.copy_calib}))
        return

    from quantized_attention_video_amd import binding as B
    from quantized_attention_video_amd import workloads as W

    w = W.get(args.workload)
    if args.latency:
        if w.varlen:
            raise SystemExit("--latency times dense shapes")
        latency(args, w, torch, B)
        return
    inp = W.make_inputs(w)
    dev = W.to_device(inp)
    q, k, v = dev["q"], dev["k"], dev["v"]
    stream = torch.cuda.current_stream()
    if w.varlen:  # packed [T, H, D] with cu_seqlens (block-diagonal attention per segment)
        T, H = q.shape[0], q.shape[1]
        nseg = len(w.seqlens)
        Bn, Lq, Lk = 1, T, T  # for the byte count below: one packed sequence of T tokens
        cq = torch.tensor(inp["cu_q"], dtype=torch.int32, device="cuda")
        ck = torch.tensor(inp["cu_k"], dtype=torch.int32, device="cuda")
        quant = B.alloc_quantized(nseg, T, T, H, with_q=args.two_pass)
        out = torch.empty((T, H, 128), dtype=torch.bfloat16, device="cuda")
        ws = B.fwd_workspace(nseg)
    else:
        Bn, Lq, H = q.shape[:3]
        Lk = k.shape[1]
        cq = ck = None
        quant = B.alloc_quantized(Bn, Bn * Lq, Bn * Lk, H, with_q=args.two_pass)
        out = torch.empty((Bn, Lq, H, 128), dtype=torch.bfloat16, device="cuda")

    def step(ev=None):
        if ev:
            ev[0].record(stream)
        B.sattn_quantize_qkv(q, k, v, cq, ck, out=quant, stream=stream)
        if ev:
            ev[1].record(stream)
        if not args.two_pass:
            B.sattn_fwd_fused(quant, q, w.sm_scale, cq, ck, Lk=Lk, out=out, workspace=ws if w.varlen else None,
                              stream=stream)
        elif w.varlen:
            B.sattn_fwd_varlen(quant, cq, ck, T, w.sm_scale, out=out, workspace=ws, stream=stream)
        else:
            B.sattn_fwd(quant, Bn, H, Lq, Lk, w.sm_scale, out=out, stream=stream)
        if ev:
            ev[2].record(stream)

    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()
    events = [[torch.cuda.Event(enable_timing=True) for _ in range(3)] for _ in range(args.steps)]
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for i in range(args.steps):
        step(events[i])
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    quant_ms = [e[0].elapsed_time(e[1]) for e in events]
    fwd_ms = [e[1].elapsed_time(e[2]) for e in events]

    ops = w.ops()
    ms_per_step = wall * 1e3 / args.steps
    fwd_avg = sum(fwd_ms) / len(fwd_ms)
    quant_avg = sum(quant_ms) / len(quant_ms)
    achieved = ops / (fwd_avg * 1e-3) / 1e12
    traffic = None if args.two_pass else measured_traffic(w.name)
    # algorithmic HBM bytes of the quantization pass: Q read once (2D) and written as INT8
    # (D); K and V read twice each (statistics, then quantization: 8D) and written once (2D)
    quant_bytes = H * Bn * ((3 * 128 * Lq if args.two_pass else 0) + 10 * 128 * Lk)
    copy_rate = copy_gbs(torch)  # after the timed steps
    step_name = ("sattn_quantize_qkv + sattn_fwd_varlen" if args.two_pass and w.varlen else
                 "sattn_quantize_qkv + sattn_fwd" if args.two_pass else "sattn_quantize_qkv (K, V) + sattn_fwd_fused")
    result = {
        "metric": ("attention TOPS (4*Lq*Lkv*D*H/s) at L=37,810 D=128; % of MFMA peak" if w.name == "h3_video_l37810"
                   else "attention TOPS (4*Lq*Lkv*D*H/s, summed over segments); % of MFMA peak"),
        "value": ops / (ms_per_step * 1e-3) / 1e12,
        "unit": "TOPS",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": ms_per_step,
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "int8 (QK) + fp8 e4m3 (PV), fp32 softmax",
        "data": _data_recipe(w),
        "config": ({"workload": w.name, "H": H, "seqlens": list(w.seqlens), "D": 128, "layout": w.layout,
                    "step": step_name} if w.varlen else
                   {"workload": w.name, "B": Bn, "H": H, "Lq": Lq, "Lk": Lk, "D": 128,
                    "layout": w.layout, "step": step_name}),
        "roofline": {
            "bound": "mfma",
            "kernel": "attn_fwd_kernel",
            "achieved": achieved,
            "peak": PEAK_TOPS,
            "unit": "TFLOP/s",
            "frac": achieved / PEAK_TOPS,
            "traffic": traffic,
            "ops_per_launch": ops,
            "avg_launch_ms": fwd_avg,
            "attn_hip_sha256_16": kernel_source_hash(),
        },
        "breakdown": {
            "fwd_ms_avg": fwd_avg,
            "fwd_ms_min": min(fwd_ms),
            "fwd_ms_p10": _pct(fwd_ms, 10),
            "fwd_ms_p50": _pct(fwd_ms, 50),
            "fwd_ms_p90": _pct(fwd_ms, 90),
            "fwd_cv": _cv(fwd_ms),
            "samples": len(fwd_ms),
            "quant_ms_avg": quant_avg,
            "fwd_tops": achieved,
            "quant_gbs": quant_bytes / (quant_avg * 1e-3) / 1e9,
            "quant_hbm_frac": quant_bytes / (quant_avg * 1e-3) / 1e9 / HBM_PEAK_GBS,
            "copy_gbs": copy_rate,
            "quant_vs_copy": quant_bytes / (quant_avg * 1e-3) / 1e9 / copy_rate,
        },
        "cpu_baseline": None,
    }
    if not args.no_cpu_baseline:
        result["cpu_baseline"] = cpu_baseline(w, inp)
    print(json.dumps(result))


if __name__ == "__main__":
    main()
