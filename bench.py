"""Benchmark of the context-parallel state-correction hot path on one MI355X.

Workload (one "step"): the 32K-token x 32-head correction in both directions and
both state layouts -- batch 1, 32 heads, 8 segments of 4096 tokens, K = V = 128,
one qla_correct_h0 call each for kv forward, vk forward, kv backward and vk
backward (1024 segment-state corrections).  Inputs are seeded synthetic data
(H ~ N(0,1), M = 0.9 I + N(0, 0.1/K), S0 ~ N(0,1)), already resident in HBM
when timing starts; backward reuses the forward arrays.

Cache perturbation: each variant's calls cycle over --rotate (16) buffer sets
(16 x 52.4 MB = 839 MB > the 256 MB MALL), and a variant's calls run back to
back, so every call streams its inputs from HBM.  The same calls on one
resident set (warm) and the bandwidth of a plain 1 GiB device copy are
reported beside it.

Timing: untimed warm-up steps first (--warmup, and at least --warmup-seconds
of back-to-back calls: a GPU that was idle runs at a low clock and needs tens
of ms of continuous work to reach its working clock), then each variant's
calls of the timed steps back to back, with HIP events on the launch stream at
the boundaries (--mode direct, default).
--mode graph follows the pages' protocol instead: each variant's launches are
captured in hipGraphs of 16 calls and replayed.

Prints one JSON line.  value = corrections/s of the whole job; roofline =
the dominant (slowest) kernel's achieved TFLOP/s (its average launch duration
from those events) against the fp32 matrix peak, and roofline_by_variant the
same for each of the four kernels; cpu_baseline = the fp64 oracle on the host,
one thread, on a sample of the same workload.  --sweep times the pages' sweep
instead (one JSON line per point).
"""
from __future__ import annotations

import argparse
import hashlib
import json
import os
import re
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

METRIC = "segment-state corrections/s + achieved HBM GB/s (% roofline), 32K tok × 32 heads"
PEAK_FP32_MFMA_TFLOPS = 157.3   # MI355X dense fp32 matrix
PEAK_HBM_GBPS = 8000.0          # MI355X HBM3E
KERNEL_SRC = os.path.join(ROOT, "linear_attention_context_amd", "csrc", "qla_kernels.hip")
TRAFFIC_FILE = os.path.join(ROOT, "profiles", "correct_h0_32k32h_traffic.md")
# The correction note (Antarx Memos), performance section, table of the 32K x
# 32-head correction kernel: per-call latency of the final (membar) scheme on
# an H100, timed as a graph of 16 calls.  Another machine and unstated head
# dims: context for the same-protocol figure below, not a target.
PAGES_H100_US = {"kv_fwd": 27.282, "vk_fwd": 29.812, "kv_bwd": 53.982, "vk_bwd": 51.474}
VARIANTS = [("kv", "fwd"), ("vk", "fwd"), ("kv", "bwd"), ("vk", "bwd")]


def parse_args(argv=None):
    p = argparse.ArgumentParser(description=__doc__, formatter_class=argparse.RawDescriptionHelpFormatter)
    p.add_argument("--gpus", type=int, default=1)
    p.add_argument("--steps", type=int, default=320)
    p.add_argument("--warmup", type=int, default=640)
    p.add_argument("--warmup-seconds", type=float, default=0.3,
                   help="warm up for at least this long (the GPU's clock ramps up over tens of ms of work)")
    p.add_argument("--mode", choices=("direct", "graph"), default="direct",
                   help="direct launches (default) or replays of captured hipGraphs")
    p.add_argument("--graph-calls", type=int, default=16, help="launches per captured graph (--mode graph)")
    p.add_argument("--rotate", type=int, default=16,
                   help="buffer sets cycled by each variant's calls (16 x 52.4 MB > the 256 MB MALL)")
    p.add_argument("--cpu-seconds", type=float, default=10.0, help="budget of the oracle CPU baseline")
    p.add_argument("--no-cpu-baseline", action="store_true")
    p.add_argument("--no-check", action="store_true", help="skip the oracle check of the timed outputs")
    p.add_argument("--sweep", action="store_true",
                   help="instead of the step: time the pages' sweep (4K/8K/32K tokens x 4/16/32 heads x "
                        "{kv,vk} x {fwd,bwd} x S0 on/off), one JSON line per point")
    p.add_argument("--configs", action="store_true",
                   help="instead of the step: time every workload configuration (tiny, 32K x 32 heads fwd and bwd, "
                        "long chain, wide grouped), one JSON line per configuration and variant")
    p.add_argument("--copy-calibration", action="store_true",
                   help="also run a plain 1 GiB device copy (for scaling rocprof byte counters); "
                        "with --configs, after the configurations")
    return p.parse_args(argv)


def kernel_source_hash() -> str:
    """sha256[:16] of the kernel source's code: // and /* */ comments and
    blank lines removed, so that a comment edit does not invalidate counters
    measured on unchanged code."""
    with open(KERNEL_SRC, encoding="utf-8") as f:
        text = f.read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    text = re.sub(r"//[^\n]*", "", text)
    code = "\n".join(line.rstrip() for line in text.splitlines() if line.strip())
    return hashlib.sha256(code.encode("utf-8")).hexdigest()[:16]


def kernel_name(variant: str, K: int) -> str:
    """Device kernel that runs a variant ("kv_fwd", ...) at head dim K: at K <= 128
    the producer kernel of the direction, above it the general kernel at
    compute size 256 (zero-padded when K < 256)."""
    layout, direction = variant.split("_")
    lay = 0 if layout == "kv" else 1
    if K <= 128:
        return f"correct_h0_{direction}_dma_kernel<{K}, {lay}>"
    return f"correct_h0_kernel<{lay}, {0 if direction == 'fwd' else 1}, {'false' if K == 256 else 'true'}>"


def read_traffic(kernel: str):
    """HBM bytes per launch of ``kernel`` from the committed rocprofv3 counter
    summary, if that summary was taken on the current kernel code."""
    if not os.path.exists(TRAFFIC_FILE):
        return None
    text = open(TRAFFIC_FILE).read()
    m_hash = re.search(r"kernel source sha256\[:16\][^`]*`([0-9a-f]{16})`", text, re.I)
    m_bytes = re.search(r"HBM bytes per launch \(scaled\),\s*`" + re.escape(kernel) + r"`:\s*([0-9.eE+]+)", text,
                        re.I)
    if not m_hash or not m_bytes or m_hash.group(1) != kernel_source_hash():
        return None
    return float(m_bytes.group(1))


def measured_copy_gbps(torch, dev) -> float:
    """Read + write bytes per second of a plain 1 GiB device-to-device copy."""
    n = 1 << 28
    a = torch.ones(n, device=dev)
    b = torch.empty(n, device=dev)
    for _ in range(2):
        b.copy_(a)
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record()
    for _ in range(5):
        b.copy_(a)
    e1.record()
    torch.cuda.synchronize()
    gbps = 2 * 4 * n * 5 / (e0.elapsed_time(e1) * 1e-3) / 1e9
    del a, b
    return gbps


def run_sweep(args) -> int:
    """The pages' sweep at K = V = 128: per point and variant, the per-call time
    on one resident buffer set (warm) and over rotating sets (> 512 MiB of
    inputs where that takes at most 64 sets), one JSON line each."""
    import torch

    import linear_attention_context_amd as qla
    import qla_inputs as qi

    qla.load_library()
    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    stream = torch.cuda.current_stream()
    K = V = 128
    copy_gbps = measured_copy_gbps(torch, dev)
    for tokens in qi.SWEEP_TOKENS:
        for heads in qi.SWEEP_HEADS:
            n = tokens // qi.SEG_TOKENS
            H, M, S0 = qi.sweep_arrays(tokens, heads)
            set_bytes = 4 * heads * (n * (2 * K * V + K * K) + K * V)
            rot = max(1, min(64, -(-(512 << 20) // set_bytes)))
            for layout in ("kv", "vk"):
                Hl = H if layout == "kv" else qi.to_vk(H)
                Sl = S0 if layout == "kv" else qi.to_vk(S0)
                sets = [dict(H=torch.from_numpy(Hl).to(dev), M=torch.from_numpy(M).to(dev),
                             S0=torch.from_numpy(Sl).to(dev), out=torch.empty(Hl.shape, device=dev))
                        for _ in range(rot)]
                # untimed calls first, at least --warmup-seconds of them: an idle GPU
                # runs at a low clock and needs tens of ms of continuous work to
                # reach its working clock
                t_w, i = time.perf_counter(), 0
                while i < 64 or time.perf_counter() - t_w < args.warmup_seconds:
                    x = sets[i % rot]
                    qla.qla_correct_h0(x["H"], x["M"], x["S0"], x["out"], layout, "fwd", 1, heads, n, K, V,
                                       stream=stream.cuda_stream)
                    i += 1
                    if i % 64 == 0:
                        torch.cuda.synchronize()
                torch.cuda.synchronize()
                for direction in ("fwd", "bwd"):
                    for s0_on in (True, False):
                        def call(x):
                            qla.qla_correct_h0(x["H"], x["M"], x["S0"] if s0_on else None, x["out"], layout,
                                               direction, 1, heads, n, K, V, stream=stream.cuda_stream)
                        times = {}
                        for label, order in (("warm", [0] * 64), ("rotated", [i % rot for i in range(max(64, rot))])):
                            for i in range(64):  # untimed
                                call(sets[order[i % len(order)]])
                            e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
                            e0.record(stream)
                            for i in order:
                                call(sets[i])
                            e1.record(stream)
                            torch.cuda.synchronize()
                            times[label] = e0.elapsed_time(e1) * 1e3 / len(order)
                        nbytes = 4.0 * heads * (n * (2 * K * V + K * K) + (K * V if s0_on else 0))
                        flop = heads * n * 2.0 * K * K * V
                        t = times["rotated"] * 1e-6
                        t_roof = max(flop / (PEAK_FP32_MFMA_TFLOPS * 1e12), nbytes / (PEAK_HBM_GBPS * 1e9))
                        print(json.dumps({
                            "sweep": {"tokens": tokens, "heads": heads, "n_seg": n, "layout": layout,
                                      "direction": direction, "s0": s0_on},
                            "us_per_call": times["rotated"], "warm_us_per_call": times["warm"],
                            "buffer_sets": rot,
                            "corrections_per_s": heads * n / t,
                            "tflops": flop / t / 1e12, "hbm_gbps": nbytes / t / 1e9,
                            "roofline_frac": t_roof / t, "measured_copy_gbps": copy_gbps,
                        }), flush=True)
                del sets
                torch.cuda.empty_cache()
    return 0


def run_configs(args) -> int:
    """Per-call time of each workload configuration and variant, with its
    algorithmic bytes and FLOP against the roofline: buffer sets rotated so
    that a call's inputs come from HBM (a single set where one already exceeds
    the 256 MB MALL), and on one resident set (warm)."""
    import torch

    import linear_attention_context_amd as qla
    import qla_inputs as qi

    qla.load_library()
    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    stream = torch.cuda.current_stream()
    for cfg in sorted(qi.CASES):
        case = qi.CASES[cfg]
        B, NH, N, K, V = case.batch, case.heads, case.n_seg, case.K, case.V
        H, M, S0 = qi.case_arrays(cfg)
        chains = B * NH
        nbytes = 4.0 * (chains * N * (2 * K * V + K * K) + (chains * K * V if S0 is not None else 0))
        flop = chains * N * 2.0 * K * K * V
        rot = max(1, min(16, -(-(768 << 20) // int(nbytes))))
        calls = ([("grouped", case.group_heads())] if case.grouped else
                 [(f"{lay}_{d}", (lay, d)) for lay, d in case.variants])
        for label, what in calls:
            if case.grouped:
                Hl, Sl = H, S0
            else:
                Hl = H if what[0] == "kv" else qi.to_vk(H)
                Sl = None if S0 is None else (S0 if what[0] == "kv" else qi.to_vk(S0))
            sets = [dict(H=torch.from_numpy(Hl).to(dev), M=torch.from_numpy(M).to(dev),
                         S0=None if Sl is None else torch.from_numpy(Sl).to(dev),
                         out=torch.empty(Hl.shape, device=dev)) for _ in range(rot)]

            def call(x):
                if case.grouped:
                    qla.qla_correct_h0_grouped(x["H"], x["M"], x["S0"], x["out"], what, B, NH, N, K, V,
                                               stream=stream.cuda_stream)
                else:
                    qla.qla_correct_h0(x["H"], x["M"], x["S0"], x["out"], what[0], what[1], B, NH, N, K, V,
                                       stream=stream.cuda_stream)
            reps = 64 if nbytes < (64 << 20) else 8
            times = {}
            for kind, order in (("warm", [0] * reps), ("rotated", [i % rot for i in range(max(reps, rot))])):
                # untimed calls first, at least --warmup-seconds of them: an idle
                # GPU runs at a low clock and needs tens of ms of continuous
                # work to reach its working clock
                t_w, i = time.perf_counter(), 0
                while i < 8 or time.perf_counter() - t_w < args.warmup_seconds:
                    call(sets[order[i % len(order)]])
                    i += 1
                    if i % 16 == 0:
                        torch.cuda.synchronize()
                torch.cuda.synchronize()
                e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
                e0.record(stream)
                for i in order:
                    call(sets[i])
                e1.record(stream)
                torch.cuda.synchronize()
                times[kind] = e0.elapsed_time(e1) * 1e3 / len(order)
            t = times["rotated"] * 1e-6
            t_hbm, t_mfma = nbytes / (PEAK_HBM_GBPS * 1e9), flop / (PEAK_FP32_MFMA_TFLOPS * 1e12)
            print(json.dumps({
                "config": cfg, "workload": case.name, "variant": label,
                "us_per_call": times["rotated"], "warm_us_per_call": times["warm"], "buffer_sets": rot,
                "corrections_per_s": chains * N / t, "hbm_gbps": nbytes / t / 1e9, "tflops": flop / t / 1e12,
                "bound": "hbm" if t_hbm > t_mfma else "mfma", "roofline_frac": max(t_hbm, t_mfma) / t,
                "algorithmic_bytes": nbytes, "flop": flop,
            }), flush=True)
            del sets
            torch.cuda.empty_cache()
    if args.copy_calibration:
        copy_calibration(torch, dev)
    return 0


def copy_calibration(torch, dev):
    """A plain 1 GiB device-to-device copy, the reference for scaling rocprof byte counters."""
    n = 1 << 28  # 1 GiB of fp32
    a = torch.empty(n, device=dev)
    b = torch.empty(n, device=dev)
    a.fill_(1.0)
    torch.cuda.synchronize()
    b.copy_(a)
    torch.cuda.synchronize()
    return {"read": 4 * n, "written": 4 * n}


def main(argv=None):
    args = parse_args(argv)
    if args.gpus != 1:
        print(f"bench.py measures one GPU; --gpus {args.gpus} is not supported (one MI355X per "
              "process; chains shard across GPUs with no exchange between them)", file=sys.stderr)
        return 2

    if args.sweep:
        return run_sweep(args)
    if args.configs:
        return run_configs(args)

    import torch

    import linear_attention_context_amd as qla
    import qla_inputs as qi

    qla.load_library()  # fail loudly before anything else if the library is missing
    case = qi.CASES[2]
    B, NH, N, K, V = case.batch, case.heads, case.n_seg, case.K, case.V
    names = [f"{l}_{d}" for l, d in VARIANTS]
    H, M, S0 = qi.case_arrays(2)
    host = {"kv": (H, S0), "vk": (qi.to_vk(H), qi.to_vk(S0))}
    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    stream = torch.cuda.current_stream()

    # Buffer sets: per layout, --rotate sets of inputs (forward and backward
    # read the same arrays); per variant, --rotate output buffers.
    inputs = {lay: [dict(H=torch.from_numpy(host[lay][0]).to(dev), M=torch.from_numpy(M).to(dev),
                         S0=torch.from_numpy(host[lay][1]).to(dev)) for _ in range(args.rotate)]
              for lay in ("kv", "vk")}
    outs = {v: [torch.full(host["kv"][0].shape, float("nan"), device=dev) for _ in range(args.rotate)]
            for v in names}
    torch.cuda.synchronize()

    def launch(v, r, stream_handle):
        layout, direction = v.split("_")
        x = inputs[layout][r]
        qla.qla_correct_h0(x["H"], x["M"], x["S0"], outs[v][r], layout, direction, B, NH, N, K, V,
                           stream=stream_handle)

    nv = len(names)
    for i in range(2 * args.rotate):  # first launches load the code objects
        for v in names:
            launch(v, i % args.rotate, stream.cuda_stream)
    torch.cuda.synchronize()

    # Host cost of one direct call (context): back to back, after warm-up.
    nd = 64
    w0 = time.perf_counter()
    for i in range(nd):
        launch(names[0], i % args.rotate, stream.cuda_stream)
    host_us = (time.perf_counter() - w0) / nd * 1e6
    torch.cuda.synchronize()

    if args.mode == "graph":
        # The pages' protocol: each variant's launches captured in a hipGraph
        # of G calls (rotating buffer sets), replayed alternately with HIP
        # events between replays on the launch stream.
        G = args.graph_calls
        if args.steps % G or args.warmup % G:
            raise SystemExit(f"--steps and --warmup must be multiples of --graph-calls ({G})")
        graphs = []
        cap = torch.cuda.Stream()
        for v in names:
            g = torch.cuda.CUDAGraph()
            with torch.cuda.graph(g, stream=cap, capture_error_mode="relaxed"):
                h = torch.cuda.current_stream().cuda_stream
                for i in range(G):
                    launch(v, i % args.rotate, h)
            graphs.append(g)
        torch.cuda.synchronize()
        for _ in range(args.warmup // G):
            for g in graphs:
                g.replay()
        torch.cuda.synchronize()
        reps = args.steps // G
        ev = [torch.cuda.Event(enable_timing=True) for _ in range(reps * nv + 1)]
        torch.cuda.synchronize()
        wall0 = time.perf_counter()
        ev[0].record(stream)
        for r in range(reps):
            for vi, g in enumerate(graphs):
                g.replay()
                ev[r * nv + vi + 1].record(stream)
        torch.cuda.synchronize()
        wall = time.perf_counter() - wall0
        gpu_ms = ev[0].elapsed_time(ev[-1])
        per_launch = {v: np.array([ev[r * nv + vi].elapsed_time(ev[r * nv + vi + 1]) for r in range(reps)]) * 1e3 / G
                      for vi, v in enumerate(names)}
        timing = f"hipGraph of {G} launches per variant, replayed alternately; events between replays"
    else:
        # Direct launches on the stream: each variant's K calls back to back
        # (same work as interleaving them), each run bracketed by HIP events on
        # the launch stream; rotating buffer sets.
        # Warm-up: --warmup steps, and at least --warmup-seconds of back-to-back
        # calls.  An idle GPU runs at a low clock and takes tens of ms of
        # continuous work to reach its working clock; calls timed before that
        # read 10-15% slow.
        t_w = time.perf_counter()
        i = 0
        while i < args.warmup or time.perf_counter() - t_w < args.warmup_seconds:
            for v in names:
                launch(v, i % args.rotate, stream.cuda_stream)
            i += 1
            if i % 64 == 0:
                torch.cuda.synchronize()
        torch.cuda.synchronize()
        ev = [torch.cuda.Event(enable_timing=True) for _ in range(nv + 1)]
        wall0 = time.perf_counter()
        ev[0].record(stream)
        for vi, v in enumerate(names):
            for i in range(args.steps):
                launch(v, i % args.rotate, stream.cuda_stream)
            ev[vi + 1].record(stream)
        torch.cuda.synchronize()
        wall = time.perf_counter() - wall0
        gpu_ms = ev[0].elapsed_time(ev[-1])
        per_launch = {v: np.array([ev[vi].elapsed_time(ev[vi + 1]) * 1e3 / args.steps]) for vi, v in enumerate(names)}
        timing = "direct launches, each variant's K calls back to back between HIP events"
    ms_per_step = max(gpu_ms, wall * 1e3) / args.steps

    # Context: the same calls on one resident buffer set (inputs warm in
    # L2/MALL), and the streaming bandwidth of a plain 1 GiB device copy.
    warm_us = {}
    for v in names:
        nw = 64
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        for _ in range(4):
            launch(v, 0, stream.cuda_stream)
        e0.record(stream)
        for _ in range(nw):
            launch(v, 0, stream.cuda_stream)
        e1.record(stream)
        torch.cuda.synchronize()
        warm_us[v] = e0.elapsed_time(e1) * 1e3 / nw
    copy_gbps = measured_copy_gbps(torch, dev)

    # Context in the pages' own protocol: a hipGraph of 16 calls on one
    # resident buffer set, per-call time of its replays.
    graph_us = {}
    cap = torch.cuda.Stream()
    for v in names:
        g = torch.cuda.CUDAGraph()
        with torch.cuda.graph(g, stream=cap, capture_error_mode="relaxed"):
            h = torch.cuda.current_stream().cuda_stream
            for _ in range(16):
                launch(v, 0, h)
        g.replay()
        torch.cuda.synchronize()
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        reps = 8
        e0.record(stream)
        for _ in range(reps):
            g.replay()
        e1.record(stream)
        torch.cuda.synchronize()
        graph_us[v] = e0.elapsed_time(e1) * 1e3 / (16 * reps)
        del g

    per_call_us = {}
    for v in names:
        d = per_launch[v]
        per_call_us[v] = {"mean": float(d.mean()), "median": float(np.median(d)),
                          "min": float(d.min()), "max": float(d.max())}
        if args.mode == "graph" and len(d) >= 75:
            # the pages' statistic: 5 rounds of 15 replays, the median of the round medians
            rounds = [np.median(d[r * 15:(r + 1) * 15]) for r in range(5)]
            per_call_us[v]["median_of_5_round_medians"] = float(np.median(rounds))

    corrections_per_step = nv * B * NH * N
    value = corrections_per_step / (ms_per_step * 1e-3)
    flop_per_launch = B * NH * N * 2.0 * K * K * V
    bytes_per_launch = 4.0 * (B * NH * N * (2 * K * V + K * K) + B * NH * K * V)
    t_roof = max(flop_per_launch / (PEAK_FP32_MFMA_TFLOPS * 1e12), bytes_per_launch / (PEAK_HBM_GBPS * 1e9))

    def roofline(v):
        t = per_call_us[v]["mean"] * 1e-6
        tflops = flop_per_launch / t / 1e12
        gbps = bytes_per_launch / t / 1e9
        return {"bound": "mfma", "achieved": tflops, "peak": PEAK_FP32_MFMA_TFLOPS, "unit": "TFLOP/s",
                "frac": tflops / PEAK_FP32_MFMA_TFLOPS, "traffic": read_traffic(kernel_name(v, K)),
                "kernel": kernel_name(v, K), "us_per_launch": per_call_us[v]["mean"],
                "flop_per_launch": flop_per_launch, "algorithmic_bytes_per_launch": bytes_per_launch,
                "hbm_gbps": gbps, "hbm_frac": gbps / PEAK_HBM_GBPS, "roofline_frac_of_max_bound": t_roof / t}

    by_variant = {v: roofline(v) for v in names}
    dominant = max(names, key=lambda v: per_call_us[v]["mean"])

    result = {
        "metric": METRIC,
        "value": value,
        "unit": "segment-state corrections/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": ms_per_step,
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "f32",
        "data": "synthetic (seeded: H~N(0,1), M=0.9I+N(0,0.1/K), S0~N(0,1))",
        "config": {"workload": "32K tokens x 32 heads: batch 1, 8 CP segments of 4096, K=V=128, forward and "
                               "backward, kv and vk layouts (one call each per step)",
                   "batch": B, "heads": NH, "n_seg": N, "K": K, "V": V,
                   "calls_per_step": names, "buffer_sets": args.rotate, "timing": timing},
        "roofline": by_variant[dominant],
        "roofline_by_variant": by_variant,
        "per_call_us": per_call_us,
        "warm_single_buffer_us_per_call": warm_us,
        "measured_copy_gbps": copy_gbps,
        "hbm_frac_of_measured_copy": by_variant[dominant]["hbm_gbps"] / copy_gbps,
        "host_us_per_call": host_us,
        "pages_protocol_context": {
            "protocol": "hipGraph of 16 calls on one resident buffer set",
            "us_per_call": graph_us,
            "h100_us_per_call_pages": PAGES_H100_US,
            "h100_over_this": {k: PAGES_H100_US[k] / graph_us[k] for k in graph_us if k in PAGES_H100_US},
        },
        "kernel_source_sha256_16": kernel_source_hash(),
    }

    if not args.no_check:
        # In-situ check: every output buffer written in the timed region
        # against the oracle.
        import oracle
        worst = 0.0
        for layout, direction in VARIANTS:
            Hl, Sl = host[layout]
            ref = oracle.correct_h0(Hl, M, Sl, layout, direction)
            den = np.sqrt((ref ** 2).sum(axis=(-1, -2)))
            for r in range(args.rotate):
                got = outs[f"{layout}_{direction}"][r].cpu().numpy().astype(np.float64)
                num = np.sqrt(((got - ref) ** 2).sum(axis=(-1, -2)))
                worst = max(worst, float((num / den).max()))
        result["timed_output_max_rel_l2"] = worst
        if not worst <= 2e-5:
            print(json.dumps(result))
            raise SystemExit(f"timed outputs fail parity: max rel L2 {worst:.3e}")

    if not args.no_cpu_baseline:
        import oracle
        oracle.build()
        # A bounded sample of the step: its four variants on the first SH of
        # the 32 heads (each head's chain is an independent unit of the same
        # work), repeated for about --cpu-seconds.
        SH = 8
        sample = {lay: (host[lay][0][:, :SH].copy(), host[lay][1][:, :SH].copy()) for lay in ("kv", "vk")}
        Ms = M[:, :SH].copy()
        per_rep = nv * B * SH * N
        reps, t0 = 0, time.perf_counter()
        while True:
            for layout, direction in VARIANTS:
                oracle.correct_h0(sample[layout][0], Ms, sample[layout][1], layout, direction)
            reps += 1
            if time.perf_counter() - t0 >= args.cpu_seconds:
                break
        el = time.perf_counter() - t0
        cpu_model = ""
        try:
            with open("/proc/cpuinfo") as f:
                cpu_model = next((ln.split(":", 1)[1].strip() for ln in f if ln.startswith("model name")), "")
        except OSError:
            pass
        result["cpu_baseline"] = {
            "value": reps * per_rep / el, "unit": "segment-state corrections/s", "cores": 1,
            "kind": "oracle", "cpu_model": cpu_model, "host_cores_available": len(os.sched_getaffinity(0)),
            "sample": f"the step's four variants on {SH} of the 32 heads ({per_rep} corrections) repeated "
                      f"{reps}x in {el:.1f} s, fp64 plain loops, 1 thread",
        }
        # Context: the same oracle over all host cores, one thread per group of
        # chains (its C loops release the interpreter lock), on the whole step.
        from concurrent.futures import ThreadPoolExecutor
        cores = max(1, min(len(os.sched_getaffinity(0)), 16, NH))
        bounds = [NH * i // cores for i in range(cores + 1)]

        def part(i):
            for layout, direction in VARIANTS:
                Hl, Sl = host[layout]
                lo, hi = bounds[i], bounds[i + 1]
                oracle.correct_h0(Hl[:, lo:hi], M[:, lo:hi], Sl[:, lo:hi], layout, direction)
        with ThreadPoolExecutor(cores) as pool:
            reps_mt, t0 = 0, time.perf_counter()
            while True:
                list(pool.map(part, range(cores)))
                reps_mt += 1
                if time.perf_counter() - t0 >= args.cpu_seconds / 2:
                    break
            el_mt = time.perf_counter() - t0
        result["cpu_baseline_all_cores"] = {
            "value": reps_mt * corrections_per_step / el_mt, "unit": "segment-state corrections/s",
            "cores": cores, "kind": "oracle",
            "sample": f"the full step repeated {reps_mt}x in {el_mt:.1f} s, heads split over {cores} threads",
        }

    if args.copy_calibration:
        result["copy_calibration_bytes"] = copy_calibration(torch, dev)

    print(json.dumps(result), flush=True)
    return 0


if __name__ == "__main__":
    sys.exit(main())
