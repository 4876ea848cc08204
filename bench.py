"""Benchmark: MoE dispatch + combine on one MI355X.

One step = the whole path on one batch: ep_layout_dispatch (the layout and
the dispatch in one call, two kernel launches) -> ep_combine, on seeded
synthetic routing and activations that are resident in HBM before timing
starts (`--two-calls` times ep_get_dispatch_layout -> ep_dispatch ->
ep_combine instead).  Successive steps take their tokens from different
copies of x, together more than twice the 256 MB MALL, so that no step
reads tokens an earlier one left in a cache.  The default workload is the
prefill configuration (4096 tokens x 7168 hidden, top-8 of 256 experts with
group-limited gating, 64 partitions, FP8 E4M3 dispatch with per-128 scales,
bf16 weighted combine).

    python bench.py [--steps K] [--warmup W] [--config prefill|decode|...]

    python bench.py --low-latency [--config decode] [--capacity C]

`--low-latency` times the decode path instead: ep_low_latency_dispatch (one
launch, fixed capacity C per expert, default C = T) -> ep_combine on expert
outputs laid out like its receive rows.  The other forms each replace the
layout and dispatch calls of the step: `--dedup` (ep_dispatch_dedup, which also
writes the layout: one copy per token and destination partition), `--align A`
(ep_layout_dispatch_aligned, every expert's run padded to a multiple of A rows)
and `--cu-budget N` (ep_layout_dispatch_cu and ep_combine_cu confined to N
CUs; with `--overlap-gemm` also timed beside a bf16 GEMM on a second stream).

Prints one JSON line (last line of stdout).  `value` is the effective HBM
throughput of a step: the algorithmic bytes of the three calls (each input
read once, each output written once) divided by the measured time per step.
`roofline` reports the dominant kernel (combine) against the 8 TB/s HBM3E
peak: its algorithmic bytes per launch over its average duration, timed with
HIP events around replays of a HIP graph of back-to-back launches on the
stream it runs on (the per-call timing inside the step, which also holds each
launch's dispatch latency, is reported beside it); `cpu_baseline` times the CPU oracle on this
host over the same workload.
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

HBM_PEAK_GBS = 8000.0
X_ROTATION_BYTES = 512 << 20      # twice the MI355X MALL (256 MB)
DOM_GRAPH_LAUNCHES = 20           # dominant-kernel launches per captured graph
METRIC = "dispatch+combine µs/call and effective HBM GB/s (% peak) at 4096×7168 top-8"
TRAFFIC_FILE = os.path.join(ROOT, "profiles", "hbm_traffic.json")
KERNEL_SOURCES = {
    "combine": ["ep_combine.hip", "ep_device.h", "ep_internal.h"],
    "dispatch": ["ep_dispatch.hip", "ep_device.h", "ep_internal.h"],
    "layout": ["ep_layout.hip", "ep_device.h", "ep_internal.h"],
    "ll_dispatch": ["ep_dispatch.hip", "ep_device.h", "ep_internal.h"],
    "layout_dispatch": ["ep_dispatch.hip", "ep_device.h", "ep_internal.h"],
    "layout_count": ["ep_layout.hip", "ep_device.h", "ep_internal.h"],
    "dispatch_dedup": ["ep_dispatch.hip", "ep_device.h", "ep_internal.h"],
}


def log(msg):
    print("[bench] " + msg, file=sys.stderr, flush=True)


def algorithmic_bytes(T, H, E, P, K, fp8):
    """Bytes the method itself must move: every input read once, every output
    written once (workspace traffic excluded)."""
    R = T * K
    G = H // 128
    layout = T * K * 8 + T * P + 4 * (E + P + (E + 1) + (P + 1))
    dispatch = T * H * 2 + T * K * 8 + R * H * (1 if fp8 else 2) + (R * G * 4 if fp8 else 0) \
        + R * 4 + R * 4
    combine = R * H * 2 + R * 4 + R * 4 + T * H * 2
    return dict(layout=layout, dispatch=dispatch, combine=combine,
                total=layout + dispatch + combine)


def ll_algorithmic_bytes(T, H, E, K, C, fp8, filled):
    """The decode path's bytes: x and the routing read once, the ``filled``
    receive rows (plus scales) written once, the whole row map and the
    counts written; combine reads the filled rows."""
    G = H // 128
    dispatch = T * H * 2 + T * K * 8 + filled * H * (1 if fp8 else 2) \
        + (filled * G * 4 if fp8 else 0) + E * C * 4 + T * K * 4 + E * 4 + 8
    combine = filled * H * 2 + T * K * 4 + T * K * 4 + T * H * 2
    return dict(ll_dispatch=dispatch, combine=combine, total=dispatch + combine)


def dedup_algorithmic_bytes(T, H, E, P, K, fp8, nd):
    """The de-duplicated path's bytes: the routing read once, the layout
    outputs, x read once, the nd used rows (codes or bf16, scales, source
    token, K local ids) written once, and the slot-row map and dst_row."""
    G = H // 128
    layout = T * K * 8 + T * P + 4 * (E + P + (E + 1) + 2 * (P + 1))
    dispatch = T * H * 2 + nd * H * (1 if fp8 else 2) + (nd * G * 4 if fp8 else 0) + nd * 4 \
        + nd * K * 4 + T * K * 4 * 2
    R = T * K
    combine = R * H * 2 + R * 4 + R * 4 + T * H * 2
    return dict(dispatch_dedup=layout + dispatch, combine=combine,
                total=layout + dispatch + combine)


def aligned_algorithmic_bytes(T, H, E, P, K, fp8, n, rows):
    """The aligned path's bytes: as the offsets path, except that only the n
    rows holding a token are written (codes or bf16, scales) while the source
    token goes to every one of the ``rows`` receive rows (padding marked)."""
    G = H // 128
    layout = T * K * 8 + T * P + 4 * (E + P + (E + 1) + (P + 1))
    dispatch = T * H * 2 + T * K * 8 + n * H * (1 if fp8 else 2) + (n * G * 4 if fp8 else 0) \
        + rows * 4 + T * K * 4
    R = T * K
    combine = R * H * 2 + R * 4 + R * 4 + T * H * 2
    return dict(layout_dispatch_aligned=layout + dispatch, combine=combine,
                total=layout + dispatch + combine)


def kernel_source_hash(kernel):
    h = hashlib.sha256()
    for name in KERNEL_SOURCES[kernel]:
        with open(os.path.join(ROOT, "combine_ep_get_dispatch_amd", "csrc", name), "rb") as f:
            h.update(f.read())
    return h.hexdigest()


def combine_kernel_name(T, H, K, num_cus):
    """Name of the kernel ep_combine launches for this shape, for the roofline
    label: top-8 without a CU budget runs in tiles of min(112 KiB / (2H), 8,
    T / 512) tokens when that is at least 2; everything else one wave per
    (token, chunk) task (the budget form under --cu-budget)."""
    kt = K if K in (1, 2, 4, 6, 8) else 0
    if num_cus:
        return "combine_budget_kernel<%d>" % kt
    if K == 8 and min(112 * 1024 // (2 * H), 8, T // 512) >= 2:
        return "combine_tile_kernel<8>"
    return "combine_kernel<%d>" % kt


def measured_traffic(kernel, config):
    """HBM bytes per launch from the committed rocprofv3 counter runs, scaled by
    the copy-kernel calibration; None when missing or taken on other code."""
    try:
        with open(TRAFFIC_FILE) as f:
            data = json.load(f)
        entry = data["kernels"][config][kernel]
        if entry["source_sha256"] != kernel_source_hash(kernel):
            return None
        cal = data["copy_calibration"]
        return int(round((entry["fetch_kib"] * cal["fetch_factor"]
                          + entry["write_kib"] * cal["write_factor"]) * 1024))
    except (OSError, KeyError, ValueError):
        return None


def pct(a, q):
    return float(np.percentile(np.asarray(a), q)) if len(a) else None


def cpu_baseline(wl_case, nbytes, seconds, capacity=None, align=0, dedup=False):
    """The CPU oracle (single-threaded C) on the same workload, repeated until
    `seconds` of CPU work have accumulated (at least one full pass).  With a
    capacity it runs the oracle's fixed-capacity path instead, with an
    alignment its aligned path (each combine on expert outputs of the
    layout's shape), with dedup its de-duplicated dispatch and the combine
    over the offsets layout's rows."""
    import oracle
    from combine_ep_get_dispatch_amd import workloads as wl
    passes, t_total = 0, 0.0
    y_ll = None
    if capacity is not None:
        y_ll = wl.normal_bf16(300 + wl.CONFIGS[wl_case.name]["c"],
                              (wl_case.E * capacity, wl_case.H))
    elif align:
        y_ll = wl.normal_bf16(300 + wl.CONFIGS[wl_case.name]["c"],
                              (oracle.aligned_rows(wl_case.T, wl_case.K, wl_case.E, align),
                               wl_case.H))
    while True:
        t0 = time.perf_counter()
        if align:
            oracle.run_aligned(wl_case.topk_idx, wl_case.x_bits, wl_case.E, wl_case.P, align,
                               wl_case.fp8, y_ll, wl_case.topk_weights)
        elif dedup:
            res = oracle.run_dedup(wl_case.topk_idx, wl_case.x_bits, wl_case.E, wl_case.P,
                                   wl_case.fp8)
            oracle.combine(wl_case.y_bits, res["dst_row"], wl_case.topk_weights)
        elif capacity is None:
            oracle.run(wl_case.topk_idx, wl_case.x_bits, wl_case.E, wl_case.P, wl_case.fp8,
                       wl_case.y_bits, wl_case.topk_weights)
        else:
            oracle.run_ll(wl_case.topk_idx, wl_case.x_bits, wl_case.E, capacity, wl_case.fp8,
                          y_ll, wl_case.topk_weights)
        t_total += time.perf_counter() - t0
        passes += 1
        log("cpu oracle pass %d: %.2f s total" % (passes, t_total))
        if t_total >= seconds:
            break
    return {"value": round(nbytes * passes / t_total / 1e9, 3), "unit": "GB/s", "cores": 1,
            "kind": "oracle",
            "sample": "%d full pass(es) of the %s workload (T=%d), %s, "
                      "single-threaded C oracle, %.1f s"
                      % (passes, wl_case.name, wl_case.T,
                         ("fixed-capacity (C=%d) dispatch+combine" % capacity) if capacity
                         else ("aligned (%d rows) layout+dispatch+combine" % align) if align
                         else "de-duplicated layout+dispatch, combine" if dedup
                         else "layout+dispatch+combine", t_total),
            "us_per_step": round(t_total / passes * 1e6, 1),
            "host": host_info()}


def host_info():
    """The host the CPU baseline ran on: logical CPUs and the CPU model."""
    model = None
    try:
        with open("/proc/cpuinfo") as f:
            for line in f:
                if line.startswith("model name"):
                    model = line.split(":", 1)[1].strip()
                    break
    except OSError:
        pass
    return {"nproc": os.cpu_count(), "cpu": model}


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=100)
    ap.add_argument("--warmup", type=int, default=10)
    ap.add_argument("--config", default=None,
                    help="workload (default: prefill; decode with --low-latency)")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--cpu-seconds", type=float, default=10.0)
    ap.add_argument("--no-copy-ceiling", action="store_true")
    ap.add_argument("--graph", action="store_true",
                    help="also time the step captured in a HIP graph and replayed")
    ap.add_argument("--graph-steps", type=int, default=10,
                    help="steps captured back to back in the one graph (--graph)")
    ap.add_argument("--two-calls", action="store_true",
                    help="layout and dispatch as two calls instead of ep_layout_dispatch")
    ap.add_argument("--cu-budget", type=int, default=0,
                    help="confine dispatch and combine to this many CUs (one-call path)")
    ap.add_argument("--overlap-gemm", action="store_true",
                    help="also time the step beside a bf16 GEMM on a second stream")
    ap.add_argument("--dedup", action="store_true",
                    help="time ep_dispatch_dedup (one copy per token and partition) + combine")
    ap.add_argument("--low-latency", action="store_true",
                    help="time the single-launch fixed-capacity decode path")
    ap.add_argument("--capacity", type=int, default=0,
                    help="rows per expert for --low-latency (default: T)")
    ap.add_argument("--flush-mb", type=int, default=512,
                    help="also time every step after reading a flush buffer of this many MiB "
                         "(0: skip)")
    ap.add_argument("--x-copies", type=int, default=0,
                    help="copies of x the steps rotate over (default: enough for 512 MiB, "
                         "at most 16; 1 = no rotation)")
    ap.add_argument("--align", type=int, default=0,
                    help="time ep_layout_dispatch_aligned with expert runs padded to this "
                         "many rows + combine")
    args = ap.parse_args()
    if args.config is None:
        args.config = "decode" if args.low_latency else "prefill"

    forms = [f for f, on in [("--two-calls", args.two_calls), ("--dedup", args.dedup),
                             ("--align", args.align), ("--low-latency", args.low_latency)] if on]
    if len(forms) > 1 or (args.cu_budget and forms):
        print("bench.py times one path at a time, and --cu-budget only the one-call path: got %s"
              % " ".join(forms + (["--cu-budget"] if args.cu_budget else [])), file=sys.stderr)
        sys.exit(2)

    world = int(os.environ.get("WORLD_SIZE", "1"))
    if args.gpus != 1 or world != 1:
        print("bench.py measures one GPU only: the library models the all-to-all's "
              "destination partitions as local HBM buffers and has no multi-GPU path; "
              "run with --gpus 1", file=sys.stderr)
        sys.exit(2)

    import torch
    from combine_ep_get_dispatch_amd import binding as ep
    from combine_ep_get_dispatch_amd import workloads as wl

    if not torch.cuda.is_available():
        print("bench.py needs a GPU", file=sys.stderr)
        sys.exit(1)
    ep.lib()
    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)

    log("generating %s inputs" % args.config)
    case = wl.make(args.config)
    T, H, E, P, K, fp8 = case.T, case.H, case.E, case.P, case.K, case.fp8
    R = T * K
    C = args.capacity or T
    if args.low_latency and T * K > ep.LL_MAX_SLOTS:
        print("--low-latency takes at most %d routing slots; %s has %d"
              % (ep.LL_MAX_SLOTS, args.config, T * K), file=sys.stderr)
        sys.exit(2)
    idx = torch.from_numpy(case.topk_idx).to(dev)
    x = torch.from_numpy(case.x_bits.view(np.int16)).to(dev).view(torch.bfloat16)
    # Steps rotate over copies of x that together exceed the 256 MB MALL twice,
    # so no step finds its tokens left in a cache by an earlier one (the
    # tokens of a real step are new each time); the routing and the outputs
    # stay put.
    n_x = args.x_copies or max(1, min(16, -(-X_ROTATION_BYTES // max(1, T * H * 2))))
    xs = [x] + [x.clone() for _ in range(n_x - 1)]
    xcur = [0]

    def xr():
        return xs[xcur[0]]
    w = torch.from_numpy(case.topk_weights).to(dev)
    out = torch.empty((T, H), dtype=torch.bfloat16, device=dev)
    if args.low_latency:
        # expert outputs laid out like the fixed-capacity receive rows
        y = torch.from_numpy(wl.normal_bf16(300 + wl.CONFIGS[args.config]["c"], (E * C, H))
                             .view(np.int16)).to(dev).view(torch.bfloat16)
        lld = ep.LowLatencyDispatched(
            torch.empty(E, dtype=torch.int32, device=dev),
            torch.empty((E * C, H), dtype=torch.uint8 if fp8 else torch.bfloat16, device=dev),
            torch.empty((E * C, H // 128), dtype=torch.float32, device=dev) if fp8 else None,
            torch.empty(E * C, dtype=torch.int32, device=dev),
            torch.empty((T, K), dtype=torch.int32, device=dev),
            torch.empty(1, dtype=torch.int64, device=dev))
        calls = [("ll_dispatch", lambda: ep.low_latency_dispatch(xr(), idx, E, C, fp8=fp8, out=lld)),
                 ("combine", lambda: ep.combine(y, lld.dst_row, w, out=out))]
    else:
        if args.align:
            # expert outputs laid out like the aligned receive rows
            R = ep.aligned_rows(T, K, E, args.align)
            y = torch.from_numpy(wl.normal_bf16(300 + wl.CONFIGS[args.config]["c"], (R, H))
                                 .view(np.int16)).to(dev).view(torch.bfloat16)
        else:
            y = torch.from_numpy(case.y_bits.view(np.int16)).to(dev).view(torch.bfloat16)
        ws = ep.new_workspace(T, K, E, P, dev)
        lay = ep.Layout(torch.empty(E, dtype=torch.int32, device=dev),
                        torch.empty(P, dtype=torch.int32, device=dev),
                        torch.empty((T, P), dtype=torch.uint8, device=dev),
                        torch.empty(E + 1, dtype=torch.int32, device=dev),
                        torch.empty(P + 1, dtype=torch.int32, device=dev), ws)
        disp = ep.Dispatched(
            torch.empty((R, H), dtype=torch.uint8 if fp8 else torch.bfloat16, device=dev),
            torch.empty((R, H // 128), dtype=torch.float32, device=dev) if fp8 else None,
            torch.empty(R, dtype=torch.int32, device=dev),
            torch.empty((T, K), dtype=torch.int32, device=dev))
        if args.dedup:
            Kp = min(K, P)
            ddo = ep.DedupDispatched(
                torch.empty(P + 1, dtype=torch.int32, device=dev),
                torch.empty((T * Kp, H), dtype=torch.uint8 if fp8 else torch.bfloat16, device=dev),
                torch.empty((T * Kp, H // 128), dtype=torch.float32, device=dev) if fp8 else None,
                torch.empty(T * Kp, dtype=torch.int32, device=dev),
                torch.empty((T * Kp, K), dtype=torch.int32, device=dev),
                torch.empty(T * K, dtype=torch.int32, device=dev), disp.dst_row)
            calls = [("dispatch_dedup", lambda: ep.dispatch_dedup(
                xr(), idx, E, P, workspace=ws, fp8=fp8, out_layout=lay, out=ddo))]
        elif args.align:
            calls = [("layout_dispatch_aligned", lambda: ep.layout_dispatch_aligned(
                xr(), idx, E, P, args.align, workspace=ws, fp8=fp8, out_layout=lay, out=disp))]
        elif args.two_calls:
            calls = [("layout", lambda: ep.get_dispatch_layout(idx, E, P, workspace=ws, out=lay)),
                     ("dispatch", lambda: ep.dispatch(xr(), idx, E, P, ws, fp8=fp8, out=disp))]
        else:
            calls = [("layout_dispatch", lambda: ep.layout_dispatch(
                xr(), idx, E, P, workspace=ws, fp8=fp8, out_layout=lay, out=disp,
                num_cus=args.cu_budget))]
        calls.append(("combine", lambda: ep.combine(y, disp.dst_row, w, out=out,
                                                    num_cus=args.cu_budget)))
    torch.cuda.synchronize()

    def step(ev=None):
        xcur[0] = (xcur[0] + 1) % n_x
        for i, (_, fn) in enumerate(calls):
            if ev is not None:
                ev[i].record()
            fn()
        if ev is not None:
            ev[len(calls)].record()

    log("warmup %d" % args.warmup)
    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()

    # ---- timed region: K back-to-back steps ---------------------------------
    t_start = torch.cuda.Event(enable_timing=True)
    t_end = torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    t_start.record()
    for _ in range(args.steps):
        step()
    t_end.record()
    torch.cuda.synchronize()
    ms_per_step = t_start.elapsed_time(t_end) / args.steps
    log("timed %d steps: %.2f us/step" % (args.steps, ms_per_step * 1e3))

    # ---- per-kernel breakdown: events around every call, same stream --------
    nc = len(calls)
    evs = [[torch.cuda.Event(enable_timing=True) for _ in range(nc + 1)]
           for _ in range(args.steps)]
    torch.cuda.synchronize()
    for i in range(args.steps):
        step(evs[i])
    torch.cuda.synchronize()
    call_us = {name: [e[i].elapsed_time(e[i + 1]) * 1e3 for e in evs]
               for i, (name, _) in enumerate(calls)}
    tot_us = [e[0].elapsed_time(e[nc]) * 1e3 for e in evs]

    # ---- cold caches: each step after a sweep over a flush buffer -----------
    # (larger than the L2s and the MALL together, read outside the timed
    # events, so no input or output of the step is cached when it starts.
    # The sweep reads, so the caches hold clean lines: a written flush buffer
    # would charge its own write-back to the step.)
    if args.flush_mb > 0:
        flush = torch.ones(args.flush_mb << 20, dtype=torch.uint8, device=dev)
        n_cold = max(1, args.steps)
        cev = [[torch.cuda.Event(enable_timing=True) for _ in range(2)] for _ in range(n_cold)]
        torch.cuda.synchronize()
        for i in range(n_cold):
            flush.sum()
            cev[i][0].record()
            step()
            cev[i][1].record()
        torch.cuda.synchronize()
        cold_us = [a.elapsed_time(b) * 1e3 for a, b in cev]
        del flush
        log("cold-cache steps: p50 %.2f us" % pct(cold_us, 50))

    # ---- the dominant kernel launched back to back on its stream ------------
    # (combine on the offsets path; the single dispatch launch on the decode
    # path, where it is the larger of the two)
    # The launches are captured in one HIP graph (DOM_GRAPH_LAUNCHES of them)
    # that is replayed between two events, so that the host's launch cost --
    # several microseconds per call from Python, more than a decode kernel
    # runs -- stays out of the per-launch figure.
    dom_name = "ll_dispatch" if args.low_latency else "combine"
    dom_fn = dict(calls)[dom_name]
    dom_g = torch.cuda.CUDAGraph()
    dside = torch.cuda.Stream()
    dside.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(dside):
        dom_fn()
    torch.cuda.current_stream().wait_stream(dside)
    torch.cuda.synchronize()
    with torch.cuda.graph(dom_g):
        for _ in range(DOM_GRAPH_LAUNCHES):
            dom_fn()
    dom_g.replay()
    dom_replays = max(1, args.steps // DOM_GRAPH_LAUNCHES)
    c0, c1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    c0.record()
    for _ in range(dom_replays):
        dom_g.replay()
    c1.record()
    torch.cuda.synchronize()
    dom_b2b_us = c0.elapsed_time(c1) / (dom_replays * DOM_GRAPH_LAUNCHES) * 1e3
    del dom_g

    # ---- the same step captured once in a HIP graph and replayed -----------
    graph_us = None
    if args.graph:
        g = torch.cuda.CUDAGraph()
        side = torch.cuda.Stream()
        side.wait_stream(torch.cuda.current_stream())
        with torch.cuda.stream(side):
            step()
        torch.cuda.current_stream().wait_stream(side)
        torch.cuda.synchronize()
        with torch.cuda.graph(g):
            for _ in range(args.graph_steps):
                step()
        for _ in range(max(1, args.warmup // args.graph_steps)):
            g.replay()
        g0, g1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        replays = max(1, args.steps // args.graph_steps)
        torch.cuda.synchronize()
        g0.record()
        for _ in range(replays):
            g.replay()
        g1.record()
        torch.cuda.synchronize()
        graph_us = g0.elapsed_time(g1) / (replays * args.graph_steps) * 1e3
        log("graph replay (%d steps per graph): %.2f us/step" % (args.graph_steps, graph_us))
        del g

    if args.low_latency:
        filled = int((lld.recv_src_token >= 0).sum().item())
        nb = ll_algorithmic_bytes(T, H, E, K, C, fp8, filled)
    elif args.dedup:
        nd = int(ddo.partition_token_offsets[-1].item())
        nb = dedup_algorithmic_bytes(T, H, E, P, K, fp8, nd)
    elif args.align:
        n_rows = int((disp.recv_src_token >= 0).sum().item())
        nb = aligned_algorithmic_bytes(T, H, E, P, K, fp8, n_rows, R)
    else:
        nb = algorithmic_bytes(T, H, E, P, K, fp8)
    value = nb["total"] / (ms_per_step * 1e-3) / 1e9

    # ---- the step beside a GEMM on another stream (CU budget use case) ------
    overlap = None
    if args.overlap_gemm:
        ga = torch.randn((4096, 7168), dtype=torch.bfloat16, device=dev)
        gb = torch.randn((7168, 2048), dtype=torch.bfloat16, device=dev)
        gc = torch.empty((4096, 2048), dtype=torch.bfloat16, device=dev)
        gs = torch.cuda.Stream()           # default priority
        n_ov = max(5, args.steps // 2)

        def gemms():
            for _ in range(n_ov):
                torch.matmul(ga, gb, out=gc)

        def steps():
            for _ in range(n_ov):
                step()

        def timed(run_steps, run_gemms):
            e0 = torch.cuda.Event(enable_timing=True)
            e1 = torch.cuda.Event(enable_timing=True)
            e2 = torch.cuda.Event(enable_timing=True)
            torch.cuda.synchronize()
            e0.record()
            gs.wait_event(e0)
            if run_gemms:
                with torch.cuda.stream(gs):
                    gemms()
            if run_steps:
                steps()
            e1.record()
            e2.record(gs)
            torch.cuda.synchronize()
            return max(e0.elapsed_time(e1), e0.elapsed_time(e2)) * 1e3 / n_ov

        timed(True, True)                  # warm-up
        g_us = timed(False, True)
        s_us = timed(True, False)
        b_us = timed(True, True)
        overlap = {"gemm": "bf16 4096x7168 @ 7168x2048 (torch.matmul) on a second stream",
                   "cu_budget": args.cu_budget, "pairs": n_ov,
                   "gemm_us": round(g_us, 2), "step_us": round(s_us, 2),
                   "both_us": round(b_us, 2),
                   "sequential_over_concurrent": round((g_us + s_us) / b_us, 3)}
        log("overlap: gemm %.1f us, step %.1f us, both %.1f us per pair" % (g_us, s_us, b_us))
        del ga, gb, gc

    # ---- copy ceiling (measured) ---------------------------------------------
    copy_gbs = None
    if not args.no_copy_ceiling:
        n = 1 << 30
        a = torch.empty(n, dtype=torch.uint8, device=dev)
        b = torch.empty(n, dtype=torch.uint8, device=dev)
        for _ in range(3):
            ep.copy(a, b)
        c0, c1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        c0.record()
        for _ in range(10):
            ep.copy(a, b)
        c1.record()
        torch.cuda.synchronize()
        copy_gbs = 2 * n * 10 / (c0.elapsed_time(c1) * 1e-3) / 1e9
        del a, b
        log("copy ceiling %.0f GB/s" % copy_gbs)

    achieved = nb[dom_name] / (dom_b2b_us * 1e-6) / 1e9
    if args.low_latency:
        kname = "ll_dispatch_kernel<%s>" % ("true" if fp8 else "false")
    else:
        kname = combine_kernel_name(T, H, K, args.cu_budget)
    roofline = {"bound": "hbm", "kernel": kname,
                "achieved": round(achieved, 1), "peak": HBM_PEAK_GBS, "unit": "GB/s",
                "frac": round(achieved / HBM_PEAK_GBS, 4),
                "traffic": measured_traffic(dom_name, args.config + ("-ll" if args.low_latency
                                                                    else "")),
                "algorithmic_bytes_per_launch": nb[dom_name],
                "avg_launch_us": round(dom_b2b_us, 2),
                "timing": "HIP events around %d replays of a HIP graph of %d back-to-back "
                          "launches on the launch stream" % (dom_replays, DOM_GRAPH_LAUNCHES),
                "avg_launch_us_in_step": round(float(np.mean(call_us[dom_name])), 2)}

    cpu = None
    if not args.no_cpu_baseline:
        cpu = cpu_baseline(case, nb["total"], args.cpu_seconds, C if args.low_latency else None,
                           args.align, args.dedup)

    def q(a):
        return {"p10": round(pct(a, 10), 2), "p50": round(pct(a, 50), 2),
                "p90": round(pct(a, 90), 2), "mean": round(float(np.mean(a)), 2)}

    result = {
        "metric": METRIC,
        "value": round(value, 1),
        "unit": "GB/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms_per_step, 5),
        "us_per_call": round(ms_per_step * 1e3, 2),
        "pct_of_hbm_peak": round(100 * value / HBM_PEAK_GBS, 2),
        "graph_replay": ({"us_per_call": round(graph_us, 2),
                          "gbs": round(nb["total"] / (graph_us * 1e-6) / 1e9, 1),
                          "steps_per_graph": args.graph_steps}
                         if graph_us else None),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "fp32",
        "io_dtypes": {"x": "bf16", "recv_x": "fp8_e4m3" if fp8 else "bf16",
                      "recv_scales": "fp32" if fp8 else None, "y": "bf16", "out": "bf16",
                      "accumulate": "fp32"},
        "data": "synthetic",
        "config": {"workload": "%s: %d tokens x %d hidden, top-%d of %d experts, %d partitions, "
                               "%s dispatch%s" % (args.config, T, H, K, E, P,
                                                  "FP8 E4M3 per-128" if fp8 else "bf16",
                                                  ", single-launch fixed capacity %d per expert"
                                                  % C if args.low_latency else ""),
                   "tokens": T, "hidden": H, "experts": E, "partitions": P, "topk": K,
                   "fp8_dispatch": fp8, "parallelism": "single GPU",
                   "cu_budget": args.cu_budget or None, "x_copies": n_x,
                   "path": "low_latency" if args.low_latency else
                           ("de-duplicated per partition" if args.dedup else
                            ("offsets, experts aligned to %d rows" % args.align if args.align else
                             ("offsets, two calls" if args.two_calls else "offsets, one call")))},
        "algorithmic_bytes": nb,
        "breakdown_us": dict({name: q(v) for name, v in call_us.items()},
                             step_with_events=q(tot_us)),
        "cold_cache_us": (dict(q(cold_us), flush_mb=args.flush_mb, steps=len(cold_us))
                          if args.flush_mb > 0 else None),
        "copy_ceiling_gbs": round(copy_gbs, 1) if copy_gbs else None,
        "pct_of_copy_ceiling": round(100 * value / copy_gbs, 2) if copy_gbs else None,
        "roofline": roofline,
        "cpu_baseline": cpu,
        "overlap": overlap,
        "device": torch.cuda.get_device_name(dev),
    }
    print(json.dumps(result), flush=True)


if __name__ == "__main__":
    main()
