"""Benchmark: MoE dispatch + combine on one MI355X.

One step = the whole path on one batch: ep_get_dispatch_layout ->
ep_dispatch -> ep_combine, on seeded synthetic routing and activations that
are resident in HBM before timing starts.  The default workload is the
prefill configuration (4096 tokens x 7168 hidden, top-8 of 256 experts with
group-limited gating, 64 partitions, FP8 E4M3 dispatch with per-128 scales,
bf16 weighted combine).

    python bench.py [--steps K] [--warmup W] [--config prefill|decode|...]

Prints one JSON line (last line of stdout).  `value` is the effective HBM
throughput of a step: the algorithmic bytes of the three calls (each input
read once, each output written once) divided by the measured time per step.
`roofline` reports the dominant kernel (combine) against the 8 TB/s HBM3E
peak: its algorithmic bytes per launch over its average duration, timed with
HIP events around back-to-back launches on the stream it runs on (the
per-call timing inside the step, which also holds each launch's dispatch
latency, is reported beside it); `cpu_baseline` times the CPU oracle on this
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
METRIC = "dispatch+combine µs/call and effective HBM GB/s (% peak) at 4096×7168 top-8"
TRAFFIC_FILE = os.path.join(ROOT, "profiles", "hbm_traffic.json")
KERNEL_SOURCES = {
    "combine": ["ep_combine.hip", "ep_device.h", "ep_internal.h"],
    "dispatch": ["ep_dispatch.hip", "ep_device.h", "ep_internal.h"],
    "layout": ["ep_layout.hip", "ep_device.h", "ep_internal.h"],
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


def kernel_source_hash(kernel):
    h = hashlib.sha256()
    for name in KERNEL_SOURCES[kernel]:
        with open(os.path.join(ROOT, "combine_ep_get_dispatch_amd", "csrc", name), "rb") as f:
            h.update(f.read())
    return h.hexdigest()


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


def cpu_baseline(wl_case, nbytes, seconds):
    """The CPU oracle (single-threaded C) on the same workload, repeated until
    `seconds` of CPU work have accumulated (at least one full pass)."""
    import oracle
    passes, t_total = 0, 0.0
    while True:
        t0 = time.perf_counter()
        oracle.run(wl_case.topk_idx, wl_case.x_bits, wl_case.E, wl_case.P, wl_case.fp8,
                   wl_case.y_bits, wl_case.topk_weights)
        t_total += time.perf_counter() - t0
        passes += 1
        log("cpu oracle pass %d: %.2f s total" % (passes, t_total))
        if t_total >= seconds or passes >= 40:
            break
    return {"value": round(nbytes * passes / t_total / 1e9, 3), "unit": "GB/s", "cores": 1,
            "kind": "oracle",
            "sample": "%d full pass(es) of the %s workload (T=%d), layout+dispatch+combine, "
                      "single-threaded C oracle, %.1f s" % (passes, wl_case.name, wl_case.T,
                                                           t_total),
            "us_per_step": round(t_total / passes * 1e6, 1)}


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=50)
    ap.add_argument("--warmup", type=int, default=10)
    ap.add_argument("--config", default="prefill")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--cpu-seconds", type=float, default=10.0)
    ap.add_argument("--no-copy-ceiling", action="store_true")
    ap.add_argument("--graph", action="store_true",
                    help="also time the step captured in a HIP graph and replayed")
    args = ap.parse_args()

    world = int(os.environ.get("WORLD_SIZE", "1"))
    if args.gpus != 1 or world != 1:
        print("bench.py measures one GPU only: this build models the all-to-all's "
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
    idx = torch.from_numpy(case.topk_idx).to(dev)
    x = torch.from_numpy(case.x_bits.view(np.int16)).to(dev).view(torch.bfloat16)
    y = torch.from_numpy(case.y_bits.view(np.int16)).to(dev).view(torch.bfloat16)
    w = torch.from_numpy(case.topk_weights).to(dev)
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
    out = torch.empty((T, H), dtype=torch.bfloat16, device=dev)
    torch.cuda.synchronize()

    def step(ev=None):
        if ev is not None:
            ev[0].record()
        ep.get_dispatch_layout(idx, E, P, workspace=ws, out=lay)
        if ev is not None:
            ev[1].record()
        ep.dispatch(x, idx, E, P, ws, fp8=fp8, out=disp)
        if ev is not None:
            ev[2].record()
        ep.combine(y, disp.dst_row, w, out=out)
        if ev is not None:
            ev[3].record()

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
    evs = [[torch.cuda.Event(enable_timing=True) for _ in range(4)] for _ in range(args.steps)]
    torch.cuda.synchronize()
    for i in range(args.steps):
        step(evs[i])
    torch.cuda.synchronize()
    lay_us = [e[0].elapsed_time(e[1]) * 1e3 for e in evs]
    dis_us = [e[1].elapsed_time(e[2]) * 1e3 for e in evs]
    com_us = [e[2].elapsed_time(e[3]) * 1e3 for e in evs]
    tot_us = [e[0].elapsed_time(e[3]) * 1e3 for e in evs]

    # ---- combine launched back to back on its stream: its kernel duration ---
    c0, c1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    c0.record()
    for _ in range(args.steps):
        ep.combine(y, disp.dst_row, w, out=out)
    c1.record()
    torch.cuda.synchronize()
    com_b2b_us = c0.elapsed_time(c1) / args.steps * 1e3

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
            step()
        for _ in range(args.warmup):
            g.replay()
        g0, g1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        torch.cuda.synchronize()
        g0.record()
        for _ in range(args.steps):
            g.replay()
        g1.record()
        torch.cuda.synchronize()
        graph_us = g0.elapsed_time(g1) / args.steps * 1e3
        log("graph replay: %.2f us/step" % graph_us)
        del g

    nb = algorithmic_bytes(T, H, E, P, K, fp8)
    value = nb["total"] / (ms_per_step * 1e-3) / 1e9

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

    com_avg = float(np.mean(com_us))
    achieved = nb["combine"] / (com_b2b_us * 1e-6) / 1e9
    roofline = {"bound": "hbm", "kernel": "combine_kernel<%d>" % K if K in (1, 2, 4, 6, 8)
                else "combine_kernel<0>",
                "achieved": round(achieved, 1), "peak": HBM_PEAK_GBS, "unit": "GB/s",
                "frac": round(achieved / HBM_PEAK_GBS, 4),
                "traffic": measured_traffic("combine", args.config),
                "algorithmic_bytes_per_launch": nb["combine"],
                "avg_launch_us": round(com_b2b_us, 2),
                "timing": "HIP events around %d back-to-back launches on the launch stream"
                          % args.steps,
                "avg_launch_us_in_step": round(com_avg, 2)}

    cpu = None
    if not args.no_cpu_baseline:
        cpu = cpu_baseline(case, nb["total"], args.cpu_seconds)

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
                          "gbs": round(nb["total"] / (graph_us * 1e-6) / 1e9, 1)}
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
                               "%s dispatch" % (args.config, T, H, K, E, P,
                                                "FP8 E4M3 per-128" if fp8 else "bf16"),
                   "tokens": T, "hidden": H, "experts": E, "partitions": P, "topk": K,
                   "fp8_dispatch": fp8, "parallelism": "single GPU"},
        "algorithmic_bytes": nb,
        "breakdown_us": {"layout": q(lay_us), "dispatch": q(dis_us), "combine": q(com_us),
                         "step_with_events": q(tot_us)},
        "copy_ceiling_gbs": round(copy_gbs, 1) if copy_gbs else None,
        "pct_of_copy_ceiling": round(100 * value / copy_gbs, 2) if copy_gbs else None,
        "roofline": roofline,
        "cpu_baseline": cpu,
        "device": torch.cuda.get_device_name(dev),
    }
    print(json.dumps(result), flush=True)


if __name__ == "__main__":
    main()
