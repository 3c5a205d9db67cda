#!/usr/bin/env python3
"""Decode-throughput benchmark for the fused lattice-rANS tile decoder.

A step is one fused decode (every tile of one compressed matrix, decoded and
reconstructed into its container) with the stream already resident in HBM.
Prints one JSON line.

  python bench.py [--gpus 1] [--steps K] [--warmup W] [--workload NAME]

Timing:
  * warmup: W untimed decodes, then untimed decodes for --settle-ms (default
    300 ms) so that the GPU clocks have ramped up before the timed region;
  * steps: K decodes captured in one HIP graph and replayed once between
    device synchronizations; `value` is numel * K / that wall time (whole-job
    throughput, host launch included).  The decodes rotate over enough
    stream/output copies (> 2x the 256 MB MALL) that each decode reads and
    writes HBM, not the Infinity Cache;
  * kernel duration (roofline): HIP events on the launch stream around
    back-to-back replays of that graph, at least --roofline-launches (200)
    launches in all, divided by the launch count.  One replay of a few
    launches would also time the gap before the graph's first kernel, which
    rocprof's per-kernel durations do not contain;
  * fill_us: torch's fill kernel writing the same outputs in the same
    rotation, timed the same way -- the cost of the output bytes alone;
  * cpu_baseline: the CPU oracle's decoder on the same stream, tiles split
    over the host cores the process may use, at most the 16 a GPU's share of
    the host holds (and on one thread, as cpu_baseline_1thread).
"""
from __future__ import annotations

import argparse
import hashlib
import json
import math
import os
import statistics
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

METRIC = "decoded Gparams/s + achieved HBM GB/s vs peak, 4096x4096 BF16 @ 4.0 bpp"
PEAK_HBM_GBPS = 8000.0
MALL_BYTES = 256 << 20
TRAFFIC_FILE = os.path.join(ROOT, "profiles", "ep_decode_bf16_4096x4096_traffic.json")
DEFAULT_WORKLOAD = "rowscale4096_bf16_4.0"  # the workload the counters in TRAFFIC_FILE were taken on
KERNEL_SRC = os.path.join(ROOT, "decode_tile_interleaved_amd", "csrc", "ep_decode.hip")


def kernel_source_hash() -> str:
    return hashlib.sha256(open(KERNEL_SRC, "rb").read()).hexdigest()[:16]


def measured_traffic(workload: str):
    """HBM bytes per launch from committed rocprofv3 counter runs, if they
    were taken on the current kernel source and on this workload (the
    counters cover the default 4096x4096 BF16 workload only)."""
    if workload != DEFAULT_WORKLOAD:
        return None
    try:
        d = json.load(open(TRAFFIC_FILE))
    except (OSError, ValueError):
        return None
    if d.get("kernel_source_sha256_16") != kernel_source_hash():
        return None
    return d.get("hbm_bytes_per_launch")


def cpu_baseline(blob, numel: int):
    """The oracle's decoder on the host cores: on every core the process may
    use (tiles split into contiguous ranges, one thread each), and on one
    thread.  Median of 3 whole-stream decodes each, reconstruction included."""
    import oracle
    available = len(os.sched_getaffinity(0))
    cores = min(16, available)  # the host cores one GPU's share of the box holds

    def median_s(fn):
        runs = []
        for _ in range(3):
            t0 = time.perf_counter()
            fn()
            runs.append(time.perf_counter() - t0)
        return statistics.median(runs)

    t_all = median_s(lambda: oracle.decompress_raw_threads(blob, cores))
    t_one = median_s(lambda: oracle.decompress_raw(blob))
    sample = f"whole stream ({numel} params), median of 3 decodes incl. reconstruction"
    return ({"value": round(numel / t_all / 1e9, 5), "unit": "Gparams/s", "cores": cores, "kind": "oracle",
             "cores_available": available, "sample": sample + f", tiles split over {cores} threads"},
            {"value": round(numel / t_one / 1e9, 5), "unit": "Gparams/s", "cores": 1, "kind": "oracle",
             "sample": sample + ", one thread"})


def main() -> int:
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=200)
    ap.add_argument("--warmup", type=int, default=20)
    ap.add_argument("--workload", default=DEFAULT_WORKLOAD)
    ap.add_argument("--settle-ms", type=float, default=300.0,
                    help="untimed decodes after the warmup steps until the clocks settle (milliseconds)")
    ap.add_argument("--roofline-launches", type=int, default=200,
                    help="launches timed back to back for the roofline's kernel duration")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--eager-only", action="store_true", help="skip the graph replay (profiling runs)")
    ap.add_argument("--copy-calibration", type=int, default=0, metavar="MIB",
                    help="only run a plain device copy of MIB MiB (steps times), to calibrate HBM byte counters")
    args = ap.parse_args()
    if args.gpus != 1:
        print(f"bench.py: this decoder is benchmarked on one GPU; --gpus {args.gpus} is not supported "
              "(tiles decode independently, so more GPUs would each decode their own matrices)", file=sys.stderr)
        return 2

    import numpy as np
    import torch

    from decode_tile_interleaved_amd import ep
    from decode_tile_interleaved_amd import workloads as W

    if not torch.cuda.is_available():
        print("bench.py: no GPU visible", file=sys.stderr)
        return 1
    dev = torch.device("cuda:0")
    if args.copy_calibration:
        n = args.copy_calibration << 20
        src = torch.empty(n, dtype=torch.uint8, device=dev).fill_(7)
        dst = torch.empty(n, dtype=torch.uint8, device=dev)
        torch.cuda.synchronize()
        for _ in range(args.steps):
            dst.copy_(src)
        torch.cuda.synchronize()
        print(json.dumps({"copy_calibration_bytes": n, "steps": args.steps}), flush=True)
        return 0
    x, target = W.make(args.workload)
    rows, cols = x.shape
    numel = rows * cols
    t0 = time.perf_counter()
    p = ep.compress(x, target)
    encode_s = time.perf_counter() - t0
    out_bytes = numel * x.element_size()
    alg_bytes = p.nbytes + out_bytes  # stream read once + reconstruction written once

    # resident copies, rotated so that each decode misses the MALL
    copies = max(2, math.ceil(2 * MALL_BYTES / alg_bytes))
    blobs = [torch.from_numpy(p.blob).to(dev) for _ in range(copies)]
    outs = [torch.empty(rows, cols, dtype=x.dtype, device=dev) for _ in range(copies)]
    packs = [ep.Packed(blob=p.blob, status=p.status, shape=p.shape, dtype=p.dtype, dev=b) for b in blobs]
    stream = torch.cuda.Stream()

    def step(i):
        ep.decompress(packs[i % copies], out=outs[i % copies], stream=stream)

    with torch.cuda.stream(stream):
        for i in range(args.warmup):
            step(i)
    stream.synchronize()

    # per-launch event pairs around eager launches (context: these include
    # each launch's event overhead, which back-to-back replay does not)
    ev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in range(args.steps)]
    with torch.cuda.stream(stream):
        for i in range(args.steps):
            ev[i][0].record(stream)
            step(i)
            ev[i][1].record(stream)
    stream.synchronize()
    eager_ms = statistics.mean(a.elapsed_time(b) for a, b in ev)

    # timed region: K decodes replayed from one graph, bracketed by HIP events
    # on the launch stream and by device synchronization
    t_start, t_end = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)

    # GPU clocks ramp up over tens of milliseconds of sustained work; right
    # before the timed region, keep the device busy with untimed decodes until
    # they have settled, so that the timed region measures steady-state
    # throughput
    def settle(run):
        if args.settle_ms <= 0:
            return 0.0
        t_settle = time.perf_counter()
        with torch.cuda.stream(stream):
            while time.perf_counter() - t_settle < args.settle_ms * 1e-3:
                run()
                stream.synchronize()
        return time.perf_counter() - t_settle

    def eager_block():
        for i in range(args.steps):
            step(i)

    if args.eager_only:
        settle_s = settle(eager_block)
        torch.cuda.synchronize()
        t0 = time.perf_counter()
        with torch.cuda.stream(stream):
            t_start.record(stream)
            for i in range(args.steps):
                step(i)
            t_end.record(stream)
        torch.cuda.synchronize()
        wall = time.perf_counter() - t0
    else:
        g = torch.cuda.CUDAGraph()
        with torch.cuda.graph(g, stream=stream):
            for i in range(args.steps):
                step(i)
        with torch.cuda.stream(stream):
            g.replay()
        settle_s = settle(g.replay)
        torch.cuda.synchronize()
        t0 = time.perf_counter()
        with torch.cuda.stream(stream):
            t_start.record(stream)
            g.replay()
            t_end.record(stream)
        torch.cuda.synchronize()
        wall = time.perf_counter() - t0
    region_kernel_ms = t_start.elapsed_time(t_end) / args.steps  # includes the gap before the graph's first kernel
    # roofline: the same graph replayed back to back until at least
    # --roofline-launches decodes have run between one pair of events
    kernel_ms = region_kernel_ms
    launches = args.steps
    if not args.eager_only:
        reps = max(1, math.ceil(args.roofline_launches / args.steps))
        r0, r1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        with torch.cuda.stream(stream):
            r0.record(stream)
            for _ in range(reps):
                g.replay()
            r1.record(stream)
        torch.cuda.synchronize()
        launches = reps * args.steps
        kernel_ms = r0.elapsed_time(r1) / launches
    ms_per_step = wall * 1e3 / args.steps

    # context only: the same decodes on one resident stream/output (warm
    # caches); the headline above rotates copies so that each decode misses
    # the MALL
    warm_ms = None
    if not args.eager_only:
        gw = torch.cuda.CUDAGraph()
        with torch.cuda.graph(gw, stream=stream):
            for i in range(args.steps):
                ep.decompress(packs[0], out=outs[0], stream=stream)
        with torch.cuda.stream(stream):
            gw.replay()
        w0, w1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        with torch.cuda.stream(stream):
            w0.record(stream)
            gw.replay()
            w1.record(stream)
        torch.cuda.synchronize()
        warm_ms = w0.elapsed_time(w1) / args.steps

    # context only: torch's fill kernel writing the same output copies in the
    # same rotation, timed like kernel_us -- what the output bytes alone cost
    # to write on this machine, the floor under a decode that must write them
    fill_ms = None
    if not args.eager_only:
        gf = torch.cuda.CUDAGraph()
        with torch.cuda.graph(gf, stream=stream):
            for i in range(args.steps):
                outs[i % copies].fill_(1)
        with torch.cuda.stream(stream):
            gf.replay()
        reps = max(1, math.ceil(args.roofline_launches / args.steps))
        f0, f1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        with torch.cuda.stream(stream):
            f0.record(stream)
            for _ in range(reps):
                gf.replay()
            f1.record(stream)
        torch.cuda.synchronize()
        fill_ms = f0.elapsed_time(f1) / (reps * args.steps)

    # the last decode of each copy must equal a fresh eager decode
    with torch.cuda.stream(stream):
        for i in range(min(copies, args.steps)):
            step(i)
    ref = ep.decompress(packs[0], stream=stream)
    stream.synchronize()
    for o in outs[: min(copies, args.steps)]:
        assert torch.equal(o.view(torch.int16 if o.element_size() == 2 else torch.int8),
                           ref.view(torch.int16 if ref.element_size() == 2 else torch.int8))
    rel_l2 = ((ref.double() - x.double().to(dev)).norm() / x.double().to(dev).norm()).item()
    rel_l2_weights = None
    if args.workload.startswith("absmax"):
        # 8-bit codes: also against the N(0,1) weights the codes stand for
        # (decoded code times the row's code scale)
        w, scale = W.absmax_weights(rows, cols, W.WORKLOADS[args.workload][4],
                                    "int8" if x.dtype == torch.int8 else "fp8")
        wd = w.double().to(dev)
        rel_l2_weights = ((ref.double() * scale.double().to(dev) - wd).norm() / wd.norm()).item()

    # context only: host time per enqueued decode (Python call included),
    # ep_decompress (checks the stream and sizes the launch on every call)
    # against a decode plan made once
    def host_us(call, n=200):
        stream.synchronize()
        t = time.perf_counter()
        with torch.cuda.stream(stream):
            for i in range(n):
                call(i)
        dt = time.perf_counter() - t
        stream.synchronize()
        return dt * 1e6 / n

    plans = [ep.plan(pk) for pk in packs]
    host_decompress_us = host_us(step)
    host_plan_us = host_us(lambda i: plans[i % copies].decompress(out=outs[i % copies], stream=stream))
    with torch.cuda.stream(stream):
        for i in range(min(copies, args.steps)):
            plans[i % copies].decompress(out=outs[i % copies], stream=stream)
    ref_plan = plans[0].decompress(stream=stream)
    stream.synchronize()

    vw = torch.int16 if ref.element_size() == 2 else torch.int8
    for o in outs[: min(copies, args.steps)] + [ref_plan]:
        assert torch.equal(o.view(vw), ref.view(vw))

    achieved = alg_bytes / (kernel_ms * 1e-3) / 1e9
    info = ep.blob_info(p.blob)
    traffic = measured_traffic(args.workload)
    line = {
        "metric": METRIC,
        "value": round(numel / (ms_per_step * 1e-3) / 1e9, 3),
        "unit": "Gparams/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms_per_step, 5),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "u32+f32",
        "data": "synthetic",
        "config": {"workload": args.workload, "rows": rows, "cols": cols, "container": str(x.dtype).split(".")[-1],
                   "target_bpp": target, "actual_bpp": round(p.actual_bpp, 5), "stream_bytes": p.nbytes,
                   "tile": f"{info['tile_vecs']} E8 vectors ({8 * info['tile_vecs']} coords), {info['n_states']} rANS states",
                   "mall_rotation_copies": copies},
        "roofline": {"bound": "hbm", "achieved": round(achieved, 1), "peak": PEAK_HBM_GBPS, "unit": "GB/s",
                     "frac": round(achieved / PEAK_HBM_GBPS, 4), "traffic": traffic},
        "kernel_us": round(kernel_ms * 1e3, 3),
        "kernel_us_launches": launches,
        "kernel_us_timed_region": round(region_kernel_ms * 1e3, 3),
        "kernel_us_eager_events": round(eager_ms * 1e3, 3),
        "kernel_us_warm": round(warm_ms * 1e3, 3) if warm_ms is not None else None,
        "fill_us": round(fill_ms * 1e3, 3) if fill_ms is not None else None,
        "fill_gbps": round(out_bytes / (fill_ms * 1e-3) / 1e9, 1) if fill_ms is not None else None,
        "clock_settle_s": round(settle_s, 3),
        "hbm_gbps_per_step": round(alg_bytes / (ms_per_step * 1e-3) / 1e9, 1),
        "rel_l2": round(rel_l2, 5),
        "rel_l2_vs_weights": round(rel_l2_weights, 5) if rel_l2_weights is not None else None,
        "encode_s": round(encode_s, 3),
        "host_us_per_call": {"ep_decompress": round(host_decompress_us, 2),
                             "ep_plan_decompress": round(host_plan_us, 2)},
    }
    if not args.no_cpu_baseline:
        line["cpu_baseline"], line["cpu_baseline_1thread"] = cpu_baseline(p.blob, numel)
    print(json.dumps(line), flush=True)
    return 0


if __name__ == "__main__":
    sys.exit(main())
