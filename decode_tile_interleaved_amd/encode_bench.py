"""Compression throughput: the GPU encoder (ep_compress_device) against the
host encoder (ep_compress_ex on every host thread), on the same matrices.

    python -m decode_tile_interleaved_amd.encode_bench [--reps R]

Matrices: the 4096 x 4096 BF16 row-scaled Gaussian at 4.0 bpp, and one
block of the DiT-style stack (four 3840 x 3840, 10240 x 3840, 3840 x 10240,
BF16 N(0, 0.02^2)) at 4.0 bpp.  Each call runs rate selection, the tables
and the full stream; the GPU call includes copying the stream back to host
memory.  Prints one JSON line; streams are checked equal.
"""
from __future__ import annotations

import argparse
import json
import os
import statistics
import sys
import time

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)


def main() -> int:
    ap = argparse.ArgumentParser()
    ap.add_argument("--reps", type=int, default=3)
    args = ap.parse_args()

    import numpy as np
    import torch

    from decode_tile_interleaved_amd import ep
    from decode_tile_interleaved_amd import workloads as W

    if not torch.cuda.is_available():
        print("encode_bench: no GPU visible", file=sys.stderr)
        return 1
    sets = {
        "rowscale4096_bf16_4.0": [W.make("rowscale4096_bf16_4.0")[0]],
        "dit_block_bf16_4.0": [W.dit_matrix(0, j) for j in range(len(W.DIT_SHAPES))],
    }
    out = {"metric": "compression throughput, GPU encoder vs host encoder", "unit": "Gparams/s", "target_bpp": 4.0,
           "host_threads": os.cpu_count()}
    same = True
    for name, mats in sets.items():
        numel = sum(m.numel() for m in mats)
        dev = [m.cuda() for m in mats]
        torch.cuda.synchronize()
        ep.compress_device(dev[0], 4.0)  # first call: module load
        t_gpu, t_host = [], []
        for _ in range(args.reps):
            t0 = time.perf_counter()
            pg = [ep.compress_device(d, 4.0) for d in dev]
            t_gpu.append(time.perf_counter() - t0)
            t0 = time.perf_counter()
            ph = [ep.compress(m, 4.0) for m in mats]
            t_host.append(time.perf_counter() - t0)
            same &= all(np.array_equal(a.blob, b.blob) for a, b in zip(pg, ph))
        g, h = statistics.median(t_gpu), statistics.median(t_host)
        out[name] = {"params": numel, "gpu_s": round(g, 4), "host_s": round(h, 4),
                     "gpu_gparams_s": round(numel / g / 1e9, 3), "host_gparams_s": round(numel / h / 1e9, 3),
                     "speedup": round(h / g, 1)}
    block = out["dit_block_bf16_4.0"]
    out["dit_stack_30_blocks_gpu_s"] = round(30 * block["gpu_s"], 2)
    out["dit_stack_30_blocks_host_s"] = round(30 * block["host_s"], 2)
    out["streams_equal"] = bool(same)
    print(json.dumps(out), flush=True)
    return 0 if same else 1


if __name__ == "__main__":
    sys.exit(main())
