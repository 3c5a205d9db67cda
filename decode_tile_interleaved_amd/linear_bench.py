"""Decode-then-GEMM timing for one block of a DiT-style transformer.

The Compressed Linear usage page decodes compressed weights on the fly in
front of each linear layer of a prefill pass.  This measures that pattern on
one GPU with the fused decoder and the platform GEMM (torch.mm, which
calls hipBLASLt):

* GEMM only: the six linears of a block, Y = X @ W^T, with every weight
  resident in BF16;
* decode + GEMM: each weight decoded from its stream into one scratch buffer
  right before its GEMM;
* decode ahead: the same on two streams with two scratch buffers: weight j+1
  is decoded on a second stream while the GEMM of weight j runs;
* fused: ep_linear on streams in the blocks layout (64 x 64 weight blocks),
  each block decoded into LDS and multiplied there by the BF16 matrix cores;
  no decoded weight reaches global memory.

Shapes: four 3840 x 3840 projections, 10240 x 3840 (up) and 3840 x 10240
(down), as (out, in); X is 4096 x 3840 (4096 x 10240 for the down
projection).  Weights N(0, 0.02^2), seeds 5000 + j; activations N(0, 1), seed
4999; weights compressed at 4.0 bits per parameter by the library's encoder.

    python -m decode_tile_interleaved_amd.linear_bench [--steps K] [--blocks B] [--tokens M]

Prints one JSON line.
"""
from __future__ import annotations

import argparse
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)


def main() -> int:
    ap = argparse.ArgumentParser()
    ap.add_argument("--steps", type=int, default=50, help="timed replays of the block")
    ap.add_argument("--warmup", type=int, default=5)
    ap.add_argument("--blocks", type=int, default=4,
                    help="distinct blocks, replayed in turn, so that weights and streams come from HBM")
    ap.add_argument("--tokens", type=int, default=4096, help="rows of X (prefill tokens)")
    args = ap.parse_args()

    import torch

    from decode_tile_interleaved_amd import ep
    from decode_tile_interleaved_amd import workloads as W

    if not torch.cuda.is_available():
        print("linear_bench: no GPU visible", file=sys.stderr)
        return 1
    dev = torch.device("cuda:0")
    target = 4.0
    M = args.tokens
    x_in = W.dit_activation(3840)[:M].contiguous().to(dev)
    x_down = W.dit_activation(10240)[:M].contiguous().to(dev)
    blocks = []
    enc_s = 0.0
    for b in range(args.blocks):
        mats = []
        for j in range(len(W.DIT_SHAPES)):
            w = W.dit_matrix(b, j)
            t0 = time.perf_counter()
            p = ep.compress(w, target)
            enc_s += time.perf_counter() - t0
            pb = ep.compress(w, target, layout=ep.LAYOUT_BLOCKS)
            mats.append((w.to(dev), p.to(dev), pb.to(dev)))
        blocks.append(mats)
    scratch = torch.empty(max(r * c for r, c in W.DIT_SHAPES), dtype=torch.bfloat16, device=dev)
    scratch2 = [torch.empty(max(r * c for r, c in W.DIT_SHAPES), dtype=torch.bfloat16, device=dev) for _ in range(2)]
    outs = [torch.empty(M, r, dtype=torch.bfloat16, device=dev) for r, _ in W.DIT_SHAPES]
    stream = torch.cuda.Stream()
    side = torch.cuda.Stream()

    def x_for(j):
        return x_down if W.DIT_SHAPES[j][1] == 10240 else x_in

    def gemm_block(b):
        for j, (w, _, _) in enumerate(blocks[b]):
            torch.mm(x_for(j), w.t(), out=outs[j])

    def fused_block(b):
        for j, (_, _, pb) in enumerate(blocks[b]):
            ep.linear(pb, x_for(j), out=outs[j], stream=stream)

    def decode_gemm_block(b):
        for j, (_, p, _) in enumerate(blocks[b]):
            r, c = W.DIT_SHAPES[j]
            w = scratch[: r * c].view(r, c)
            ep.decompress(p, out=w, stream=stream)
            torch.mm(x_for(j), w.t(), out=outs[j])

    def decode_ahead_run(b):
        mats = blocks[b]
        gemm_done = []
        for j, (_, p, _) in enumerate(mats):
            r, c = W.DIT_SHAPES[j]
            w = scratch2[j % 2][: r * c].view(r, c)
            with torch.cuda.stream(side):
                if j >= 2:
                    side.wait_event(gemm_done[j - 2])
                else:
                    side.wait_stream(stream)
                ep.decompress(p, out=w, stream=side)
                e = torch.cuda.Event()
                e.record(side)
            # the GEMM of weight j waits for its decode; decodes of j + 1 (and
            # j + 2 after this GEMM) proceed meanwhile
            stream.wait_event(e)
            torch.mm(x_for(j), w.t(), out=outs[j])
            g = torch.cuda.Event()
            g.record(stream)
            gemm_done.append(g)
        # join the side stream back before the block ends
        stream.wait_stream(side)

    def decode_block(b):
        for j, (_, p, _) in enumerate(blocks[b]):
            r, c = W.DIT_SHAPES[j]
            ep.decompress(p, out=scratch[: r * c].view(r, c), stream=stream)

    # the decoded weights equal the resident ones (rANS is lossless up to the
    # lattice; the resident copy is the decoder's own output here)
    for b in range(args.blocks):
        with torch.cuda.stream(stream):
            for j, (w, p, pb) in enumerate(blocks[b]):
                blocks[b][j] = (ep.decompress(p, stream=stream), p, pb)
    stream.synchronize()

    def timed(fn):
        # eager pass first: the GEMM library creates its handle and picks its
        # kernels outside the capture
        with torch.cuda.stream(stream):
            for i in range(args.blocks):
                fn(i)
        stream.synchronize()
        g = torch.cuda.CUDAGraph()
        with torch.cuda.graph(g, stream=stream):
            for i in range(args.blocks):
                fn(i)
        with torch.cuda.stream(stream):
            for _ in range(args.warmup):
                g.replay()
        # settle the clocks, then time
        t_settle = time.perf_counter()
        with torch.cuda.stream(stream):
            while time.perf_counter() - t_settle < 0.3:
                g.replay()
                stream.synchronize()
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        with torch.cuda.stream(stream):
            e0.record(stream)
            for _ in range(args.steps):
                g.replay()
            e1.record(stream)
        torch.cuda.synchronize()
        return e0.elapsed_time(e1) / (args.steps * args.blocks)  # ms per block

    t_gemm = timed(gemm_block)
    t_dec = timed(decode_block)
    t_both = timed(decode_gemm_block)
    t_ahead = timed(decode_ahead_run)
    t_fused = timed(fused_block)
    # the fused product against X times its own stream's decoded weights
    # (FP32 accumulation in another order, each rounded to BF16: a few ulps)
    with torch.cuda.stream(stream):
        fused_block(0)
        fused_out = [o.float() for o in outs]
        ref_f = [torch.mm(x_for(j).float(), ep.decompress(pb, stream=stream).float().t())
                 for j, (_, _, pb) in enumerate(blocks[0])]
    stream.synchronize()
    fused_rel = max(float((o - r).abs().max() / r.abs().max()) for o, r in zip(fused_out, ref_f))
    with torch.cuda.stream(stream):
        decode_ahead_run(0)
        ref2 = [torch.mm(x_for(j), w.t()) for j, (w, _, _) in enumerate(blocks[0])]
    torch.cuda.synchronize()
    same_ahead = all(torch.equal(o, r) for o, r in zip(outs, ref2))
    # the decoded-then-multiplied result equals the product with the decoded
    # weight held resident
    with torch.cuda.stream(stream):
        decode_gemm_block(0)
        ref = [torch.mm(x_for(j), w.t()) for j, (w, _, _) in enumerate(blocks[0])]
    stream.synchronize()
    same = all(torch.equal(o, r) for o, r in zip(outs, ref))

    flops = sum(2 * M * r * c for r, c in W.DIT_SHAPES)
    params = sum(r * c for r, c in W.DIT_SHAPES)
    stream_bytes = sum(p.nbytes for _, p, _ in blocks[0])
    blocks_bytes = sum(pb.nbytes for _, _, pb in blocks[0])
    line = {
        "metric": f"DiT block prefill (6 linears, {M} tokens): fused decode+MFMA and decode + GEMM vs GEMM with "
                  "resident BF16 weights",
        "unit": "ms per block",
        "gemm_only_ms": round(t_gemm, 4),
        "decode_only_ms": round(t_dec, 4),
        "decode_plus_gemm_ms": round(t_both, 4),
        "decode_overhead_pct": round(100.0 * (t_both - t_gemm) / t_gemm, 2),
        "decode_ahead_ms": round(t_ahead, 4),
        "decode_ahead_overhead_pct": round(100.0 * (t_ahead - t_gemm) / t_gemm, 2),
        "decode_ahead_outputs_equal": same_ahead,
        "fused_ms": round(t_fused, 4),
        "fused_overhead_pct": round(100.0 * (t_fused - t_gemm) / t_gemm, 2),
        "fused_tflops": round(flops / (t_fused * 1e-3) / 1e12, 1),
        "fused_max_rel_diff": fused_rel,
        "blocks_stream_bytes": blocks_bytes,
        "blocks_actual_bpp": round(8 * blocks_bytes / params, 4),
        "tokens": M,
        "gemm_tflops": round(flops / (t_gemm * 1e-3) / 1e12, 1),
        "decode_gparams_s": round(params / (t_dec * 1e-3) / 1e9, 1),
        "weights_bf16_bytes": 2 * params,
        "weights_stream_bytes": stream_bytes,
        "actual_bpp": round(8 * stream_bytes / params, 4),
        "outputs_equal": same,
        "blocks": args.blocks,
        "steps": args.steps,
        "encode_s_per_block": round(enc_s / args.blocks, 3),
        "data": "synthetic",
    }
    print(json.dumps(line), flush=True)
    return 0 if same and same_ahead else 1


if __name__ == "__main__":
    sys.exit(main())
