"""Relative L2 weight error of the lattice-rANS codec at 4 bits per
parameter next to NF4 on the same synthetic matrices (context for the
abstract's "about 24% lower relative L2 weight error than NF4" on
Z-Image-Turbo's weights, which are not available here).

NF4 is built from its published definition (QLoRA, "4-bit NormalFloat"):
quantiles of N(0, 1) scaled to [-1, 1], with an exact zero obtained by
taking 2^(k-1) levels for the negative half and 2^(k-1) + 1 for the
positive half and dropping the duplicated zero; weights are scaled by the
absolute maximum of their block of 64 and rounded to the nearest level.
The quantile probabilities are this script's reading: level j of a half is
the normal quantile at probability 1/2 + (j / n) (p_max - 1/2), n levels
past zero, then each half divided by its largest level.  p_max = 0.94
minimizes the round-trip error of N(0, 1) blocks of 64 over [0.90, 0.99]
(8.95% there; 9.25% at 0.9675, 10.9% at 0.99), so NF4 gets its best case.
Storage: 4 bits per weight plus one absmax per block (16 bits: 4.25 bpp;
32 bits: 4.5 bpp).

    python -m decode_tile_interleaved_amd.nf4_compare

Needs a GPU (the codec's decoder is the gfx950 kernel).  Prints one JSON line.
"""
from __future__ import annotations

import json
import os
import sys
from statistics import NormalDist

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

BLOCK = 64
P_MAX = 0.94  # the probability of the outermost level (see above)


def nf4_levels() -> list[float]:
    """The 16 NF4 levels in [-1, 1], ascending, with an exact zero."""
    nd = NormalDist()
    p_max = P_MAX

    def half(n: int) -> list[float]:
        q = [nd.inv_cdf(0.5 + (j / n) * (p_max - 0.5)) for j in range(1, n + 1)]
        return [v / q[-1] for v in q]

    pos = half(8)   # 2^(k-1) + 1 levels with zero
    neg = half(7)   # 2^(k-1) levels with zero
    return sorted([-v for v in neg] + [0.0] + pos)


def nf4_round_trip(w, scale_dtype):
    """w (float32 tensor, numel a multiple of 64) through NF4: blockwise
    absmax (stored in scale_dtype), nearest level, back to float32."""
    import torch
    lv = torch.tensor(nf4_levels(), dtype=torch.float32)
    b = w.reshape(-1, BLOCK)
    amax = b.abs().amax(dim=1, keepdim=True).to(scale_dtype).to(torch.float32)
    safe = torch.where(amax > 0, amax, torch.ones_like(amax))
    u = b / safe
    idx = (u.unsqueeze(-1) - lv).abs().argmin(dim=-1)
    return (lv[idx] * amax).reshape(w.shape)


def main() -> int:
    import torch

    from decode_tile_interleaved_amd import ep
    from decode_tile_interleaved_amd import workloads as W

    if not torch.cuda.is_available():
        print("nf4_compare: no GPU visible", file=sys.stderr)
        return 1
    cases = {
        "rowscale4096_bf16": W.make("rowscale4096_bf16_4.0")[0],
        "t4outlier3072x12288_bf16": W.make("t4outlier3072x12288_bf16_2.75")[0],
        "dit_3840x3840_bf16": W.dit_matrix(0, 0),
        "dit_10240x3840_bf16": W.dit_matrix(0, 4),
    }
    out = {"metric": "relative L2 weight error at about 4 bits per parameter", "nf4_levels": [round(v, 4) for v in nf4_levels()],
           "nf4_block": BLOCK, "data": "synthetic"}
    for name, x in cases.items():
        xf = x.float()
        ref = xf.double()
        p = ep.compress(x, 4.0).to("cuda")
        y = ep.decompress(p).cpu().double()
        ours = ((y - ref).norm() / ref.norm()).item()
        nf16 = ((nf4_round_trip(xf, torch.float16).double() - ref).norm() / ref.norm()).item()
        nf32 = ((nf4_round_trip(xf, torch.float32).double() - ref).norm() / ref.norm()).item()
        out[name] = {"codec_bpp": round(p.actual_bpp, 4), "codec_rel_l2": round(ours, 5),
                     "nf4_f16_scales_bpp": 4.25, "nf4_f16_scales_rel_l2": round(nf16, 5),
                     "nf4_f32_scales_bpp": 4.5, "nf4_f32_scales_rel_l2": round(nf32, 5),
                     "codec_vs_nf4_f16": round(1.0 - ours / nf16, 4)}
    print(json.dumps(out), flush=True)
    return 0


if __name__ == "__main__":
    sys.exit(main())
