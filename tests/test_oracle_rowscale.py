"""Pins for the oracle's row normalization, independent of its own code.

The arXiv abstract (mlsanity index page) names "row-normalized E8 lattice
quantization"; the reading here is that each row is divided by its RMS and
the stream keeps one f32 per row, g_r = f32(rms_r * a / 2), so that the
lattice point of 8 consecutive coordinates is the E8 point nearest to
x / (2 g_r) and the weight comes back as v * g_r (v = twice the point).

Every other transport pin goes through the oracle's own quantize_matrix, which
calls the same row-scale code; these tests do not.  They read g_r straight
out of the stream's scales section and recompute it with numpy, bit for bit:
a sequential f64 sum of squares (numpy's cumsum adds in column order), the
division by the unpadded column count, the square root, the product with the
stream's resolution a and the halving, rounded once to f32.  They then check,
for one vector of every row, that the decoded lattice point is the E8 point
nearest to x / (2 g_r) by brute-force enumeration.  An absmax statistic, a
division by the padded column count, or a dropped 1/2 all fail here.
"""
import numpy as np
import pytest
import torch

import oracle
from decode_tile_interleaved_amd import workloads as W
from test_oracle_e8 import brute_force_nearest


def stream_scales(blob):
    """(a, g[R]) read from the stream: the header's lattice resolution (f64 at
    byte 48) and the f32 scales section (its byte offset is the u64 at 72)."""
    blob = np.ascontiguousarray(blob, dtype=np.uint8)
    a = float(blob[48:56].view(np.float64)[0])
    off = int(blob[72:80].view(np.uint64)[0])
    rows = int(blob[24:32].view(np.uint64)[0])
    return a, blob[off:off + 4 * rows].view(np.float32).copy()


def numpy_scales(x64, a):
    """g_r = f32(sqrt(sum_c x[r, c]^2 / C) * a / 2), the sum in column order."""
    C = x64.shape[1]
    ss = np.cumsum(x64 * x64, axis=1)[:, -1]
    rms = np.sqrt(ss / C)
    return ((rms * a) * 0.5).astype(np.float32)


def _cases():
    g = torch.Generator().manual_seed(4242)
    ragged = (torch.randn(37, 100, generator=g) * 0.03).to(torch.bfloat16)  # 100 mod 8 = 4: padded columns
    zero = (torch.randn(24, 56, generator=g) * 0.02).to(torch.bfloat16)
    zero[7] = 0
    zero[19] = 0
    # rows with very different scales: a wrong statistic moves them apart
    spread = (torch.randn(16, 64, generator=g) * torch.logspace(-4, 1, 16).unsqueeze(1)).to(torch.float16)
    t4 = W.t4_outliers(96, 1536, 1003)  # the heavy-tailed recipe with 20-sigma outliers, at a smaller size
    return {"ragged_37x100": (ragged, 3.0), "zero_rows": (zero, 4.0), "row_spread_fp16": (spread, 5.0),
            "t4_outliers_96x1536": (t4, 2.75)}


CASES = _cases()


@pytest.mark.parametrize("name", list(CASES))
def test_stream_scales_equal_numpy_rms(name):
    t, target = CASES[name]
    blob, rc, _ = oracle.compress(t, target)
    assert rc == 0
    a, g = stream_scales(blob)
    x64 = t.to(torch.float64).numpy()
    want = numpy_scales(x64, a)
    assert np.array_equal(g.view(np.uint32), want.view(np.uint32))
    # zero rows store a zero scale and decode to exact zeros
    zero_rows = np.where(~x64.any(axis=1))[0]
    assert np.all(g[zero_rows] == 0)
    if len(zero_rows):
        v = oracle.decode_symbols(blob)
        assert not v[zero_rows].any()


@pytest.mark.parametrize("name", list(CASES))
def test_one_vector_per_row_is_the_nearest_e8_point(name):
    t, target = CASES[name]
    blob, rc, _ = oracle.compress(t, target)
    assert rc == 0
    a, g = stream_scales(blob)
    x64 = t.to(torch.float64).numpy()
    R, C = x64.shape
    Cp = (C + 7) // 8 * 8
    xp = np.zeros((R, Cp))
    xp[:, :C] = x64
    v = oracle.decode_symbols(blob).astype(np.int64)
    rng = np.random.default_rng(7)
    rows = [r for r in range(R) if g[r] != 0]
    ks = rng.integers(0, Cp // 8, size=len(rows))
    ks[0] = Cp // 8 - 1  # the padded vector at the end of a row
    U = np.stack([xp[r, 8 * k:8 * k + 8] / (2.0 * np.float64(g[r])) for r, k in zip(rows, ks)])
    best, _ = brute_force_nearest(U)
    got = np.stack([v[r, 8 * k:8 * k + 8] for r, k in zip(rows, ks)]) / 2.0
    d = ((U - got) ** 2).sum(axis=1)
    # every decoded point is an E8 point at the brute-force minimum distance
    assert np.allclose(d, best, rtol=0, atol=1e-12)


def test_plausible_slips_would_fail():
    """The numpy statistic separates the reading from its plausible
    alternatives on these inputs (absmax, padded column count, no halving)."""
    t, target = CASES["ragged_37x100"]
    blob, _, _ = oracle.compress(t, target)
    a, g = stream_scales(blob)
    x64 = t.to(torch.float64).numpy()
    C = x64.shape[1]
    padded = np.sqrt(np.cumsum(x64 * x64, axis=1)[:, -1] / ((C + 7) // 8 * 8))
    for wrong in (np.abs(x64).max(axis=1) * a * 0.5, padded * a * 0.5, np.sqrt((x64 ** 2).mean(axis=1)) * a):
        assert not np.array_equal(g, wrong.astype(np.float32))
