"""GPU parity of the blocks-layout decode and of the fused linear (ep_linear).

Streams come from the ORACLE (blocks layout, 64 x 64 weight blocks).  Checks:
  * ep_decode_symbols / ep_decompress of a blocks stream against the oracle's
    decode: symbols bit-exact, BF16 weights bit-exact;
  * ep_linear's Y = X W^T against the product of X with the ORACLE-decoded
    W, computed in float64 on the CPU.  Every product of two BF16 values is
    exact in FP32, so the only error is the FP32 accumulation: recursive
    summation of K terms errs by at most gamma_K * sum_k |x_k w_k| with
    gamma_K = K u / (1 - K u), u = 2^-24, which is the bound the FP32
    output is held to.  A BF16 output additionally carries its own rounding
    (half an ulp of |Y|, 2^-9 |Y|).
"""
import math

import numpy as np
import pytest
import torch

import oracle
from decode_tile_interleaved_amd import ep
from decode_tile_interleaved_amd import workloads as W

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def need_gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    ep.lib()


def blocks_stream(rows, cols, target, seed, std=0.02):
    """An oracle stream in the blocks layout; target 0: a fixed resolution
    (matrices too small for any target to pay for the stream's metadata)."""
    x = W.gaussian(rows, cols, std, seed=seed, dtype=torch.bfloat16)
    if target:
        blob, rc, _ = oracle.compress(x, target, layout=oracle.LAYOUT_BLOCKS)
    else:
        blob, rc, _ = oracle.compress(x, 4.0, fixed_a=0.1, layout=oracle.LAYOUT_BLOCKS)
    assert rc == 0, rc
    assert oracle.info(blob)["layout"] == oracle.LAYOUT_BLOCKS
    return x, blob


def oracle_weights(blob) -> np.ndarray:
    """The oracle's BF16 reconstruction as float64."""
    raw = oracle.decompress_raw(blob)  # uint16 BF16 bit patterns
    return (raw.astype(np.uint32) << 16).view(np.float32).astype(np.float64)


def gamma(k: int) -> float:
    u = 2.0 ** -24
    return k * u / (1.0 - k * u)


def check_linear(y: torch.Tensor, x: torch.Tensor, w64: np.ndarray, rows_idx=None, what=""):
    """y (m x N, on the GPU) against X W^T in float64 on the rows rows_idx."""
    x64 = x.float().double().numpy()
    if rows_idx is not None:
        x64 = x64[rows_idx]
    ref = x64 @ w64.T
    mag = np.abs(x64) @ np.abs(w64).T
    got = y.float().cpu().double().numpy()
    if rows_idx is not None:
        got = got[rows_idx]
    K = w64.shape[1]
    tol = gamma(K) * mag + 1e-30
    if y.dtype == torch.bfloat16:
        tol = tol + 2.0 ** -8 * np.abs(ref)
    err = np.abs(got - ref)
    bad = err > tol
    assert not bad.any(), (f"{what}: {int(bad.sum())} of {bad.size} outputs outside the bound; worst "
                           f"{float((err / np.maximum(tol, 1e-300)).max()):.3g}x of it")
    return float(err.max()), float((err / np.maximum(mag, 1e-300)).max())


@pytest.mark.parametrize("rows,cols,target", [(64, 64, 4.0), (200, 136, 4.0), (130, 520, 3.0), (257, 72, 5.0),
                                              (1, 8, 0), (3, 72, 0), (640, 1024, 2.75)])
def test_blocks_decode_matches_oracle(rows, cols, target):
    x, blob = blocks_stream(rows, cols, target, seed=rows * 31 + cols)
    print(f"blocks decode {rows}x{cols} @ {target}", flush=True)
    p = ep.from_blob(blob).to("cuda")
    v = ep.decode_symbols(p)
    y = ep.decompress(p)
    torch.cuda.synchronize()
    assert np.array_equal(v.cpu().numpy(), oracle.decode_symbols(blob)), "symbols differ from the oracle's"
    assert np.array_equal(y.cpu().view(torch.int16).numpy(), oracle.decompress_raw(blob).view(np.int16)), \
        "weights differ from the oracle's"


@pytest.mark.parametrize("m,rows,cols,target", [
    (1, 64, 64, 4.0),          # one block, one token
    (5, 1, 8, 0),              # one row of one vector
    (37, 200, 136, 4.0),       # ragged rows (N % 64), ragged K (K % 64 = 8)
    (129, 130, 520, 3.0),      # m just past one row block
    (300, 257, 72, 5.0),       # one row past a block; K one vector past a block
    (1000, 384, 640, 4.0),     # several chunks of K, m over 512
    (520, 64, 4104, 2.75),     # K: eight full chunks and one vector
    (32, 257, 520, 3.0),       # few rows (wave-independent kernel), ragged N and K
    (17, 64, 4104, 2.75),      # few rows, several blocks per wave, one vector past a block
    (16, 1000, 1032, 4.0),     # few rows, many block rows
    (64, 200, 2056, 3.0),      # up to 64 rows: four row blocks per wave
    (45, 130, 136, 4.0),       # ragged rows inside the last row block
])
@pytest.mark.parametrize("out_dtype", [torch.float32, torch.bfloat16])
def test_linear_matches_fp64_product(m, rows, cols, target, out_dtype):
    x_w, blob = blocks_stream(rows, cols, target, seed=rows * 7 + cols)
    print(f"linear m={m} W {rows}x{cols} @ {target} -> {out_dtype}", flush=True)
    w64 = oracle_weights(blob)
    g = torch.Generator().manual_seed(m * 13 + rows)
    x = torch.randn(m, cols, generator=g).to(torch.bfloat16)
    p = ep.from_blob(blob).to("cuda")
    y = ep.linear(p, x.to("cuda"), out_dtype=out_dtype)
    torch.cuda.synchronize()
    check_linear(y, x, w64, what=f"m={m} {rows}x{cols}")


def test_linear_deterministic_and_no_weight_traffic_dependence():
    """Two calls give identical bits; the output does not depend on what the
    output buffer held before."""
    x_w, blob = blocks_stream(300, 520, 4.0, seed=5)
    x = torch.randn(777, 520, generator=torch.Generator().manual_seed(2)).to(torch.bfloat16).cuda()
    p = ep.from_blob(blob).to("cuda")
    y1 = torch.full((777, 300), float("nan"), device="cuda")
    y2 = torch.zeros((777, 300), device="cuda")
    ep.linear(p, x, out=y1, out_dtype=torch.float32)
    ep.linear(p, x, out=y2, out_dtype=torch.float32)
    torch.cuda.synchronize()
    assert torch.equal(y1.view(torch.int32), y2.view(torch.int32))


def test_linear_zero_rows_and_errors():
    x_w, blob = blocks_stream(64, 64, 4.0, seed=9)
    p = ep.from_blob(blob).to("cuda")
    y = ep.linear(p, torch.empty(0, 64, dtype=torch.bfloat16, device="cuda"))
    assert y.shape == (0, 64)
    # a row-major stream is refused
    rb, rc, _ = oracle.compress(x_w, 4.0)
    pr = ep.from_blob(rb).to("cuda")
    with pytest.raises(ep.EPError) as e:
        ep.linear(pr, torch.zeros(4, 64, dtype=torch.bfloat16, device="cuda"))
    assert e.value.code == ep.ERR_ARG


@pytest.mark.parametrize("j", [0, 4, 5])
def test_linear_dit_prefill_sampled_rows(j):
    """A DiT block's linears (3840x3840, 10240x3840, 3840x10240) at a
    4096-token prefill, the launch ep_linear makes at full size: the decoded
    weights exact against the oracle, and 96 sampled rows of Y plus the last
    row against the float64 product."""
    w = W.dit_matrix(0, j)
    blob, rc, _ = oracle.compress(w, 4.0, layout=oracle.LAYOUT_BLOCKS)
    assert rc == 0
    print(f"dit linear {j}: W {tuple(w.shape)} {8 * blob.size / w.numel():.4f} bpp", flush=True)
    w64 = oracle_weights(blob)
    x = W.gaussian(4096, w.shape[1], 1.0, seed=4999, dtype=torch.bfloat16)
    p = ep.from_blob(blob).to("cuda")
    wd = ep.decompress(p)
    y = ep.linear(p, x.to("cuda"), out_dtype=torch.float32)
    torch.cuda.synchronize()
    assert np.array_equal(wd.cpu().view(torch.int16).numpy(), oracle.decompress_raw(blob).view(np.int16))
    rows = np.sort(np.random.default_rng(j).choice(4096, 96, replace=False))
    rows = np.unique(np.append(rows, 4095))
    check_linear(y, x, w64, rows_idx=rows, what=f"dit {j}")


@pytest.mark.parametrize("m", [1, 16, 100])
def test_linear_split_k_matches_unsplit_bound_and_is_deterministic(m):
    """Small m: the sum over K is split across workgroups (partials added in
    slab order by a second kernel).  Split and unsplit results both lie
    within the FP32 summation bound of the float64 product; repeated split
    calls give identical bits."""
    w = W.dit_matrix(1, 0)
    blob, rc, _ = oracle.compress(w, 4.0, layout=oracle.LAYOUT_BLOCKS)
    assert rc == 0
    w64 = oracle_weights(blob)
    x = W.gaussian(m, 3840, 1.0, seed=77 + m, dtype=torch.bfloat16)
    p = ep.from_blob(blob).to("cuda")
    need = ep.linear_workspace_bytes(p, m)
    print(f"split-K m={m}: workspace {need} bytes", flush=True)
    assert need > 0
    ws = torch.empty(need, dtype=torch.uint8, device="cuda")
    xd = x.to("cuda")
    y1 = ep.linear(p, xd, out_dtype=torch.float32, workspace=ws)
    y2 = ep.linear(p, xd, out_dtype=torch.float32, workspace=ws)
    y0 = ep.linear(p, xd, out_dtype=torch.float32, workspace=torch.empty(0, dtype=torch.uint8, device="cuda"))
    torch.cuda.synchronize()
    assert torch.equal(y1.view(torch.int32), y2.view(torch.int32))
    check_linear(y1, x, w64, what=f"split m={m}")
    check_linear(y0, x, w64, what=f"unsplit m={m}")


@pytest.mark.parametrize("m", [1, 32, 300])
def test_linear_plan_matches_call_and_replays_in_a_graph(m):
    """A linear plan gives ep_linear's bits; captured in a HIP graph it
    replays exactly, with eager work on the same stream between replays."""
    w = W.gaussian(384, 1032, 0.02, seed=m + 3, dtype=torch.bfloat16)
    blob, rc, _ = oracle.compress(w, 4.0, layout=oracle.LAYOUT_BLOCKS)
    assert rc == 0
    print(f"linear plan m={m}", flush=True)
    p = ep.from_blob(blob).to("cuda")
    x = W.gaussian(m, 1032, 1.0, seed=m, dtype=torch.bfloat16).cuda()
    plan = ep.LinearPlan(p, m)
    ws = torch.empty(ep.linear_workspace_bytes(p, m), dtype=torch.uint8, device="cuda")
    ref = ep.linear(p, x, out_dtype=torch.float32, workspace=ws)
    got = plan.run(x, out_dtype=torch.float32)
    torch.cuda.synchronize()
    assert torch.equal(got.view(torch.int32), ref.view(torch.int32))
    s = torch.cuda.Stream()
    y = torch.empty(m, 384, dtype=torch.float32, device="cuda")
    with torch.cuda.stream(s):
        plan.run(x, out=y, out_dtype=torch.float32, stream=s)  # eager pass on the capture stream
    s.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g, stream=s):
        plan.run(x, out=y, out_dtype=torch.float32, stream=s)
    for i in range(3):
        with torch.cuda.stream(s):
            y.fill_(float("nan"))
            junk = torch.randn(257, 259, device="cuda") @ torch.randn(259, 263, device="cuda")
            g.replay()
        s.synchronize()
        assert torch.equal(y.view(torch.int32), ref.view(torch.int32)), f"replay {i}"
        del junk


@pytest.mark.parametrize("m", [0, 16, 300])
def test_corrupt_words_blocks_stream_within_bounds(m):
    """A blocks-layout stream whose whole word section is random bytes (pair
    counts, length codes and start bits included): the host checks the
    header, tables and tile offsets but not the words.  Decode and the fused
    linear (the wave-independent kernel at 16 rows, the chunk kernel at 300)
    still complete: each lane's word pointer starts clamped into its tile and
    moves at most one word per symbol (64 per lane), inside the LDS slack
    after the word buffers or the words and tables before them; table
    addresses are masked into the tables.  Coordinates stay in the value
    range, the products are finite, and a clean call right after is exact."""
    w = W.gaussian(200, 1032, 0.02, seed=8300, dtype=torch.bfloat16)
    blob, rc, _ = oracle.compress(w, 4.0, layout=oracle.LAYOUT_BLOCKS)
    assert rc == 0
    n_words = ep.blob_info(blob)["n_words"]
    o_w = blob.size - (2 * n_words + 15) // 16 * 16  # the word section ends the stream
    bad = blob.copy()
    bad[o_w:o_w + 2 * n_words] = np.random.default_rng(8301 + m).integers(0, 256, 2 * n_words, dtype=np.uint8)
    print(f"corrupt blocks stream, m={m}", flush=True)
    pb = ep.from_blob(bad).to("cuda")
    v = ep.decode_symbols(pb)
    yw = ep.decompress(pb)
    x = W.gaussian(max(m, 1), 1032, 1.0, seed=m, dtype=torch.bfloat16).cuda()
    yl = ep.linear(pb, x, out_dtype=torch.float32) if m else None
    torch.cuda.synchronize()
    assert int(v.abs().max()) <= 2047
    assert bool(torch.isfinite(yw.float()).all())
    if m:
        assert bool(torch.isfinite(yl).all())
    p = ep.from_blob(blob).to("cuda")
    y2 = ep.decompress(p)
    torch.cuda.synchronize()
    assert np.array_equal(y2.cpu().view(torch.int16).numpy(), oracle.decompress_raw(blob).view(np.int16))
