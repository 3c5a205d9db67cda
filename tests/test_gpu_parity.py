"""GPU parity of the fused tile decoder against the CPU oracle.

Every case feeds the ORACLE's stream (built from seeded inputs) to the
product's C ABI and compares, element by element:
  * ep_decode_symbols with the oracle's decoded lattice coordinates: bit-exact;
  * ep_decompress with the oracle's reconstruction: BF16/FP16 within 1 ulp
    (the kernel's arithmetic is the same single f32 product with RNE
    conversion, so 0 ulp is expected and reported), FP8/INT8 codes exact.
"""
import functools
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


@functools.lru_cache(maxsize=None)
def oracle_case(name: str):
    """(input, oracle stream, oracle symbols, oracle container codes)."""
    if name.startswith("dit"):
        _, blk, j = name.split("_")
        x, target = W.dit_matrix(int(blk), int(j)), 4.0
        blob, rc, _ = oracle.compress(x, target)
    elif name.startswith("codes"):
        _, r, c, kind, t = name.split("_")
        x = W.absmax_codes(int(r), int(c), seed=int(r) * 7 + int(c), kind=kind)
        blob, rc, _ = oracle.compress(x, float(t))
    elif name.startswith("ragged"):
        _, r, c, dt, a = name.split("_")
        dtype = {"bf16": torch.bfloat16, "fp16": torch.float16}[dt]
        x = W.gaussian(int(r), int(c), 0.02, seed=int(r) * 7 + int(c), dtype=dtype)
        blob, rc, _ = oracle.compress(x, 4.0, fixed_a=float(a))
    else:
        x, target = W.make(name)
        blob, rc, _ = oracle.compress(x, target)
    assert rc == 0, rc
    return x, blob, oracle.decode_symbols(blob), oracle.decompress_raw(blob)


def gpu_packed(blob):
    return ep.from_blob(blob).to("cuda")


def ulp_diff(a: np.ndarray, b: np.ndarray, dtype) -> int:
    """Largest distance in units in the last place between two arrays of
    BF16/FP16 bit patterns (sign-magnitude -> ordered integers)."""
    def ordered(u):
        u = u.astype(np.int64)
        return np.where(u & 0x8000, 0x8000 - (u & 0x7FFF), 0x8000 + u)
    return int(np.abs(ordered(a.view(np.uint16)) - ordered(b.view(np.uint16))).max()) if a.size else 0


WORKLOADS = ["gauss256_bf16_3.5", "rowscale4096_bf16_4.0", "t4outlier3072x12288_bf16_2.75", "absmax8192_int8_3.0",
             "absmax8192_fp8_3.0", "rowscale4096_bf16_0.2"]
RAGGED = ["ragged_1_8_bf16_0.3", "ragged_3_5_bf16_0.3", "ragged_7_13_fp16_0.2", "ragged_3_2736_bf16_0.5",
          "ragged_129_64_bf16_0.05", "ragged_64_1032_fp16_1.0", "ragged_5_4100_bf16_2.0", "ragged_1030_8_bf16_0.3",
          # more tiles than one round of workgroups covers (the multi-tile
          # kernel, some waves without a tile in the last pass): wide tables
          # with padded columns, and FP16
          "ragged_3200_8190_bf16_0.05", "ragged_3200_8192_fp16_0.3"]
DIT = ["dit_0_0", "dit_0_4", "dit_0_5"]
# 8-bit code containers with padded columns (per-element stores), narrow and
# wide tables, in one round of workgroups and in the multi-tile kernel
CODES = ["codes_37_1030_int8_3.0", "codes_37_1030_fp8_3.0", "codes_300_1030_int8_7.0", "codes_2100_8190_int8_3.0",
         "codes_2100_8190_fp8_7.0",
         # unpadded FP8 reconstructions beyond 448 in one round of workgroups
         "codes_300_1024_fp8_2.0"]


@pytest.mark.parametrize("name", WORKLOADS + RAGGED + DIT + CODES)
def test_symbols_bit_exact(name):
    x, blob, v_ref, _ = oracle_case(name)
    p = gpu_packed(blob)
    v = ep.decode_symbols(p)
    torch.cuda.synchronize()
    v = v.cpu().numpy()
    assert v.shape == v_ref.shape
    bad = np.argwhere(v != v_ref)
    assert bad.size == 0, f"{bad.shape[0]} symbol mismatches, first at {bad[:4].tolist()}"


@pytest.mark.parametrize("name", WORKLOADS + RAGGED + DIT + CODES)
def test_decompress_matches_oracle(name):
    x, blob, _, ref = oracle_case(name)
    p = gpu_packed(blob)
    y = ep.decompress(p)
    torch.cuda.synchronize()
    assert y.dtype == x.dtype and tuple(y.shape) == tuple(x.shape)
    got = y.cpu().view(torch.int16 if y.element_size() == 2 else torch.int8).numpy()
    if x.dtype in (torch.bfloat16, torch.float16):
        d = ulp_diff(got.view(np.uint16), ref.view(np.uint16), x.dtype)
        print(f"{name}: max ulp difference {d}")
        assert d <= 1
    else:
        assert np.array_equal(got.view(np.uint8), ref.view(np.uint8))


@pytest.mark.parametrize("name", ["rowscale4096_bf16_4.0", "t4outlier3072x12288_bf16_2.75"])
def test_product_stream_round_trip(name):
    """The product's own encoder and decoder end to end: the stream equals
    the oracle's, the decode equals the oracle's, the rate is within 2%."""
    x, blob, _, ref = oracle_case(name)
    p = ep.compress(x, W.WORKLOADS[name][3]).to("cuda")
    assert np.array_equal(p.blob, blob)
    assert abs(p.actual_bpp - W.WORKLOADS[name][3]) / W.WORKLOADS[name][3] <= 0.02
    y = ep.decompress(p)
    torch.cuda.synchronize()
    assert np.array_equal(y.cpu().view(torch.int16).numpy(), ref.view(np.int16))
    rel = ((y.double() - x.double().cuda()).norm() / x.double().cuda().norm()).item()
    print(f"{name}: actual_bpp {p.actual_bpp:.4f} rel L2 {rel:.4f}")


def test_deterministic_and_stream_ordered():
    x, blob, _, ref = oracle_case("rowscale4096_bf16_4.0")
    p = gpu_packed(blob)
    s = torch.cuda.Stream()
    with torch.cuda.stream(s):
        a = ep.decompress(p)
        b = ep.decompress(p)
    s.synchronize()
    assert torch.equal(a.view(torch.int16), b.view(torch.int16))


def test_raw_stream_on_gpu():
    t = torch.zeros(4, 4096, dtype=torch.bfloat16)
    t[:, 0] = 1.0
    t[:, 1:] = 1e-3
    blob, rc, _ = oracle.compress(t, 10.0)
    assert rc == oracle.WARN_RAW
    y = ep.decompress(gpu_packed(blob))
    torch.cuda.synchronize()
    assert torch.equal(y.cpu(), t)
    with pytest.raises(ep.EPError):
        ep.decode_symbols(gpu_packed(blob))


def test_device_argument_errors():
    x, blob, _, _ = oracle_case("gauss256_bf16_3.5")
    p = gpu_packed(blob)
    lib = ep.lib()
    out = torch.empty(256, 256, dtype=torch.bfloat16, device="cuda")
    import ctypes
    h = blob.ctypes.data
    rc = lib.ep_decompress(h, blob.size, ctypes.c_void_p(p.dev.data_ptr() + 2), ctypes.c_void_p(out.data_ptr()), -1,
                           None)
    assert rc == ep.ERR_ARG
    rc = lib.ep_decompress(h, blob.size, ctypes.c_void_p(p.dev.data_ptr()), ctypes.c_void_p(out.data_ptr()),
                           ep.FP16, None)
    assert rc == ep.ERR_ARG
    bad = blob.copy()
    bad[4] ^= 1
    rc = lib.ep_decompress(bad.ctypes.data, bad.size, ctypes.c_void_p(p.dev.data_ptr()),
                           ctypes.c_void_p(out.data_ptr()), -1, None)
    assert rc == ep.ERR_FORMAT
    torch.cuda.synchronize()


@pytest.mark.parametrize("name", ["gauss256_bf16_3.5", "absmax8192_int8_3.0", "rowscale4096_bf16_0.2",
                                  "ragged_64_1032_fp16_1.0", "codes_2100_8190_fp8_7.0"])
def test_plan_decode_equals_decompress(name):
    """ep_plan_decompress (geometry and arguments computed once) writes what
    ep_decompress writes, which equals the oracle's reconstruction: one
    round of workgroups and the multi-tile kernel, a 16-state stream, padded
    FP16 columns and 8-bit codes; three calls into different outputs, then
    five replays of a captured plan decode with eager work between them."""
    x, blob, _, codes = oracle_case(name)
    p = gpu_packed(blob)
    pl = ep.plan(p)
    s = torch.cuda.Stream()
    with torch.cuda.stream(s):
        ref = ep.decompress(p, stream=s)
        outs = [pl.decompress(stream=s) for _ in range(3)]
    s.synchronize()
    view = torch.int16 if ref.element_size() == 2 else torch.int8
    got = ref.cpu().view(view).numpy()
    if x.dtype in (torch.bfloat16, torch.float16):
        assert ulp_diff(got.view(np.uint16), codes.view(np.uint16), x.dtype) <= 1
    else:
        assert np.array_equal(got.view(np.uint8), codes.view(np.uint8))
    for o in outs:
        assert torch.equal(o.view(view), ref.view(view))
    out = torch.empty_like(ref)
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g, stream=s):
        pl.decompress(out=out, stream=s)
    for _ in range(5):
        out.zero_()
        torch.cuda.synchronize()
        with torch.cuda.stream(s):
            g.replay()
        s.synchronize()
        assert torch.equal(out.view(view), ref.view(view))
        with torch.cuda.stream(s):
            pl.decompress(stream=s)
        s.synchronize()
    pl.close()


def test_plan_of_raw_stream():
    """A raw container's plan copies the payload."""
    t = torch.zeros(4, 4096, dtype=torch.bfloat16)
    t[:, 0] = 1.0
    t[:, 1:] = 1e-3
    p = ep.compress(t, 10.0).to("cuda")
    assert p.status == ep.WARN_RAW
    out = ep.plan(p).decompress()
    torch.cuda.synchronize()
    assert torch.equal(out.cpu().view(torch.int16), t.view(torch.int16))


def test_decode_replays_from_a_graph():
    """ep_decompress enqueues kernels only (no allocation, no memset, no
    synchronization), so it can be captured in a HIP graph: five replays,
    with eager decodes and synchronizations between them, each equal the
    eager result, for the single-round and the multi-tile kernel."""
    for rows, cols in ((512, 4096), (3072, 8192)):
        x = W.rowscale_gaussian(rows, cols, 8300)
        p = ep.compress(x, 4.0).to("cuda")
        s = torch.cuda.Stream()
        with torch.cuda.stream(s):
            ref = ep.decompress(p, stream=s)
            out = torch.empty_like(ref)
            ep.decompress(p, out=out, stream=s)  # warm-up outside the capture
        s.synchronize()
        g = torch.cuda.CUDAGraph()
        with torch.cuda.graph(g, stream=s):
            ep.decompress(p, out=out, stream=s)
        for _ in range(5):
            out.zero_()
            torch.cuda.synchronize()
            with torch.cuda.stream(s):
                g.replay()
            s.synchronize()
            assert torch.equal(out.view(torch.int16), ref.view(torch.int16))
            with torch.cuda.stream(s):
                ep.decompress(p, stream=s)  # eager work between replays
            s.synchronize()
