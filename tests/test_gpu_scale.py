"""GPU parity beyond the named workloads: a large stream checked on sampled
tiles (the oracle decodes only those), and seeded random shapes, containers
and rates checked in full."""
import numpy as np
import pytest
import torch

import oracle
from decode_tile_interleaved_amd import ep
from decode_tile_interleaved_amd import workloads as W

from cases import extreme_cases

pytestmark = pytest.mark.gpu


def _tile_elements(tile: int, rows: int, cols: int, tile_vecs: int):
    """(row, column) slices of the elements tile `tile` reconstructs."""
    vpr = (cols + 7) // 8
    out = []
    v0, v1 = tile * tile_vecs, min((tile + 1) * tile_vecs, rows * vpr)
    vid = v0
    while vid < v1:
        r, k = divmod(vid, vpr)
        k_end = min(vpr, k + (v1 - vid))
        out.append((r, slice(8 * k, min(cols, 8 * k_end))))
        vid += k_end - k
    return out


def test_large_stream_sampled_tiles():
    """24576 x 24576 BF16 (604M parameters, 73,728 tiles of 1024 vectors: the
    multi-tile kernel, 288 tiles per CU in 18 passes of 16 waves): the host
    encoder's stream, decoded on the GPU, against the oracle's decode of 24
    tiles."""
    rows = cols = 24576
    x = W.rowscale_gaussian(rows, cols, seed=4242)
    p = ep.compress(x, 4.0)
    assert abs(p.actual_bpp - 4.0) <= 0.02 * 4.0
    y = ep.decompress(p.to("cuda"))
    torch.cuda.synchronize()
    got = y.cpu().view(torch.int16).numpy()
    T, TV = p.info()["n_tiles"], p.info()["tile_vecs"]
    rng = np.random.default_rng(7)
    tiles = sorted(set([0, 1, T // 2, T - 2, T - 1] + rng.integers(0, T, 19).tolist()))
    ref = np.zeros((rows, cols), np.uint16)
    work = np.zeros((rows, cols), np.int32)
    for t in tiles:
        oracle.decompress_tile_range(p.blob, t, t + 1, out=ref, work=work)
        for r, cs in _tile_elements(t, rows, cols, TV):
            assert np.array_equal(got[r, cs].view(np.uint16), ref[r, cs]), (t, r)


def _random_cases(n: int, seed: int):
    rng = np.random.default_rng(seed)
    kinds = ["bf16", "fp16", "int8", "fp8"]
    for i in range(n):
        kind = kinds[i % 4]
        rows = int(rng.integers(1, 400))
        cols = int(rng.choice([int(rng.integers(1, 64)), int(rng.integers(64, 3000))]))
        a = float(np.exp(rng.uniform(np.log(0.02), np.log(2.0))))  # fixed resolution: any rate, any table width
        yield i, kind, rows, cols, a


@pytest.mark.parametrize("case", list(_random_cases(24, 2024)), ids=lambda c: f"{c[1]}_{c[2]}x{c[3]}_a{c[4]:.3f}")
def test_random_shapes_containers_rates(case):
    i, kind, rows, cols, a = case
    if kind in ("bf16", "fp16"):
        x = W.gaussian(rows, cols, 0.02, seed=900 + i, dtype=torch.bfloat16 if kind == "bf16" else torch.float16)
    else:
        x = W.absmax_codes(rows, cols, 900 + i, kind)
    blob, rc, _ = oracle.compress(x, 4.0, fixed_a=a)
    if rc == oracle.WARN_RAW:  # coordinates beyond the stream's range: raw container, copied
        y = ep.decompress(ep.from_blob(blob).to("cuda"))
        torch.cuda.synchronize()
        assert torch.equal(y.cpu().view(torch.uint8 if x.element_size() == 1 else torch.int16),
                           x.view(torch.uint8 if x.element_size() == 1 else torch.int16))
        return
    assert rc == 0
    p = ep.from_blob(blob).to("cuda")
    v = ep.decode_symbols(p)
    y = ep.decompress(p)
    torch.cuda.synchronize()
    assert np.array_equal(v.cpu().numpy(), oracle.decode_symbols(blob))
    ref = oracle.decompress_raw(blob)
    got = y.cpu().view(torch.int16 if x.element_size() == 2 else torch.int8).numpy()
    # exact for every container: the kernel rounds as the oracle does (f32
    # product, then the container's rounding); the stated bar for BF16/FP16
    # is one unit in the last place
    bad = np.argwhere(got.view(np.uint8) != ref.view(np.uint8))
    assert bad.size == 0, f"{len(bad)} bytes differ, first {bad[:4].tolist()}"


def test_fp16_padded_rounds_through_f32():
    """FP16 with padded columns (per-element stores): y = f32(v * g) first,
    then round to FP16, as the oracle does.  A fused multiply-and-narrow
    (one rounding) differs by one unit in the last place where f32(v * g)
    lies on an FP16 midpoint; this matrix has twelve such elements."""
    x = W.gaussian(363, 2751, 0.02, seed=901, dtype=torch.float16)
    blob, rc, _ = oracle.compress(x, 4.0, fixed_a=0.0385029163886993)
    assert rc == 0
    y = ep.decompress(ep.from_blob(blob).to("cuda"))
    torch.cuda.synchronize()
    got = y.cpu().view(torch.int16).numpy().view(np.uint16)
    ref = oracle.decompress_raw(blob).view(np.uint16)
    bad = np.argwhere(got != ref)
    assert bad.size == 0, f"{len(bad)} elements differ, first {bad[:4].tolist()}"


@pytest.mark.parametrize("name", list(extreme_cases()))
def test_extreme_inputs(name):
    """Magnitudes at the ends of each format (f32 subnormal products, FP16
    values at its maximum reconstructed past it, FP16 subnormal inputs), a
    single short row, zero rows, an all-zero matrix (nothing to code: raw
    container) and a 10^6-sigma spike: the oracle's stream, decoded on the
    GPU, equals the oracle's decode exactly, and the host encoder writes the
    oracle's stream."""
    x, target, fixed = extreme_cases()[name]
    blob, rc, _ = oracle.compress(x, target, fixed_a=fixed)
    host = ep.compress(x, target, fixed_scale=fixed)
    assert host.status == rc and np.array_equal(host.blob, blob)
    p = ep.from_blob(blob).to("cuda")
    y = ep.decompress(p)
    torch.cuda.synchronize()
    got = y.cpu().view(torch.int16).numpy().view(np.uint16)
    ref = oracle.decompress_raw(blob).view(np.uint16)
    bad = np.argwhere(got != ref)
    assert bad.size == 0, f"{len(bad)} elements differ, first {bad[:4].tolist()}: " \
                          f"{[hex(int(got[tuple(i)])) for i in bad[:4]]} vs {[hex(int(ref[tuple(i)])) for i in bad[:4]]}"


def _random_multitile(n: int, seed: int):
    rng = np.random.default_rng(seed)
    kinds = ["bf16", "fp16", "int8", "fp8"]
    for i in range(n):
        kind = kinds[i % 4]
        rows, cols = int(rng.integers(2100, 2600)), int(rng.integers(8100, 9000))
        hi = 7.5 if kind in ("int8", "fp8") else 8.0
        yield i, kind, rows, cols, round(float(rng.uniform(1.0, hi)), 3)


@pytest.mark.parametrize("case", list(_random_multitile(4, 55)), ids=lambda c: f"{c[1]}_{c[2]}x{c[3]}_t{c[4]}")
def test_random_multitile_streams(case):
    """Seeded random shapes of 2100-2600 x 8100-9000 (more than one round of
    workgroups: the multi-tile kernel, uneven tile counts per CU, padded
    columns), containers and targets: symbols and values equal the oracle's."""
    i, kind, rows, cols, target = case
    if kind in ("bf16", "fp16"):
        x = W.t4_outliers(rows, cols, 5500 + i, dtype=torch.bfloat16 if kind == "bf16" else torch.float16)
    else:
        x = W.absmax_codes(rows, cols, 5500 + i, kind)
    blob, rc, _ = oracle.compress(x, target)
    p = ep.from_blob(blob).to("cuda")
    y = ep.decompress(p)
    torch.cuda.synchronize()
    got = y.cpu().view(torch.int16 if x.element_size() == 2 else torch.int8).numpy().view(np.uint8)
    if rc == oracle.WARN_RAW:  # outliers beyond the stream's value range at this rate: raw container
        assert np.array_equal(got, x.view(torch.int16 if x.element_size() == 2 else torch.int8).numpy().view(np.uint8))
        return
    assert rc == 0
    v = ep.decode_symbols(p)
    torch.cuda.synchronize()
    assert np.array_equal(v.cpu().numpy(), oracle.decode_symbols(blob))
    assert np.array_equal(got, oracle.decompress_raw(blob).view(np.uint8))


def test_multitile_lds_limited_waves():
    """A 4096 x 10240 BF16 stream at 8.0 bpp (wide tables): a tile's words
    take about 8 KB, so beside the 56 KB of tables the LDS holds fewer than
    16 word buffers, and each CU's run of 20 tiles takes two passes of its
    waves.  Symbols and values equal the oracle's."""
    x = W.rowscale_gaussian(4096, 10240, 6100)
    blob, rc, _ = oracle.compress(x, 8.0)
    assert rc == 0
    inf = oracle.info(blob)
    tile_bytes = 2 * inf["n_words"] / inf["n_tiles"]
    assert 16 * tile_bytes + 7 * 8192 > 160 * 1024  # sixteen buffers cannot fit
    assert inf["n_tiles"] > 16 * 256  # more tiles per CU than waves (256 CUs)
    p = ep.from_blob(blob).to("cuda")
    v = ep.decode_symbols(p)
    y = ep.decompress(p)
    torch.cuda.synchronize()
    assert np.array_equal(v.cpu().numpy(), oracle.decode_symbols(blob))
    assert np.array_equal(y.cpu().view(torch.int16).numpy().view(np.uint16), oracle.decompress_raw(blob).view(np.uint16))


@pytest.mark.parametrize("rows,cols,target", [(512, 4096, 4.0), (3072, 8192, 4.0), (512, 4096, 0.2),
                                              (3072, 8192, 0.15), (256, 8192, 0.06)],
                         ids=["one_round", "multi_tile", "one_round_16", "multi_tile_16", "16_states_1024"])
def test_corrupt_words_decode_within_bounds(rows, cols, target):
    """The host checks a stream's header, tables and tile offsets but not its
    words (that would mean decoding it).  With the whole word section
    overwritten by random bytes (pair counts, length codes and start bits
    included) the decoder still completes: a lane's word pointer starts
    clamped into its tile and moves at most one word per symbol (8 per vector,
    64 vectors per lane at most), inside the LDS slack after the buffers or
    the tables before them; start-state reads stay within 300 bytes of the
    tile; table addresses are masked into the tables.  Every decoded
    coordinate stays in the stream's value range, and a clean decode right
    after is exact.  64-state and 16-state tiles (512 and 1024 vectors) in
    the single-round and the multi-tile kernel."""
    x = W.rowscale_gaussian(rows, cols, 8100)
    blob, rc, _ = oracle.compress(x, target)
    assert rc == 0
    n_words = ep.blob_info(blob)["n_words"]
    o_w = blob.size - (2 * n_words + 15) // 16 * 16  # the word section ends the stream
    bad = blob.copy()
    bad[o_w:o_w + 2 * n_words] = np.random.default_rng(8101).integers(0, 256, 2 * n_words, dtype=np.uint8)
    pb = ep.from_blob(bad).to("cuda")
    v = ep.decode_symbols(pb)
    y = ep.decompress(pb)
    torch.cuda.synchronize()
    assert int(v.abs().max()) <= 2047
    assert bool(torch.isfinite(y.float()).all())
    p = ep.from_blob(blob).to("cuda")
    y2 = ep.decompress(p)
    torch.cuda.synchronize()
    assert np.array_equal(y2.cpu().view(torch.int16).numpy().view(np.uint16), oracle.decompress_raw(blob).view(np.uint16))


def _low_rate_cases():
    yield "bf16_one_round", W.rowscale_gaussian(512, 4096, 8200), 0.2
    yield "bf16_1024_vector_tiles", W.rowscale_gaussian(256, 8192, 8206), 0.06
    yield "bf16_multi_tile", W.rowscale_gaussian(3072, 8192, 8201), 0.15
    yield "t4_bf16", W.t4_outliers(384, 6144, 8202, dtype=torch.bfloat16), 0.3
    yield "fp16_padded", W.rowscale_gaussian(300, 1000, 8203).to(torch.float16), 0.2
    yield "int8_codes", W.absmax_codes(512, 2048, 8204, "int8"), 0.3
    yield "fp8_padded", W.absmax_codes(256, 3000, 8205, "fp8"), 0.25


@pytest.mark.parametrize("case", list(_low_rate_cases()), ids=lambda c: c[0])
def test_low_rate_16_state_streams(case):
    """Low targets take 16 states per tile: a wave decodes four tiles, one per
    16-lane DPP row, each lane 32 vectors (64 for 1024-vector tiles at the
    lowest targets) in groups of 8 whose row scales load during the group
    before.  Symbols and values equal the oracle's in the single-round and the
    multi-tile kernel, for every container."""
    _, x, target = case
    blob, rc, _ = oracle.compress(x, target)
    assert rc == 0 and oracle.info(blob)["n_states"] == 16
    assert abs(8 * blob.size / x.numel() - target) <= 0.02 * target
    p = ep.from_blob(blob).to("cuda")
    v = ep.decode_symbols(p)
    y = ep.decompress(p)
    torch.cuda.synchronize()
    assert np.array_equal(v.cpu().numpy(), oracle.decode_symbols(blob))
    got = y.cpu().view(torch.int16 if x.element_size() == 2 else torch.int8).numpy().view(np.uint8)
    assert np.array_equal(got, oracle.decompress_raw(blob).view(np.uint8))


@pytest.mark.parametrize("n_states,tile_vecs,target,kind", [(64, 1024, 0.3, "bf16"), (16, 512, 4.0, "bf16"),
                                                            (16, 1024, 2.0, "fp16"), (64, 512, 0.45, "int8"),
                                                            (16, 512, 3.0, "fp8")])
def test_forced_geometry_streams(n_states, tile_vecs, target, kind):
    """ep_options force the tile geometry: a 64-state stream at a low target
    and a 16-state stream at a high one (and the other pairings) decode on
    the GPU to the oracle's symbols and values; the host encoder's stream is
    the oracle's byte for byte."""
    if kind in ("int8", "fp8"):
        x = W.absmax_codes(384, 2048, 8300 + n_states, kind)
    else:
        x = W.rowscale_gaussian(384, 2056, 8300 + n_states)
        if kind == "fp16":
            x = x.to(torch.float16)
    p = ep.compress(x, target, n_states=n_states, tile_vecs=tile_vecs)
    blob, rc, _ = oracle.compress(x, target, n_states=n_states, tile_vecs=tile_vecs)
    assert p.status == rc == 0 and np.array_equal(p.blob, blob)
    d = ep.blob_info(blob)
    assert (d["n_states"], d["tile_vecs"]) == (n_states, tile_vecs)
    p.to("cuda")
    v = ep.decode_symbols(p)
    y = ep.decompress(p)
    torch.cuda.synchronize()
    assert np.array_equal(v.cpu().numpy(), oracle.decode_symbols(blob))
    got = y.cpu().view(torch.int16 if x.element_size() == 2 else torch.int8).numpy().view(np.uint8)
    assert np.array_equal(got, oracle.decompress_raw(blob).view(np.uint8))
