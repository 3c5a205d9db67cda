"""GPU encoder (ep_compress_device): the stream it writes for a matrix in
device memory equals, byte for byte, the oracle's stream and the host
encoder's stream for the same input.  Covers BF16/FP16/INT8/FP8 containers,
narrow and wide tables, padded columns, a stream of more tiles than one round
of workgroups, rate selection and a fixed resolution, the raw fallback and
the input errors."""
import numpy as np
import pytest
import torch

import oracle
from decode_tile_interleaved_amd import ep
from decode_tile_interleaved_amd import workloads as W

from cases import extreme_cases

pytestmark = pytest.mark.gpu

CASES = {
    # name: (matrix, target, fixed resolution or 0)
    "gauss256_bf16_3.5": lambda: (W.make("gauss256_bf16_3.5")[0], 3.5, 0.0),
    "rowscale4096_bf16_4.0": lambda: (W.make("rowscale4096_bf16_4.0")[0], 4.0, 0.0),
    "t4outlier3072x12288_bf16_2.75": lambda: (W.make("t4outlier3072x12288_bf16_2.75")[0], 2.75, 0.0),
    "ragged_7_13_fp16_fixed": lambda: (W.gaussian(7, 13, 0.02, seed=62, dtype=torch.float16), 4.0, 0.2),
    "ragged_1030_8_bf16_fixed": lambda: (W.gaussian(1030, 8, 0.02, seed=7218, dtype=torch.bfloat16), 4.0, 0.3),
    "codes_37_1030_int8_3.0": lambda: (W.absmax_codes(37, 1030, 37 * 7 + 1030, "int8"), 3.0, 0.0),
    "codes_300_1030_int8_7.0": lambda: (W.absmax_codes(300, 1030, 300 * 7 + 1030, "int8"), 7.0, 0.0),
    "codes_2100_8190_fp8_5.0": lambda: (W.absmax_codes(2100, 8190, 2100 * 7 + 8190, "fp8"), 5.0, 0.0),
}


@pytest.mark.parametrize("name", list(CASES))
def test_device_stream_equals_oracle_and_host(name):
    x, target, fixed = CASES[name]()
    if fixed > 0:
        ref, rc_ref, _ = oracle.compress(x, target, fixed_a=fixed)
    else:
        ref, rc_ref, _ = oracle.compress(x, target)
    host = ep.compress(x, target, fixed_scale=fixed)
    dev = ep.compress_device(x.cuda(), target, fixed_scale=fixed)
    assert dev.status == rc_ref == host.status
    assert np.array_equal(host.blob, ref)
    assert dev.blob.size == ref.size
    bad = np.flatnonzero(dev.blob != ref)
    assert bad.size == 0, f"{bad.size} bytes differ, first at {bad[:8].tolist()}"


def test_device_round_trip_through_decoder():
    x, target = W.make("rowscale4096_bf16_4.0")
    p = ep.compress_device(x.cuda(), target).to("cuda")
    y = ep.decompress(p)
    torch.cuda.synchronize()
    assert np.array_equal(y.cpu().view(torch.int16).numpy(), oracle.decompress_raw(p.blob).view(np.int16))


def test_device_raw_fallback_and_errors():
    t = torch.zeros(4, 4096, dtype=torch.bfloat16)
    t[:, 0] = 1.0
    t[:, 1:] = 1e-3
    ref, rc, _ = oracle.compress(t, 10.0)
    assert rc == oracle.WARN_RAW
    p = ep.compress_device(t.cuda(), 10.0)
    assert p.status == ep.WARN_RAW and np.array_equal(p.blob, ref)
    bad = W.gaussian(16, 64, 0.02, seed=3).cuda()
    bad[3, 5] = float("nan")
    with pytest.raises(ep.EPError) as e:
        ep.compress_device(bad, 4.0)
    assert e.value.code == ep.ERR_NONFINITE
    with pytest.raises(ep.EPError) as e:
        ep.compress_device(W.gaussian(16, 64, 0.02, seed=3).cuda(), 20.0)
    assert e.value.code == ep.ERR_TARGET


def test_device_alphabet_overflow_falls_back_to_raw():
    """At 9.0 bpp a context of this matrix needs more than 2^10 symbols: the
    GPU encoder warns and stores the raw container, as the oracle does."""
    x = W.rowscale_gaussian(1024, 4096, 6100)
    ref, rc, _ = oracle.compress(x, 9.0)
    assert rc == oracle.WARN_RAW
    p = ep.compress_device(x.cuda(), 9.0)
    assert p.status == ep.WARN_RAW and np.array_equal(p.blob, ref)


@pytest.mark.parametrize("name", list(extreme_cases()))
def test_device_stream_at_format_extremes(name):
    """The GPU encoder at the ends of the formats (tiny and huge BF16, FP16
    near its maximum and subnormal, a short row, zero rows, an all-zero
    matrix, a spike): the oracle's stream, byte for byte."""
    x, target, fixed = extreme_cases()[name]
    ref, rc, _ = oracle.compress(x, target, fixed_a=fixed)
    dev = ep.compress_device(x.cuda(), target, fixed_scale=fixed)
    assert dev.status == rc
    assert np.array_equal(dev.blob, ref)


def _random_targets(n: int, seed: int):
    rng = np.random.default_rng(seed)
    kinds = ["bf16", "fp16", "int8", "fp8"]
    for i in range(n):
        kind = kinds[i % 4]
        rows, cols = int(rng.integers(16, 600)), int(rng.integers(16, 4000))
        hi = 7.5 if kind in ("int8", "fp8") else 9.0
        yield i, kind, rows, cols, round(float(rng.uniform(1.5, hi)), 3)


@pytest.mark.parametrize("case", list(_random_targets(8, 31)), ids=lambda c: f"{c[1]}_{c[2]}x{c[3]}_t{c[4]}")
def test_device_stream_random_targets(case):
    """Seeded random shapes, containers and targets through rate selection:
    the GPU encoder's stream equals the oracle's."""
    i, kind, rows, cols, target = case
    if kind in ("bf16", "fp16"):
        x = W.rowscale_gaussian(rows, cols, 3100 + i, dtype=torch.bfloat16 if kind == "bf16" else torch.float16)
    else:
        x = W.absmax_codes(rows, cols, 3100 + i, kind)
    try:
        ref, rc, _ = oracle.compress(x, target)
    except oracle.OracleError as e:  # a target this shape cannot reach: the device encoder must refuse it too
        with pytest.raises(ep.EPError) as d:
            ep.compress_device(x.cuda(), target)
        assert d.value.code == e.rc
        return
    dev = ep.compress_device(x.cuda(), target)
    assert dev.status == rc
    assert np.array_equal(dev.blob, ref)


@pytest.mark.parametrize("target", [0.36, 0.4, 7.0])
def test_device_stream_rate_corrections(target):
    """Low targets (16-state tiles) and heavy tails at 7.0 bpp, where the
    sampled selection is corrected by whole-matrix histograms (no encode).
    The GPU encoder's stream equals the oracle's and it encodes once."""
    if target < 1.0:
        x = W.rowscale_gaussian(512, 4096, 7001)
    else:
        x = W.t4_outliers(384, 6144, 7002, dtype=torch.bfloat16)
    ref, rc, _ = oracle.compress(x, target)
    p = ep.compress_device(x.cuda(), target)
    assert ep.last_encode_count() == 1
    assert p.status == rc == 0 and np.array_equal(p.blob, ref)
    assert abs(8 * ref.size / x.numel() - target) <= 0.02 * target


@pytest.mark.parametrize("target", [0.15, 0.3])
def test_device_16_state_streams(target):
    """At low targets (16 states per tile) the GPU encoder writes the
    oracle's 16-state stream, byte for byte."""
    x = W.rowscale_gaussian(512, 4096, 7001)
    ref, rc, _ = oracle.compress(x, target)
    assert rc == 0 and oracle.info(ref)["n_states"] == 16
    p = ep.compress_device(x.cuda(), target)
    assert p.status == 0 and np.array_equal(p.blob, ref)
