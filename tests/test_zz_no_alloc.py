"""ep_compress_device_noalloc, the compression entry point that allocates
nothing, called through the C ABI: its stream equals ep_compress_device's
byte for byte on two calls in a row on one GPU, the second with a smaller
input (the scratch array keeps the first call's contents, which must not
leak into the second).  Also its limits: a matrix past 2^22 padded elements
is refused before any device work, and a too-small output buffer reports
the size it needs."""
import ctypes

import numpy as np
import pytest
import torch

from decode_tile_interleaved_amd import ep
from decode_tile_interleaved_amd import workloads as W

pytestmark = pytest.mark.gpu


def _noalloc(t: torch.Tensor, target: float, capacity: int | None = None, **opts):
    """(status, stream bytes or None, nbytes) from ep_compress_device_noalloc."""
    L = ep.lib()
    rows, cols = t.shape
    if capacity is None:  # the raw container bounds every target-selected stream
        capacity = 128 + (rows * cols * t.element_size() + 15) // 16 * 16
    out = np.zeros(capacity, np.uint8)
    nb = ctypes.c_size_t(0)
    opt = ep._options(**opts)
    stream = torch.cuda.current_stream(t.device)
    rc = L.ep_compress_device_noalloc(ctypes.c_void_p(t.data_ptr()), ep._DTYPE_CODE[t.dtype], rows, cols,
                                      float(target), ctypes.byref(opt), ctypes.c_void_p(stream.cuda_stream),
                                      ctypes.c_void_p(out.ctypes.data), capacity, ctypes.byref(nb))
    return rc, (out[:nb.value].copy() if rc >= 0 else None), nb.value


def test_two_calls_match_the_allocating_entry_point():
    big = W.rowscale_gaussian(1024, 4096, 9001).cuda()        # 2^22 elements: the largest allowed
    small = W.t4_outliers(200, 1000, 9002).cuda()            # padded columns, heavy tails
    for t, target in ((big, 4.0), (small, 2.75)):
        rc, blob, _ = _noalloc(t, target)
        assert rc == ep.OK, (rc, ep.last_error())
        assert ep.last_encode_count() == 1
        ref = ep.compress_device(t, target)
        assert ref.status == rc
        assert np.array_equal(blob, ref.blob)
        # and the stream decodes like the allocating entry point's
        p = ep.from_blob(blob).to("cuda")
        y = ep.decompress(p)
        y_ref = ep.decompress(ref.to("cuda"))
        torch.cuda.synchronize()
        assert torch.equal(y.view(torch.int16), y_ref.view(torch.int16))


def test_options_and_low_rates_match():
    t = W.rowscale_gaussian(300, 2000, 9003).cuda()
    for target, opts in ((0.2, {}), (3.0, {"n_states": 16}), (2.0, {"tile_vecs": 1024, "seed": 5})):
        rc, blob, _ = _noalloc(t, target, **opts)
        assert rc == ep.OK, (rc, ep.last_error(), target, opts)
        ref = ep.compress_device(t, target, **opts)
        assert rc == ref.status
        assert np.array_equal(blob, ref.blob), (target, opts)


def test_limits():
    t = W.rowscale_gaussian(64, 1000, 9004).cuda()
    rc, _, need = _noalloc(t, 4.0, capacity=1000)
    assert rc == ep.ERR_ARG and need > 1000
    rc, blob, n = _noalloc(t, 4.0, capacity=need)
    assert rc == ep.OK and n == need
    assert np.array_equal(blob, ep.compress_device(t, 4.0).blob)
    # past 2^22 padded elements: refused on the host, nothing enqueued
    L = ep.lib()
    out = np.zeros(16, np.uint8)
    nb = ctypes.c_size_t(0)
    rc = L.ep_compress_device_noalloc(ctypes.c_void_p(t.data_ptr()), ep.BF16, 1025, 4096, 4.0, None, None,
                                      ctypes.c_void_p(out.ctypes.data), 16, ctypes.byref(nb))
    assert rc == ep.ERR_SHAPE
    assert "scratch" in ep.last_error()
