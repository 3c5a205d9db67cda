"""CPU oracle for lattice-rANS weight compression.

TEST INFRASTRUCTURE ONLY: the test suite, ``__graft_entry__.smoke()`` and the
benchmark's ``cpu_baseline`` leg are the only code that may import this
package.  The product (``decode_tile_interleaved_amd``) never imports it and
shares no code with it; the two meet only through byte streams and arrays.

The arithmetic lives in ``oracle.c`` (plain scalar C, f64).  It follows the
EntroPack pages:

* mlsanity index page, arXiv abstract: row-normalized E8 lattice quantization,
  a conditional probability model of lattice coordinates, resolution
  selection from sampled storage estimates, entropy coding in independently
  decodable tiles, BF16/FP16/FP8/INT8 containers;
* EntroPack API reference page, ``compress``: a non-empty 2-D tensor of
  finite values; some encoding failures return an uncompressed ``"raw"``
  container;
* EntroPack API reference page, ``CompressedTensor``:
  ``actual_bpp = 8 * storage_nbytes() / prod(shape)``, header included;
* EntroPack README, "Direct tensor compression" and configuration table:
  ``0.001 <= target_bpp <= 11``; Compressed Linear usage page: FP8/INT8 code
  containers take ``target_bpp < 8``.

What pins each function (tests under ``tests/``, ``-m "not gpu"``):

* ``e8_nearest``: brute-force enumeration of E8 points in numpy (independent
  code), near-tie inputs, E8 membership, covering radius, idempotence,
  translation invariance, the 240 minimal vectors, and the Monte-Carlo
  normalized second moment against G(E8) = 929/12960.
* ``rans_encode``/``rans_decode`` and the tile coder: exact symbol round trip,
  size against the information content (within the state overhead), the
  uniform-table special case (k raw bits per symbol exactly), the end-state
  invariant.
* ``normalize``: sums to M, no used symbol dropped, closed-form cases.
* the model: every decoded vector lies in E8, contexts recomputable.
* ``compress``/``decompress``: decode equals direct quantize-and-reconstruct
  (the closed definition: rANS is lossless), ``actual_bpp * numel / 8`` equals
  the byte count, the rate lands within 2% of the target, and the relative L2
  error matches high-rate lattice theory within a loose band.
* conversions: against torch CPU's own BF16/FP16/FP8-E4M3FN conversions and
  round-half-even for INT8, as library special cases.
"""
from __future__ import annotations

import ctypes
import os
import subprocess

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "oracle.c")
_LIB = os.path.join(_HERE, "liboracle.so")

OK, WARN_RAW = 0, 1
ERR_ARG, ERR_SHAPE, ERR_NONFINITE, ERR_TARGET, ERR_FORMAT, ERR_NOMEM = -1, -2, -3, -4, -5, -7
BF16, FP16, FP8, INT8 = 0, 1, 2, 3
PROB_BITS = 10
N_STATES = 64
TILE_VECS = 1024
STATE_L = 1 << 11
LAYOUT_ROWS, LAYOUT_BLOCKS = 0, 1


def build(force: bool = False) -> str:
    """Compile oracle.c into liboracle.so with gcc (no fast-math, no FMA)."""
    if force or not os.path.exists(_LIB) or os.path.getmtime(_LIB) < os.path.getmtime(_SRC):
        tmp = _LIB + ".tmp"
        subprocess.check_call(["gcc", "-O2", "-std=c99", "-Wall", "-ffp-contract=off", "-fno-fast-math",
                               "-fPIC", "-shared", "-o", tmp, _SRC, "-lm"])
        os.replace(tmp, _LIB)
    return _LIB


_lib = None


def lib():
    global _lib
    if _lib is None:
        build()
        L = ctypes.CDLL(_LIB)
        P = ctypes.POINTER
        u8p, u16p, i16p, i32p, u32p, u64p, i64p, f32p, f64p = (
            P(ctypes.c_uint8), P(ctypes.c_uint16), P(ctypes.c_int16), P(ctypes.c_int32), P(ctypes.c_uint32),
            P(ctypes.c_uint64), P(ctypes.c_int64), P(ctypes.c_float), P(ctypes.c_double))
        L.or_e8_nearest.argtypes = [f64p, i32p]
        L.or_compress.argtypes = [f64p, ctypes.c_void_p, ctypes.c_int64, ctypes.c_int64, ctypes.c_int, ctypes.c_double,
                                  ctypes.c_double, ctypes.c_int, ctypes.c_int64, ctypes.c_int64, ctypes.c_uint64,
                                  ctypes.c_int, ctypes.c_int, ctypes.c_int, P(u8p), P(ctypes.c_size_t), f64p]
        L.or_last_encode_count.argtypes = []
        L.or_last_encode_count.restype = ctypes.c_long
        L.or_estimate_bpp.argtypes = [f64p, ctypes.c_int64, ctypes.c_int64, ctypes.c_double, ctypes.c_int,
                                      ctypes.c_int64, ctypes.c_int64, ctypes.c_uint64, ctypes.c_int, ctypes.c_int]
        L.or_estimate_bpp.restype = ctypes.c_double
        L.or_free.argtypes = [ctypes.c_void_p]
        L.or_quantize_matrix.argtypes = [f64p, ctypes.c_int64, ctypes.c_int64, ctypes.c_double, ctypes.c_int, f32p,
                                         i32p]
        L.or_decode_symbols.argtypes = [u8p, ctypes.c_size_t, i16p]
        L.or_decompress.argtypes = [u8p, ctypes.c_size_t, ctypes.c_void_p]
        L.or_decompress_tiles.argtypes = [u8p, ctypes.c_size_t, ctypes.c_int64, ctypes.c_int64, i32p,
                                          ctypes.c_void_p]
        L.or_reconstruct.argtypes = [i32p, f32p, ctypes.c_int64, ctypes.c_int64, ctypes.c_int, ctypes.c_void_p]
        L.or_blob_info.argtypes = [u8p, ctypes.c_size_t, i64p, f64p]
        L.or_f32_to_bf16.argtypes = [ctypes.c_float]
        L.or_f32_to_bf16.restype = ctypes.c_uint16
        L.or_f32_to_f16.argtypes = [ctypes.c_float]
        L.or_f32_to_f16.restype = ctypes.c_uint16
        L.or_f32_to_e4m3fn.argtypes = [ctypes.c_float]
        L.or_f32_to_e4m3fn.restype = ctypes.c_uint8
        L.or_f32_to_int8.argtypes = [ctypes.c_float]
        L.or_f32_to_int8.restype = ctypes.c_int8
        L.or_rans_encode.argtypes = [u32p, ctypes.c_int, ctypes.c_int, i32p, ctypes.c_int64, ctypes.c_int, u32p, u16p,
                                     i64p, ctypes.c_int64]
        L.or_rans_decode.argtypes = [u32p, ctypes.c_int, ctypes.c_int, u32p, ctypes.c_int, u16p, ctypes.c_int64,
                                     ctypes.c_int64, i32p, u32p]
        L.or_normalize.argtypes = [u64p, ctypes.c_int, ctypes.c_int, u32p, P(ctypes.c_int)]
        L.or_vector_symbols.argtypes = [i32p, i32p, i32p]
        _lib = L
    return _lib


def _ptr(a: np.ndarray, ctype):
    return a.ctypes.data_as(ctypes.POINTER(ctype))


class OracleError(RuntimeError):
    def __init__(self, rc: int, what: str):
        super().__init__(f"oracle {what} failed with status {rc}")
        self.rc = rc


# ---------------------------------------------------------------------------
# container helpers: the oracle takes f64 values widened exactly from the
# container plus the container's own bytes (for the raw fallback)
# ---------------------------------------------------------------------------
def _as_container(t):
    import torch
    dt = {torch.bfloat16: BF16, torch.float16: FP16, torch.float8_e4m3fn: FP8, torch.int8: INT8}[t.dtype]
    t = t.contiguous().cpu()
    x = t.to(torch.float64).numpy()
    raw = t.view(torch.uint8).numpy() if t.element_size() == 1 else t.view(torch.int16).numpy()
    return dt, np.ascontiguousarray(x), np.ascontiguousarray(raw)


def e8_nearest(u) -> np.ndarray:
    """v = 2 * nearest E8 point (int32[8])."""
    u = np.ascontiguousarray(u, dtype=np.float64)
    assert u.shape == (8,)
    v = np.zeros(8, np.int32)
    lib().or_e8_nearest(_ptr(u, ctypes.c_double), _ptr(v, ctypes.c_int32))
    return v


def compress(t, target_bpp: float, fixed_a: float = 0.0, n_states: int = 0, prob_bits: int = PROB_BITS,
             exact_select: bool = False, tile_vecs: int = 0, sample_vecs: int = 0, seed: int = 0,
             layout: int = 0):
    """Returns (blob bytes as np.uint8, status, chosen lattice scale a).
    n_states / tile_vecs = 0 pick the tile geometry as the product does (see
    or_compress); sample_vecs = 0 samples 65536 vectors; seed is the sample's
    phase; layout LAYOUT_ROWS (row-major tiles) or LAYOUT_BLOCKS (64 x 64
    weight blocks, BF16 only)."""
    dt, x, raw = _as_container(t)
    if x.ndim != 2:
        raise OracleError(ERR_SHAPE, "compress")
    R, C = x.shape
    out = ctypes.POINTER(ctypes.c_uint8)()
    nb = ctypes.c_size_t(0)
    a = ctypes.c_double(0.0)
    rc = lib().or_compress(_ptr(x, ctypes.c_double), raw.ctypes.data_as(ctypes.c_void_p), R, C, dt,
                           float(target_bpp), float(fixed_a), n_states, tile_vecs, sample_vecs, seed, prob_bits,
                           int(exact_select), int(layout), ctypes.byref(out), ctypes.byref(nb), ctypes.byref(a))
    if rc < 0:
        raise OracleError(rc, "compress")
    blob = np.ctypeslib.as_array(out, shape=(nb.value,)).copy()
    lib().or_free(out)
    return blob, rc, a.value


def compress_status(x: np.ndarray, dtype: int, target_bpp: float) -> int:
    """Status code only, for input-validation tests on arbitrary f64 arrays."""
    x = np.ascontiguousarray(x, dtype=np.float64)
    R, C = (x.shape + (1,))[:2] if x.ndim == 1 else x.shape
    out = ctypes.POINTER(ctypes.c_uint8)()
    nb = ctypes.c_size_t(0)
    a = ctypes.c_double(0.0)
    raw = np.zeros(max(1, x.size * 2), np.uint8)
    rc = lib().or_compress(_ptr(x, ctypes.c_double), raw.ctypes.data_as(ctypes.c_void_p), R, C, dtype,
                           float(target_bpp), 0.0, 0, 0, 0, 0, PROB_BITS, 0, 0, ctypes.byref(out), ctypes.byref(nb),
                           ctypes.byref(a))
    if rc >= 0:
        lib().or_free(out)
    return rc


def last_encode_count() -> int:
    """Full encodes the last compress() ran."""
    return int(lib().or_last_encode_count())


def estimate_bpp(t, a: float, n_states: int = N_STATES, prob_bits: int = PROB_BITS, tile_vecs: int = TILE_VECS,
                 sample_vecs: int = 0, seed: int = 0, layout: int = 0) -> float:
    _, x, _ = _as_container(t)
    R, C = x.shape
    return lib().or_estimate_bpp(_ptr(x, ctypes.c_double), R, C, float(a), n_states, tile_vecs, sample_vecs, seed,
                                 prob_bits, layout)


def quantize_matrix(t, a: float, prob_bits: int = PROB_BITS):
    """Direct quantization without entropy coding: (g f32[R], v int32[R, Cp])."""
    _, x, _ = _as_container(t)
    R, C = x.shape
    Cp = (C + 7) // 8 * 8
    g = np.zeros(R, np.float32)
    v = np.zeros((R, Cp), np.int32)
    rc = lib().or_quantize_matrix(_ptr(x, ctypes.c_double), R, C, float(a), prob_bits, _ptr(g, ctypes.c_float),
                                  _ptr(v, ctypes.c_int32))
    if rc:
        raise OracleError(rc, "quantize_matrix")
    return g, v


def info(blob: np.ndarray) -> dict:
    blob = np.ascontiguousarray(blob, dtype=np.uint8)
    out = np.zeros(10, np.int64)
    a = ctypes.c_double(0.0)
    rc = lib().or_blob_info(_ptr(blob, ctypes.c_uint8), blob.size, _ptr(out, ctypes.c_int64), ctypes.byref(a))
    if rc:
        raise OracleError(rc, "blob_info")
    keys = ["rows", "cols", "method", "dtype", "n_states", "n_tiles", "prob_bits", "n_words", "tile_vecs", "layout"]
    d = dict(zip(keys, (int(v) for v in out)))
    d["a"] = a.value
    return d


def decode_symbols(blob: np.ndarray) -> np.ndarray:
    """Lattice coordinates v (int16, rows x padded cols)."""
    blob = np.ascontiguousarray(blob, dtype=np.uint8)
    d = info(blob)
    v = np.zeros((d["rows"], (d["cols"] + 7) // 8 * 8), np.int16)
    rc = lib().or_decode_symbols(_ptr(blob, ctypes.c_uint8), blob.size, _ptr(v, ctypes.c_int16))
    if rc:
        raise OracleError(rc, "decode_symbols")
    return v


_NP_CONTAINER = {BF16: np.uint16, FP16: np.uint16, FP8: np.uint8, INT8: np.int8}


def decompress_raw(blob: np.ndarray) -> np.ndarray:
    """Decoded container values as raw integer codes (uint16 for BF16/FP16,
    uint8 for FP8, int8 for INT8), rows x cols."""
    blob = np.ascontiguousarray(blob, dtype=np.uint8)
    d = info(blob)
    out = np.zeros((d["rows"], d["cols"]), _NP_CONTAINER[d["dtype"]])
    rc = lib().or_decompress(_ptr(blob, ctypes.c_uint8), blob.size, out.ctypes.data_as(ctypes.c_void_p))
    if rc:
        raise OracleError(rc, "decompress")
    return out


def decompress_raw_threads(blob: np.ndarray, threads: int) -> np.ndarray:
    """decompress_raw with the tiles split into ``threads`` contiguous ranges,
    each decoded by ``or_decompress_tiles`` on its own thread (ctypes releases
    the GIL during the call).  Same arithmetic, same result."""
    from concurrent.futures import ThreadPoolExecutor

    blob = np.ascontiguousarray(blob, dtype=np.uint8)
    d = info(blob)
    if d["method"] != 0:
        return decompress_raw(blob)
    out = np.zeros((d["rows"], d["cols"]), _NP_CONTAINER[d["dtype"]])
    work = np.zeros((d["rows"], (d["cols"] + 7) // 8 * 8), np.int32)
    T = d["n_tiles"]
    bounds = [T * k // threads for k in range(threads + 1)]

    def run(k):
        return lib().or_decompress_tiles(_ptr(blob, ctypes.c_uint8), blob.size, bounds[k], bounds[k + 1],
                                         _ptr(work, ctypes.c_int32), out.ctypes.data)

    with ThreadPoolExecutor(max_workers=threads) as ex:
        rcs = list(ex.map(run, range(threads)))
    for rc in rcs:
        if rc:
            raise OracleError(rc, "decompress_tiles")
    return out


def decompress_tile_range(blob: np.ndarray, t0: int, t1: int, out: np.ndarray | None = None,
                          work: np.ndarray | None = None) -> np.ndarray:
    """Decodes tiles [t0, t1) only, into a full-size container array (other
    elements untouched: zero in a fresh array).  out/work may be passed in to
    reuse them across calls."""
    blob = np.ascontiguousarray(blob, dtype=np.uint8)
    d = info(blob)
    if d["method"] != 0:
        raise OracleError(ERR_ARG, "decompress_tile_range")
    if out is None:
        out = np.zeros((d["rows"], d["cols"]), _NP_CONTAINER[d["dtype"]])
    if work is None:
        work = np.zeros((d["rows"], (d["cols"] + 7) // 8 * 8), np.int32)
    rc = lib().or_decompress_tiles(_ptr(blob, ctypes.c_uint8), blob.size, t0, t1, _ptr(work, ctypes.c_int32),
                                   out.ctypes.data)
    if rc:
        raise OracleError(rc, "decompress_tiles")
    return out


def to_torch(raw: np.ndarray, dtype: int):
    import torch
    t = torch.from_numpy(np.ascontiguousarray(raw))
    return {BF16: lambda: t.view(torch.bfloat16), FP16: lambda: t.view(torch.float16),
            FP8: lambda: t.view(torch.float8_e4m3fn), INT8: lambda: t}[dtype]()


def decompress(blob: np.ndarray):
    """Decoded tensor (torch CPU) in the container dtype."""
    d = info(blob)
    return to_torch(decompress_raw(blob), d["dtype"])


def reconstruct(v: np.ndarray, g: np.ndarray, cols: int, dtype: int) -> np.ndarray:
    """Closed form convert(f32(v * g)) -> raw container codes (rows x cols)."""
    v = np.ascontiguousarray(v, dtype=np.int32)
    g = np.ascontiguousarray(g, dtype=np.float32)
    R = v.shape[0]
    out = np.zeros((R, cols), _NP_CONTAINER[dtype])
    rc = lib().or_reconstruct(_ptr(v, ctypes.c_int32), _ptr(g, ctypes.c_float), R, cols, dtype,
                              out.ctypes.data_as(ctypes.c_void_p))
    if rc:
        raise OracleError(rc, "reconstruct")
    return out


def convert_scalar(y: float, dtype: int) -> int:
    L = lib()
    return {BF16: L.or_f32_to_bf16, FP16: L.or_f32_to_f16, FP8: L.or_f32_to_e4m3fn, INT8: L.or_f32_to_int8}[dtype](y)


def rans_encode(freq, syms, n_states: int, prob_bits: int = PROB_BITS):
    freq = np.ascontiguousarray(freq, dtype=np.uint32)
    syms = np.ascontiguousarray(syms, dtype=np.int32)
    states = np.zeros(n_states, np.uint32)
    cap = syms.size + 16
    words = np.zeros(cap, np.uint16)
    nw = ctypes.c_int64(0)
    rc = lib().or_rans_encode(_ptr(freq, ctypes.c_uint32), freq.size, prob_bits, _ptr(syms, ctypes.c_int32),
                              syms.size, n_states, _ptr(states, ctypes.c_uint32), _ptr(words, ctypes.c_uint16),
                              ctypes.byref(nw), cap)
    if rc:
        raise OracleError(rc, "rans_encode")
    return states, words[: nw.value].copy()


def rans_decode(freq, states, words, n: int, prob_bits: int = PROB_BITS):
    freq = np.ascontiguousarray(freq, dtype=np.uint32)
    states = np.ascontiguousarray(states, dtype=np.uint32)
    words = np.ascontiguousarray(words, dtype=np.uint16)
    syms = np.zeros(n, np.int32)
    final = np.zeros(states.size, np.uint32)
    rc = lib().or_rans_decode(_ptr(freq, ctypes.c_uint32), freq.size, prob_bits, _ptr(states, ctypes.c_uint32),
                              states.size, _ptr(words, ctypes.c_uint16), words.size, n, _ptr(syms, ctypes.c_int32),
                              _ptr(final, ctypes.c_uint32))
    if rc:
        raise OracleError(rc, "rans_decode")
    return syms, final


def normalize(counts, prob_bits: int = PROB_BITS):
    counts = np.ascontiguousarray(counts, dtype=np.uint64)
    f = np.zeros(counts.size + 1, np.uint32)
    n = ctypes.c_int(0)
    rc = lib().or_normalize(_ptr(counts, ctypes.c_uint64), counts.size, prob_bits, _ptr(f, ctypes.c_uint32),
                            ctypes.byref(n))
    if rc:
        raise OracleError(rc, "normalize")
    return f[: n.value].copy()


def vector_symbols(v):
    v = np.ascontiguousarray(v, dtype=np.int32)
    ctx = np.zeros(8, np.int32)
    sym = np.zeros(8, np.int32)
    lib().or_vector_symbols(_ptr(v, ctypes.c_int32), _ptr(ctx, ctypes.c_int32), _ptr(sym, ctypes.c_int32))
    return ctx, sym
