"""Thin ctypes binding to libep.so (include/ep.h).

Argument marshalling only: every step of compression runs in the library's
host encoder (or, for a matrix on the GPU, its gfx950 encoder passes) and
every step of decompression runs in its gfx950 kernels.
PyTorch supplies host/device buffers and the current HIP stream.  There is
no fallback: if libep.so is missing the calls raise.
"""
from __future__ import annotations

import ctypes
import math
import os
import weakref
from dataclasses import dataclass

import numpy as np
import torch

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "libep.so")

BF16, FP16, FP8_E4M3FN, INT8, F32 = 0, 1, 2, 3, 4
LAYOUT_ROWS, LAYOUT_BLOCKS = 0, 1
OK, WARN_RAW = 0, 1
ERR_ARG, ERR_SHAPE, ERR_NONFINITE, ERR_TARGET, ERR_FORMAT, ERR_DEVICE, ERR_NOMEM = -1, -2, -3, -4, -5, -6, -7

_DTYPE_CODE = {torch.bfloat16: BF16, torch.float16: FP16, torch.float8_e4m3fn: FP8_E4M3FN, torch.int8: INT8}
_CODE_DTYPE = {v: k for k, v in _DTYPE_CODE.items()}

EXPORTS = ["ep_compress", "ep_compress_ex", "ep_compress_device", "ep_compress_device_noalloc", "ep_free",
           "ep_decompress", "ep_decode_symbols", "ep_actual_bpp", "ep_storage_nbytes", "ep_blob_info", "ep_last_error",
           "ep_last_encode_count", "ep_plan_create", "ep_plan_decompress", "ep_plan_free", "ep_linear",
           "ep_linear_workspace_bytes", "ep_linear_plan_create", "ep_linear_plan_workspace_bytes", "ep_linear_plan_run",
           "ep_linear_plan_free"]


class EPError(RuntimeError):
    def __init__(self, code: int, what: str, msg: str):
        super().__init__(f"{what} failed ({code}): {msg}")
        self.code = code


class _Options(ctypes.Structure):
    _fields_ = [("fixed_scale", ctypes.c_double), ("n_threads", ctypes.c_int), ("n_states", ctypes.c_int),
                ("tile_vecs", ctypes.c_int), ("sample_vecs", ctypes.c_int), ("seed", ctypes.c_uint64),
                ("layout", ctypes.c_int), ("reserved", ctypes.c_int * 3)]


class _Info(ctypes.Structure):
    _fields_ = [("rows", ctypes.c_int64), ("cols", ctypes.c_int64), ("dtype", ctypes.c_int), ("method", ctypes.c_int),
                ("n_states", ctypes.c_int), ("tile_vecs", ctypes.c_int), ("prob_bits", ctypes.c_int),
                ("n_tiles", ctypes.c_int64), ("n_words", ctypes.c_int64), ("scale_a", ctypes.c_double),
                ("target_bpp", ctypes.c_double), ("layout", ctypes.c_int)]


def _options(fixed_scale=0.0, n_threads=0, n_states=0, tile_vecs=0, sample_vecs=0, seed=0, layout=0) -> _Options:
    return _Options(float(fixed_scale), int(n_threads), int(n_states), int(tile_vecs), int(sample_vecs), int(seed),
                    int(layout), (ctypes.c_int * 3)())


_lib = None


def lib() -> ctypes.CDLL:
    """Loads libep.so; raises if it has not been built."""
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            raise RuntimeError(f"{LIB_PATH} is missing: build it with decode_tile_interleaved_amd/build.py")
        L = ctypes.CDLL(LIB_PATH)
        u8p = ctypes.POINTER(ctypes.c_uint8)
        L.ep_compress.argtypes = [ctypes.c_void_p, ctypes.c_int, ctypes.c_int64, ctypes.c_int64, ctypes.c_double,
                                  ctypes.POINTER(u8p), ctypes.POINTER(ctypes.c_size_t)]
        L.ep_compress_ex.argtypes = [ctypes.c_void_p, ctypes.c_int, ctypes.c_int64, ctypes.c_int64, ctypes.c_double,
                                     ctypes.POINTER(_Options), ctypes.POINTER(u8p), ctypes.POINTER(ctypes.c_size_t)]
        L.ep_compress_device.argtypes = [ctypes.c_void_p, ctypes.c_int, ctypes.c_int64, ctypes.c_int64,
                                         ctypes.c_double, ctypes.POINTER(_Options), ctypes.c_void_p,
                                         ctypes.POINTER(u8p), ctypes.POINTER(ctypes.c_size_t)]
        L.ep_compress_device_noalloc.argtypes = [ctypes.c_void_p, ctypes.c_int, ctypes.c_int64, ctypes.c_int64,
                                                 ctypes.c_double, ctypes.POINTER(_Options), ctypes.c_void_p,
                                                 ctypes.c_void_p, ctypes.c_size_t, ctypes.POINTER(ctypes.c_size_t)]
        L.ep_free.argtypes = [u8p]
        L.ep_free.restype = None
        L.ep_decompress.argtypes = [ctypes.c_void_p, ctypes.c_size_t, ctypes.c_void_p, ctypes.c_void_p, ctypes.c_int,
                                    ctypes.c_void_p]
        L.ep_decode_symbols.argtypes = [ctypes.c_void_p, ctypes.c_size_t, ctypes.c_void_p, ctypes.c_void_p,
                                        ctypes.c_void_p]
        L.ep_actual_bpp.argtypes = [ctypes.c_void_p, ctypes.c_size_t]
        L.ep_actual_bpp.restype = ctypes.c_double
        L.ep_storage_nbytes.argtypes = [ctypes.c_void_p, ctypes.c_size_t, ctypes.c_int]
        L.ep_storage_nbytes.restype = ctypes.c_int64
        L.ep_blob_info.argtypes = [ctypes.c_void_p, ctypes.c_size_t, ctypes.POINTER(_Info)]
        L.ep_last_error.argtypes = []
        L.ep_last_error.restype = ctypes.c_char_p
        L.ep_plan_create.argtypes = [ctypes.c_void_p, ctypes.c_size_t, ctypes.c_void_p, ctypes.c_int,
                                     ctypes.POINTER(ctypes.c_void_p)]
        L.ep_plan_decompress.argtypes = [ctypes.c_void_p, ctypes.c_void_p, ctypes.c_void_p]
        L.ep_plan_free.argtypes = [ctypes.c_void_p]
        L.ep_plan_free.restype = None
        L.ep_linear.argtypes = [ctypes.c_void_p, ctypes.c_size_t, ctypes.c_void_p, ctypes.c_void_p, ctypes.c_int64,
                                ctypes.c_void_p, ctypes.c_int, ctypes.c_void_p, ctypes.c_size_t, ctypes.c_void_p]
        L.ep_linear_workspace_bytes.argtypes = [ctypes.c_void_p, ctypes.c_size_t, ctypes.c_int64]
        L.ep_linear_workspace_bytes.restype = ctypes.c_int64
        L.ep_linear_plan_create.argtypes = [ctypes.c_void_p, ctypes.c_size_t, ctypes.c_void_p, ctypes.c_int64,
                                            ctypes.POINTER(ctypes.c_void_p)]
        L.ep_linear_plan_workspace_bytes.argtypes = [ctypes.c_void_p]
        L.ep_linear_plan_workspace_bytes.restype = ctypes.c_int64
        L.ep_linear_plan_run.argtypes = [ctypes.c_void_p, ctypes.c_void_p, ctypes.c_void_p, ctypes.c_int,
                                         ctypes.c_void_p, ctypes.c_size_t, ctypes.c_void_p]
        L.ep_linear_plan_free.argtypes = [ctypes.c_void_p]
        L.ep_linear_plan_free.restype = None
        L.ep_last_encode_count.argtypes = []
        L.ep_last_encode_count.restype = ctypes.c_int64
        _lib = L
    return _lib


def last_error() -> str:
    return lib().ep_last_error().decode()


def _check(code: int, what: str) -> int:
    if code < 0:
        raise EPError(code, what, last_error())
    return code


@dataclass
class Packed:
    """A compressed matrix: the stream on the host, optionally on a device."""
    blob: np.ndarray                  # uint8 stream (host)
    status: int                       # OK or WARN_RAW
    shape: tuple
    dtype: torch.dtype
    dev: torch.Tensor | None = None   # the same bytes on a GPU

    @property
    def nbytes(self) -> int:
        return int(self.blob.size)

    @property
    def actual_bpp(self) -> float:
        return actual_bpp(self.blob)

    def info(self) -> dict:
        return blob_info(self.blob)

    def to(self, device) -> "Packed":
        """Copies the stream to `device` (a torch uint8 tensor)."""
        self.dev = torch.from_numpy(self.blob).to(device)
        return self


def _take_blob(ptr, n: int) -> np.ndarray:
    """The library's malloc'ed stream as a uint8 array, without a copy; the
    memory goes back to ep_free once the array and every view of it are gone."""
    arr = np.ctypeslib.as_array(ptr, shape=(n,))
    weakref.finalize(arr.base, lib().ep_free, ptr)
    return arr


def _host_ptr(a: np.ndarray) -> int:
    return a.ctypes.data


def compress(t: torch.Tensor, target_bpp: float, fixed_scale: float = 0.0, n_threads: int = 0, n_states: int = 0,
             tile_vecs: int = 0, sample_vecs: int = 0, seed: int = 0, layout: int = LAYOUT_ROWS) -> Packed:
    """ep_compress_ex on a 2-D CPU tensor (BF16, FP16, FP8-E4M3FN or INT8);
    the keyword arguments are the ep_options fields."""
    if t.dtype not in _DTYPE_CODE:
        raise EPError(ERR_ARG, "compress", f"unsupported dtype {t.dtype}")
    if t.dim() != 2:
        raise EPError(ERR_SHAPE, "compress", "input must be 2-D")
    t = t.detach().to("cpu").contiguous()
    opt = _options(fixed_scale, n_threads, n_states, tile_vecs, sample_vecs, seed, layout)
    out = ctypes.POINTER(ctypes.c_uint8)()
    nb = ctypes.c_size_t(0)
    src = t.view(torch.uint8) if t.element_size() == 1 else t.view(torch.int16)
    rc = lib().ep_compress_ex(ctypes.c_void_p(src.data_ptr() if t.numel() else 0), _DTYPE_CODE[t.dtype],
                              t.shape[0], t.shape[1], float(target_bpp), ctypes.byref(opt), ctypes.byref(out),
                              ctypes.byref(nb))
    _check(rc, "ep_compress")
    return Packed(blob=_take_blob(out, nb.value), status=rc, shape=tuple(t.shape), dtype=t.dtype)


def compress_device(t: torch.Tensor, target_bpp: float, fixed_scale: float = 0.0, stream=None, n_states: int = 0,
                    tile_vecs: int = 0, sample_vecs: int = 0, seed: int = 0) -> Packed:
    """ep_compress_device on a 2-D tensor in GPU memory: the same stream as
    compress() of the same values, with the passes over the matrix on the GPU
    (on `stream`, default: the current stream, synchronized on return)."""
    if t.dtype not in _DTYPE_CODE:
        raise EPError(ERR_ARG, "compress_device", f"unsupported dtype {t.dtype}")
    if t.dim() != 2:
        raise EPError(ERR_SHAPE, "compress_device", "input must be 2-D")
    if not t.is_cuda:
        raise EPError(ERR_ARG, "compress_device", "input must be on a GPU")
    t = t.detach().contiguous()
    if stream is None:
        stream = torch.cuda.current_stream(t.device)
    opt = _options(fixed_scale, 0, n_states, tile_vecs, sample_vecs, seed)
    out = ctypes.POINTER(ctypes.c_uint8)()
    nb = ctypes.c_size_t(0)
    with torch.cuda.device(t.device):
        rc = lib().ep_compress_device(ctypes.c_void_p(t.data_ptr() if t.numel() else 0), _DTYPE_CODE[t.dtype],
                                      t.shape[0], t.shape[1], float(target_bpp), ctypes.byref(opt),
                                      ctypes.c_void_p(stream.cuda_stream), ctypes.byref(out), ctypes.byref(nb))
    _check(rc, "ep_compress_device")
    return Packed(blob=_take_blob(out, nb.value), status=rc, shape=tuple(t.shape), dtype=t.dtype)


def last_encode_count() -> int:
    """ep_last_encode_count: full encodes of the last compress on this thread."""
    return int(lib().ep_last_encode_count())


def actual_bpp(blob: np.ndarray) -> float:
    v = lib().ep_actual_bpp(_host_ptr(blob), blob.size)
    if math.isnan(v):
        raise EPError(ERR_FORMAT, "ep_actual_bpp", last_error())
    return v


def storage_nbytes(blob: np.ndarray, include_header: bool = True) -> int:
    return _check(lib().ep_storage_nbytes(_host_ptr(blob), blob.size, int(include_header)), "ep_storage_nbytes")


def blob_info(blob: np.ndarray) -> dict:
    info = _Info()
    _check(lib().ep_blob_info(_host_ptr(blob), blob.size, ctypes.byref(info)), "ep_blob_info")
    return {name: getattr(info, name) for name, _ in _Info._fields_}


def _stream_handle(stream) -> int:
    s = stream if stream is not None else torch.cuda.current_stream()
    return int(s.cuda_stream)


def decompress(p: Packed, out: torch.Tensor | None = None, stream=None) -> torch.Tensor:
    """ep_decompress: enqueues the fused decode on `stream` (default: the
    current stream) into `out` (allocated if None) and returns it."""
    if p.dev is None:
        raise EPError(ERR_ARG, "decompress", "stream is not on a device; call Packed.to('cuda') first")
    rows, cols = p.shape
    if out is None:
        out = torch.empty(rows, cols, dtype=p.dtype, device=p.dev.device)
    if out.dtype != p.dtype or tuple(out.shape) != (rows, cols) or not out.is_contiguous():
        raise EPError(ERR_ARG, "decompress", "out must be a contiguous tensor of the stored shape and dtype")
    rc = lib().ep_decompress(_host_ptr(p.blob), p.blob.size, ctypes.c_void_p(p.dev.data_ptr()),
                             ctypes.c_void_p(out.data_ptr()), -1, ctypes.c_void_p(_stream_handle(stream)))
    _check(rc, "ep_decompress")
    return out


class DecodePlan:
    """ep_plan_create / ep_plan_decompress: a Packed stream's decode with its
    host-side checks and launch geometry computed once.  Holds a reference to
    the stream's device copy, which must not be modified while the plan lives."""

    def __init__(self, p: Packed):
        if p.dev is None:
            raise EPError(ERR_ARG, "plan", "stream is not on a device; call Packed.to('cuda') first")
        self.shape, self.dtype, self._dev = p.shape, p.dtype, p.dev
        h = ctypes.c_void_p()
        _check(lib().ep_plan_create(_host_ptr(p.blob), p.blob.size, ctypes.c_void_p(p.dev.data_ptr()), -1,
                                    ctypes.byref(h)), "ep_plan_create")
        self._h = h
        self._free = weakref.finalize(self, lib().ep_plan_free, h)

    def decompress(self, out: torch.Tensor | None = None, stream=None) -> torch.Tensor:
        rows, cols = self.shape
        if out is None:
            out = torch.empty(rows, cols, dtype=self.dtype, device=self._dev.device)
        if out.dtype != self.dtype or tuple(out.shape) != (rows, cols) or not out.is_contiguous():
            raise EPError(ERR_ARG, "plan.decompress", "out must be a contiguous tensor of the stored shape and dtype")
        _check(lib().ep_plan_decompress(self._h, ctypes.c_void_p(out.data_ptr()),
                                        ctypes.c_void_p(_stream_handle(stream))), "ep_plan_decompress")
        return out

    def close(self) -> None:
        self._free()


def plan(p: Packed) -> DecodePlan:
    """A decode plan for p (see DecodePlan)."""
    return DecodePlan(p)


def decode_symbols(p: Packed, out: torch.Tensor | None = None, stream=None) -> torch.Tensor:
    """ep_decode_symbols: the lattice coordinates v (int16, rows x cols8)."""
    if p.dev is None:
        raise EPError(ERR_ARG, "decode_symbols", "stream is not on a device; call Packed.to('cuda') first")
    rows, cols = p.shape
    cols8 = (cols + 7) // 8 * 8
    if out is None:
        out = torch.empty(rows, cols8, dtype=torch.int16, device=p.dev.device)
    rc = lib().ep_decode_symbols(_host_ptr(p.blob), p.blob.size, ctypes.c_void_p(p.dev.data_ptr()),
                                 ctypes.c_void_p(out.data_ptr()), ctypes.c_void_p(_stream_handle(stream)))
    _check(rc, "ep_decode_symbols")
    return out


def from_blob(blob: np.ndarray) -> Packed:
    """Wraps an existing stream (for example one written elsewhere)."""
    d = blob_info(blob)
    return Packed(blob=np.ascontiguousarray(blob, dtype=np.uint8), status=OK if d["method"] == 0 else WARN_RAW,
                  shape=(d["rows"], d["cols"]), dtype=_CODE_DTYPE[d["dtype"]])


def linear_workspace_bytes(p: Packed, m: int) -> int:
    """ep_linear_workspace_bytes: device scratch ep_linear uses for m rows."""
    return _check(lib().ep_linear_workspace_bytes(_host_ptr(p.blob), p.blob.size, m), "ep_linear_workspace_bytes")


def linear(p: Packed, x: torch.Tensor, out: torch.Tensor | None = None, out_dtype: torch.dtype = torch.bfloat16,
           stream=None, workspace: torch.Tensor | None = None) -> torch.Tensor:
    """ep_linear: Y = X W^T with W decoded inside the product (p: a BF16
    stream in the blocks layout, on the device; x: BF16, m x cols of W, on
    the same device).  Y is m x rows of W, BF16 or FP32.  workspace: a
    device tensor of at least linear_workspace_bytes(p, m) bytes (allocated
    here when None and needed; pass an empty tensor to forbid the split)."""
    if p.dev is None:
        raise EPError(ERR_ARG, "linear", "stream is not on a device; call Packed.to('cuda') first")
    rows, cols = p.shape
    if x.dtype != torch.bfloat16 or x.dim() != 2 or x.shape[1] != cols or not x.is_contiguous():
        raise EPError(ERR_ARG, "linear", "x must be a contiguous BF16 m x cols tensor")
    if out_dtype not in (torch.bfloat16, torch.float32):
        raise EPError(ERR_ARG, "linear", "out_dtype must be bfloat16 or float32")
    m = x.shape[0]
    if out is None:
        out = torch.empty(m, rows, dtype=out_dtype, device=p.dev.device)
    if out.dtype != out_dtype or tuple(out.shape) != (m, rows) or not out.is_contiguous():
        raise EPError(ERR_ARG, "linear", "out must be a contiguous m x rows tensor of out_dtype")
    if workspace is None:
        need = linear_workspace_bytes(p, m)
        workspace = torch.empty(need, dtype=torch.uint8, device=p.dev.device)
    ws_bytes = workspace.numel() * workspace.element_size()
    rc = lib().ep_linear(_host_ptr(p.blob), p.blob.size, ctypes.c_void_p(p.dev.data_ptr()),
                         ctypes.c_void_p(x.data_ptr() if m else 0), m,
                         ctypes.c_void_p(out.data_ptr() if m else 0),
                         F32 if out_dtype == torch.float32 else BF16,
                         ctypes.c_void_p(workspace.data_ptr() if ws_bytes else 0), ws_bytes,
                         ctypes.c_void_p(_stream_handle(stream)))
    _check(rc, "ep_linear")
    return out


class LinearPlan:
    """ep_linear_plan_*: ep_linear on one stream and row count with its host
    work done once.  Holds a reference to the stream's device copy, which
    must not be modified while the plan lives, and its own workspace."""

    def __init__(self, p: Packed, m: int):
        if p.dev is None:
            raise EPError(ERR_ARG, "linear plan", "stream is not on a device; call Packed.to('cuda') first")
        self.shape, self.m, self._dev = p.shape, int(m), p.dev
        h = ctypes.c_void_p()
        _check(lib().ep_linear_plan_create(_host_ptr(p.blob), p.blob.size, ctypes.c_void_p(p.dev.data_ptr()), self.m,
                                           ctypes.byref(h)), "ep_linear_plan_create")
        self._h = h
        self._free = weakref.finalize(self, lib().ep_linear_plan_free, h)
        need = _check(lib().ep_linear_plan_workspace_bytes(h), "ep_linear_plan_workspace_bytes")
        self.workspace = torch.empty(need, dtype=torch.uint8, device=p.dev.device)

    def run(self, x: torch.Tensor, out: torch.Tensor | None = None, out_dtype: torch.dtype = torch.bfloat16,
            stream=None) -> torch.Tensor:
        rows, cols = self.shape
        if x.dtype != torch.bfloat16 or tuple(x.shape) != (self.m, cols) or not x.is_contiguous():
            raise EPError(ERR_ARG, "linear plan", "x must be a contiguous BF16 m x cols tensor")
        if out is None:
            out = torch.empty(self.m, rows, dtype=out_dtype, device=self._dev.device)
        if out.dtype != out_dtype or tuple(out.shape) != (self.m, rows) or not out.is_contiguous():
            raise EPError(ERR_ARG, "linear plan", "out must be a contiguous m x rows tensor of out_dtype")
        ws = self.workspace
        _check(lib().ep_linear_plan_run(self._h, ctypes.c_void_p(x.data_ptr() if self.m else 0),
                                        ctypes.c_void_p(out.data_ptr() if self.m else 0),
                                        F32 if out_dtype == torch.float32 else BF16,
                                        ctypes.c_void_p(ws.data_ptr() if ws.numel() else 0), ws.numel(),
                                        ctypes.c_void_p(_stream_handle(stream))), "ep_linear_plan_run")
        return out

    def close(self) -> None:
        self._free()
