"""Python binding of libncc.so: NCC template matching with summed-area tables
on MI355X (gfx950).

This module only marshals torch tensors (device memory and streams) into the C
ABI declared in ``include/ncc.h``; every step of the computation runs in the
library's HIP kernels.  The library must be built (``python -m
normalized_cross_correlation_amd.build``); without it every call raises.

Functions take and return torch tensors on a ROCm device and enqueue work on
the tensor device's current torch stream:

* ``sat_build(img)``             -> (S, Q) int64 summed-area tables
* ``box(S, rects)``              -> int64 four-corner box sums
* ``correlate(img, tpl, sums)``  -> (coef float32 [n][Ho][Wo], sums int32 or None)
* ``correlate_rect(img, tpl, x0, y0, w, h)`` -> the same over a w x h rectangle
  of positions, read in place from a row-strided image, written to row-strided
  output
* ``set_option(name, value)``, ``get_option(name)``, ``options(**settings)``
  (a context manager restoring the previous values): the process-wide route
  and tuning options of ``ncc_set_option``
* ``stream_status()``  -> waits for the current stream; raises NCCError when a
  single-pass table build on it reported a failure

``correlate`` and ``correlate_rect`` take ``tables=(S, Q)``, summed-area
tables of the whole image from ``sat_build``, for the routes that read them.
"""
from __future__ import annotations

import ctypes
import os

__all__ = ["sat_build", "box", "correlate", "correlate_rect", "release", "lib", "NCCError",
           "set_option", "get_option", "options", "stream_status", "OPTIONS", "ROUTES",
           "ABI_FUNCTIONS", "LIB_PATH", "MAX_WIDTH", "MAX_TEMPLATE_PIXELS"]

LIB_PATH = os.path.join(os.path.dirname(os.path.abspath(__file__)), "libncc.so")
ABI_FUNCTIONS = ("ncc_sat_build", "ncc_sat_build_noalloc", "ncc_box", "ncc_correlate", "ncc_correlate_rect",
                 "ncc_set_option", "ncc_get_option", "ncc_stream_status",
                 "ncc_strerror", "ncc_release", "ncc_version")
ABI_VERSION = 201
# option numbers and values of ncc.h
OPTIONS = {"route": 1, "sat_build": 2, "tz_strip": 3, "stream_rows": 4, "sat_spin": 5,
           "sat_stale": 6}
ROUTES = {"auto": 0, "generic": 1, "fft": 2, "single": 3, "dot4": 4, "tile": 5}
SAT_BUILDS = {"two_pass": 0, "single_pass": 1}
MAX_WIDTH = 66051
MAX_TEMPLATE_PIXELS = 33025
MAX_OUT_PITCH = 1 << 24

_lib = None


class NCCError(RuntimeError):
    def __init__(self, fn: str, code: int, msg: str):
        super().__init__("%s failed: %s (%d)" % (fn, msg, code))
        self.code = code


def lib():
    """The loaded libncc.so (ctypes), with argument types set."""
    global _lib
    if _lib is None:
        import torch  # noqa: F401  (loads torch's HIP runtime first; libncc shares it)
        if not os.path.exists(LIB_PATH):
            raise RuntimeError("libncc.so is not built: run `python -m "
                               "normalized_cross_correlation_amd.build` (%s)" % LIB_PATH)
        L = ctypes.CDLL(LIB_PATH)
        P, I, I64 = ctypes.c_void_p, ctypes.c_int, ctypes.c_int64
        L.ncc_sat_build.argtypes = [P, I, I, P, P, P]
        L.ncc_sat_build.restype = I
        L.ncc_sat_build_noalloc.argtypes = [P, I, I, P, P, P]
        L.ncc_sat_build_noalloc.restype = I
        L.ncc_box.argtypes = [P, I, I, P, I64, P, P]
        L.ncc_box.restype = I
        L.ncc_correlate.argtypes = [P, I, I, P, I, I, I, P, P, P, P, P]
        L.ncc_correlate.restype = I
        Z = ctypes.c_size_t
        L.ncc_correlate_rect.argtypes = [P, I, I, Z, P, I, I, I, I, I, I, I, Z, P, P, P, P, P]
        L.ncc_correlate_rect.restype = I
        L.ncc_set_option.argtypes = [I, I]
        L.ncc_set_option.restype = I
        L.ncc_get_option.argtypes = [I, ctypes.POINTER(I)]
        L.ncc_get_option.restype = I
        L.ncc_stream_status.argtypes = [P]
        L.ncc_stream_status.restype = I
        L.ncc_strerror.argtypes = [I]
        L.ncc_strerror.restype = ctypes.c_char_p
        L.ncc_release.argtypes = []
        L.ncc_release.restype = None
        L.ncc_version.argtypes = []
        L.ncc_version.restype = I
        if L.ncc_version() != ABI_VERSION:
            raise RuntimeError("libncc.so ABI %d, binding expects %d: rebuild the library"
                               % (L.ncc_version(), ABI_VERSION))
        _lib = L
    return _lib


def _check(fn: str, rc: int):
    if rc != 0:
        raise NCCError(fn, rc, lib().ncc_strerror(rc).decode())


def _stream(t):
    import torch
    return ctypes.c_void_p(torch.cuda.current_stream(t.device).cuda_stream)


def _dev_tensor(t, dtype, name, ndim=None):
    import torch
    if not isinstance(t, torch.Tensor):
        raise TypeError("%s must be a torch.Tensor" % name)
    if t.device.type != "cuda":
        raise ValueError("%s must be on a ROCm device" % name)
    if t.dtype != dtype:
        raise TypeError("%s must be %s, got %s" % (name, dtype, t.dtype))
    if ndim is not None and t.dim() != ndim:
        raise ValueError("%s must have %d dimensions" % (name, ndim))
    if not t.is_contiguous():
        raise ValueError("%s must be contiguous" % name)
    return t


def sat_build(img, S=None, Q=None):
    """Summed-area tables of a [H][W] uint8 image: S of I and Q of I^2 (int64,
    inclusive).  Pass S, Q to write into existing tensors."""
    import torch
    _dev_tensor(img, torch.uint8, "img", 2)
    H, W = img.shape
    if S is None:
        S = torch.empty((H, W), dtype=torch.int64, device=img.device)
    if Q is None:
        Q = torch.empty((H, W), dtype=torch.int64, device=img.device)
    for name, t in (("S", S), ("Q", Q)):
        _dev_tensor(t, torch.int64, name, 2)
        if tuple(t.shape) != (H, W) or t.device != img.device:
            raise ValueError("%s must be [H][W] on the image's device" % name)
    with torch.cuda.device(img.device):
        _check("ncc_sat_build", lib().ncc_sat_build(
            img.data_ptr(), W, H, S.data_ptr(), Q.data_ptr(), _stream(img)))
    return S, Q


def box(S, rects, out=None):
    """Four-corner box sums of one table S for rects [n][4] int32 {x0,y0,x1,y1}.
    Boxes outside the table give INT64_MIN, empty boxes 0."""
    import torch
    _dev_tensor(S, torch.int64, "S", 2)
    _dev_tensor(rects, torch.int32, "rects", 2)
    if rects.shape[1] != 4:
        raise ValueError("rects must be [n][4]")
    H, W = S.shape
    n = rects.shape[0]
    if out is None:
        out = torch.empty((n,), dtype=torch.int64, device=S.device)
    _dev_tensor(out, torch.int64, "out", 1)
    if out.shape[0] != n:
        raise ValueError("out must have n elements")
    with torch.cuda.device(S.device):
        _check("ncc_box", lib().ncc_box(S.data_ptr(), W, H, rects.data_ptr(), n,
                                        out.data_ptr(), _stream(S)))
    return out


def _tables(tables, H, W, device):
    """Device pointers of a (S, Q) pair of [H][W] int64 tables, or (None, None)."""
    import torch
    if tables is None:
        return None, None
    S, Q = tables
    for name, t in (("S", S), ("Q", Q)):
        _dev_tensor(t, torch.int64, name, 2)
        if tuple(t.shape) != (H, W) or t.device != device:
            raise ValueError("%s must be [H][W] on the image's device" % name)
    return S.data_ptr(), Q.data_ptr()


def correlate(img, tpl, want_sums: bool = False, coef=None, sums=None, tables=None):
    """Valid-mode NCC of a [H][W] uint8 image with a [hT][wT] template or a
    [n][hT][wT] bank.  Returns (coef float32 [n][Ho][Wo], sums int32
    [2+n][Ho][Wo] or None): sums planes are SumI, SumISq, then SumIT per
    template.  tables: optional (S, Q) from sat_build(img)."""
    import torch
    _dev_tensor(img, torch.uint8, "img", 2)
    if tpl.dim() == 2:
        tpl = tpl.unsqueeze(0)
    _dev_tensor(tpl, torch.uint8, "tpl", 3)
    H, W = img.shape
    n, hT, wT = tpl.shape
    Ho, Wo = H - hT + 1, W - wT + 1
    if Ho < 1 or Wo < 1:
        raise ValueError("template larger than the image")
    if coef is None:
        coef = torch.empty((n, Ho, Wo), dtype=torch.float32, device=img.device)
    _dev_tensor(coef, torch.float32, "coef", 3)
    if tuple(coef.shape) != (n, Ho, Wo):
        raise ValueError("coef must be [n][Ho][Wo]")
    if want_sums and sums is None:
        sums = torch.empty((2 + n, Ho, Wo), dtype=torch.int32, device=img.device)
    if sums is not None:
        _dev_tensor(sums, torch.int32, "sums", 3)
        if tuple(sums.shape) != (2 + n, Ho, Wo):
            raise ValueError("sums must be [2+n][Ho][Wo]")
    pS, pQ = _tables(tables, H, W, img.device)
    with torch.cuda.device(img.device):
        _check("ncc_correlate", lib().ncc_correlate(
            img.data_ptr(), W, H, tpl.data_ptr(), wT, hT, n,
            sums.data_ptr() if sums is not None else None, coef.data_ptr(), pS, pQ, _stream(img)))
    return coef, sums


def _row_strided(t, dtype, name, ndim):
    """A tensor whose last dimension is dense (rows may be strided)."""
    import torch
    if not isinstance(t, torch.Tensor):
        raise TypeError("%s must be a torch.Tensor" % name)
    if t.device.type != "cuda":
        raise ValueError("%s must be on a ROCm device" % name)
    if t.dtype != dtype:
        raise TypeError("%s must be %s, got %s" % (name, dtype, t.dtype))
    if t.dim() != ndim:
        raise ValueError("%s must have %d dimensions" % (name, ndim))
    if t.shape[-1] > 1 and t.stride(-1) != 1:
        raise ValueError("%s must have unit stride along its rows" % name)
    return t


def _pitched(t, name, planes, h, w):
    """Row pitch (elements) of a [planes][h][w] output view whose planes are
    h rows apart; None when the view does not fix it (one row in all)."""
    if tuple(t.shape) != (planes, h, w):
        raise ValueError("%s must be [%d][%d][%d]" % (name, planes, h, w))
    if t.numel() == 0 or (h == 1 and planes == 1):
        return None
    pitch = t.stride(1) if h > 1 else t.stride(0)  # h == 1: one row per plane
    if pitch < w or (planes > 1 and t.stride(0) != h * pitch):
        raise ValueError("%s: planes must be h rows apart, rows >= w elements apart" % name)
    return pitch


def correlate_rect(img, tpl, x0: int, y0: int, w: int, h: int, want_sums: bool = False,
                   out_pitch=None, coef=None, sums=None, tables=None):
    """NCC at the positions x0..x0+w-1 by y0..y0+h-1 only (each window inside
    the image).  img is [H][W] uint8 with dense rows (a row-strided view, e.g.
    a crop, is read in place).  Returns (coef float32 [n][h][w], sums int32
    [2+n][h][w] or None), views of buffers whose rows are out_pitch (default
    w) elements apart; coef / sums may be given as such views.  tables:
    optional (S, Q), [H][W] tables of the whole image."""
    import torch
    _row_strided(img, torch.uint8, "img", 2)
    if tpl.dim() == 2:
        tpl = tpl.unsqueeze(0)
    _dev_tensor(tpl, torch.uint8, "tpl", 3)
    H, W = img.shape
    ip = img.stride(0) if H > 1 else W
    n, hT, wT = tpl.shape
    given = [out_pitch] if out_pitch is not None else []
    if coef is not None:
        _row_strided(coef, torch.float32, "coef", 3)
        given.append(_pitched(coef, "coef", n, h, w))
    if sums is not None:
        _row_strided(sums, torch.int32, "sums", 3)
        given.append(_pitched(sums, "sums", 2 + n, h, w))
    given = [p for p in given if p is not None]
    if any(p != given[0] for p in given):
        raise ValueError("out_pitch, coef and sums disagree on the output row pitch")
    out_pitch = given[0] if given else w
    if coef is None:
        coef = torch.empty((n, h, out_pitch), dtype=torch.float32, device=img.device)[:, :, :w]
    if want_sums and sums is None:
        sums = torch.empty((2 + n, h, out_pitch), dtype=torch.int32, device=img.device)[:, :, :w]
    pS, pQ = _tables(tables, H, W, img.device)
    with torch.cuda.device(img.device):
        _check("ncc_correlate_rect", lib().ncc_correlate_rect(
            img.data_ptr(), W, H, ip, tpl.data_ptr(), wT, hT, n, x0, y0, w, h, out_pitch,
            sums.data_ptr() if sums is not None and sums.numel() else None,
            coef.data_ptr() if coef.numel() else None, pS, pQ, _stream(img)))
    return coef, sums


def _option_value(name, value):
    if name == "route" and isinstance(value, str):
        return ROUTES[value]
    if name == "sat_build" and isinstance(value, str):
        return SAT_BUILDS[value]
    return int(value)


def set_option(name: str, value):
    """Sets a process-wide option: route ("auto", "generic", "fft", "single",
    "dot4", "tile"), sat_build ("two_pass", "single_pass"), tz_strip (0, 16,
    32), stream_rows (0, 16, 32, 64), sat_spin (>= 0), sat_stale (0, 1)."""
    _check("ncc_set_option", lib().ncc_set_option(OPTIONS[name], _option_value(name, value)))


def get_option(name: str) -> int:
    v = ctypes.c_int()
    _check("ncc_get_option", lib().ncc_get_option(OPTIONS[name], ctypes.byref(v)))
    return v.value


class options:
    """Context manager: sets the given options, restores the previous values
    on exit (``with options(route="generic", sat_build="single_pass"): ...``)."""

    def __init__(self, **settings):
        self.settings = {k: v for k, v in settings.items() if v is not None}

    def __enter__(self):
        self.old = {k: get_option(k) for k in self.settings}
        for k, v in self.settings.items():
            set_option(k, v)
        return self

    def __exit__(self, *exc):
        for k, v in self.old.items():
            set_option(k, v)


def stream_status(device=None):
    """Waits for the current stream of `device` and raises NCCError if a
    single-pass table build on it reported a failure (ncc_stream_status)."""
    import torch
    d = torch.device("cuda", torch.cuda.current_device()) if device is None else torch.device(device)
    with torch.cuda.device(d):
        _check("ncc_stream_status", lib().ncc_stream_status(
            ctypes.c_void_p(torch.cuda.current_stream(d).cuda_stream)))


def release():
    """Frees the library's cached workspaces."""
    lib().ncc_release()
