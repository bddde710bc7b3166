"""Plain CPU oracle for NCC template matching with summed-area-table denominators.

TEST INFRASTRUCTURE ONLY.  Only ``tests/``, ``__graft_entry__.smoke()`` and the
CPU-baseline leg of ``bench.py`` may import this package.  The GPU library never
imports, links or calls it, and it imports nothing from the GPU library.

The arithmetic lives in ``ncc_oracle.c`` (plain C loops, int64 sums, one IEEE
double evaluation of each coefficient).  This module only compiles it with gcc
and marshals numpy arrays through ctypes.  See the header of ``ncc_oracle.c``
for the passages of The CUDA Handbook ch. 15 that each function follows and for
the readings taken where the pages are silent.

Parity status: every function here is pinned by the ``-m "not gpu"`` tests
(brute force, library routines, closed forms and invariants).  The exact
coefficient formula rests on the textbook Pearson definition, because the pages
do not print the body of their CorrelationValue routine; the pin for it is a
per-window ``numpy.corrcoef`` comparison.
"""
from __future__ import annotations

import ctypes
import os
import subprocess

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "ncc_oracle.c")
_LIB = os.path.join(_HERE, "libncc_oracle.so")
# The planted-mistake tests point this at a deliberately broken build of the
# oracle to show that the pins catch it; nothing else sets it.
_LIB_OVERRIDE = os.environ.get("NCC_ORACLE_MUTANT_LIB")

CFLAGS = ["-O2", "-std=c11", "-fPIC", "-shared", "-fopenmp", "-Wall", "-Wextra"]

_lib = None


def build(force: bool = True) -> str:
    """Compile ncc_oracle.c with gcc (no fast-math) into libncc_oracle.so."""
    if force or not os.path.exists(_LIB):
        tmp = _LIB + ".tmp%d" % os.getpid()
        subprocess.check_call(["gcc", *CFLAGS, _SRC, "-o", tmp, "-lm"])
        os.replace(tmp, _LIB)
    return _LIB


def _load():
    global _lib
    if _lib is None:
        if _LIB_OVERRIDE:
            lib = ctypes.CDLL(_LIB_OVERRIDE)
        else:
            if not os.path.exists(_LIB) or os.path.getmtime(_LIB) < os.path.getmtime(_SRC):
                build()
            lib = ctypes.CDLL(_LIB)
        P = ctypes.c_void_p
        I = ctypes.c_int
        I64 = ctypes.c_int64
        lib.oracle_row_partials.argtypes = [P, I, I, P, P]
        lib.oracle_row_partials.restype = None
        lib.oracle_sat_build.argtypes = [P, I, I, P, P]
        lib.oracle_sat_build.restype = I
        lib.oracle_sat_box.argtypes = [P, I, I, I, I, I, I]
        lib.oracle_sat_box.restype = I64
        lib.oracle_box_batch.argtypes = [P, I, I, P, I64, P]
        lib.oracle_box_batch.restype = None
        lib.oracle_template_stats.argtypes = [P, I, I, P, P, P]
        lib.oracle_template_stats.restype = None
        lib.oracle_coefficient.argtypes = [I64] * 6
        lib.oracle_coefficient.restype = ctypes.c_float
        lib.oracle_correlate.argtypes = [P, I, I, P, I, I, I, P, P, I]
        lib.oracle_correlate.restype = I
        lib.oracle_correlate_at.argtypes = [P, I, I, P, P, P, I, I, I, P, I64, P, P, I]
        lib.oracle_correlate_at.restype = I
        lib.oracle_threads.argtypes = [I]
        lib.oracle_threads.restype = I
        _lib = lib
    return _lib


def _p(a: np.ndarray):
    return a.ctypes.data_as(ctypes.c_void_p)


def _u8_2d(img) -> np.ndarray:
    img = np.ascontiguousarray(img, dtype=np.uint8)
    if img.ndim != 2:
        raise ValueError("image must be 2-D [H][W]")
    return img


def _templates(tpl) -> np.ndarray:
    tpl = np.ascontiguousarray(tpl, dtype=np.uint8)
    if tpl.ndim == 2:
        tpl = tpl[None]
    if tpl.ndim != 3:
        raise ValueError("templates must be [hT][wT] or [nTpl][hT][wT]")
    return tpl


def row_partials(img):
    """uint32 inclusive row running sums (R1 of I, R2 of I^2)."""
    img = _u8_2d(img)
    H, W = img.shape
    r1 = np.empty((H, W), np.uint32)
    r2 = np.empty((H, W), np.uint32)
    _load().oracle_row_partials(_p(img), W, H, _p(r1), _p(r2))
    return r1, r2


def sat_build(img):
    """int64 summed-area tables (S of I, Q of I^2), inclusive, [H][W]."""
    img = _u8_2d(img)
    H, W = img.shape
    S = np.empty((H, W), np.int64)
    Q = np.empty((H, W), np.int64)
    if _load().oracle_sat_build(_p(img), W, H, _p(S), _p(Q)) != 0:
        raise ValueError("bad image size")
    return S, Q


def sat_box(S, x0, y0, x1, y1) -> int:
    """Four-corner box sum over [x0,x1) x [y0,y1)."""
    S = np.ascontiguousarray(S, dtype=np.int64)
    H, W = S.shape
    if not (0 <= x0 <= x1 <= W and 0 <= y0 <= y1 <= H):
        raise ValueError("rectangle outside the table")
    return int(_load().oracle_sat_box(_p(S), W, H, x0, y0, x1, y1))


def box_batch(S, rects):
    """Box sums for rects [n][4] = {x0, y0, x1, y1} (int32)."""
    S = np.ascontiguousarray(S, dtype=np.int64)
    rects = np.ascontiguousarray(rects, dtype=np.int32).reshape(-1, 4)
    H, W = S.shape
    ok = ((rects[:, 0] >= 0) & (rects[:, 0] <= rects[:, 2]) & (rects[:, 2] <= W)
          & (rects[:, 1] >= 0) & (rects[:, 1] <= rects[:, 3]) & (rects[:, 3] <= H))
    if not ok.all():
        raise ValueError("rectangle outside the table")
    out = np.empty(rects.shape[0], np.int64)
    _load().oracle_box_batch(_p(S), W, H, _p(rects), rects.shape[0], _p(out))
    return out


def template_stats(tpl):
    """(SumT, SumTSq, varT) of one [hT][wT] template."""
    tpl = np.ascontiguousarray(tpl, dtype=np.uint8)
    hT, wT = tpl.shape
    a, b, c = ctypes.c_int64(), ctypes.c_int64(), ctypes.c_int64()
    _load().oracle_template_stats(_p(tpl), wT, hT, ctypes.byref(a),
                                  ctypes.byref(b), ctypes.byref(c))
    return a.value, b.value, c.value


def coefficient(K, sumI, sumISq, sumIT, sumT, sumTSq) -> np.float32:
    return np.float32(_load().oracle_coefficient(int(K), int(sumI), int(sumISq),
                                                 int(sumIT), int(sumT), int(sumTSq)))


def correlate(img, tpl, want_sums: bool = True, nthreads: int = 0):
    """Valid-mode NCC of img with one template [hT][wT] or a bank [n][hT][wT].

    Returns (coef float32 [n][Ho][Wo], sums int32 [2+n][Ho][Wo] or None).
    """
    img = _u8_2d(img)
    tpl = _templates(tpl)
    H, W = img.shape
    n, hT, wT = tpl.shape
    if not (1 <= wT <= W and 1 <= hT <= H):
        raise ValueError("template larger than image")
    Ho, Wo = H - hT + 1, W - wT + 1
    coef = np.empty((n, Ho, Wo), np.float32)
    sums = np.empty((2 + n, Ho, Wo), np.int32) if want_sums else None
    rc = _load().oracle_correlate(_p(img), W, H, _p(tpl), wT, hT, n,
                                  _p(sums) if want_sums else None, _p(coef), nthreads)
    if rc != 0:
        raise RuntimeError("oracle_correlate failed (%d)" % rc)
    return coef, sums


def correlate_at(img, tpl, pos, S=None, Q=None, nthreads: int = 0):
    """The same values at positions pos [n][2] = {x, y} only.

    Returns (coef float32 [n][nTpl], sums int64 [n][2+nTpl]).  S, Q are the
    tables from sat_build (built here when not given).
    """
    img = _u8_2d(img)
    tpl = _templates(tpl)
    H, W = img.shape
    nT, hT, wT = tpl.shape
    if S is None or Q is None:
        S, Q = sat_build(img)
    S = np.ascontiguousarray(S, dtype=np.int64)
    Q = np.ascontiguousarray(Q, dtype=np.int64)
    pos = np.ascontiguousarray(pos, dtype=np.int32).reshape(-1, 2)
    n = pos.shape[0]
    coef = np.empty((n, nT), np.float32)
    sums = np.empty((n, 2 + nT), np.int64)
    rc = _load().oracle_correlate_at(_p(img), W, H, _p(S), _p(Q), _p(tpl), wT, hT, nT,
                                     _p(pos), n, _p(sums), _p(coef), nthreads)
    if rc != 0:
        raise ValueError("oracle_correlate_at: bad sizes or positions")
    return coef, sums


def correlate_rect(img, tpl, x0: int, y0: int, w: int, h: int, nthreads: int = 0):
    """Values at the positions x0..x0+w-1 by y0..y0+h-1 only: the sample
    program's rectangle of positions ("Image in shared memory", the offsets
    of corrShared_kernel), each window inside the image.

    Returns (coef float32 [nTpl][h][w], sums int64 [2+nTpl][h][w]), the
    per-position values of correlate_at laid out as the rectangle.
    """
    img = _u8_2d(img)
    tpl = _templates(tpl)
    H, W = img.shape
    nT, hT, wT = tpl.shape
    if w < 0 or h < 0 or x0 < 0 or y0 < 0 or x0 + w > W - wT + 1 or y0 + h > H - hT + 1:
        raise ValueError("rectangle outside the valid positions")
    ys, xs = np.meshgrid(np.arange(y0, y0 + h), np.arange(x0, x0 + w), indexing="ij")
    pos = np.stack([xs.ravel(), ys.ravel()], axis=1)
    if pos.shape[0] == 0:
        return np.zeros((nT, h, w), np.float32), np.zeros((2 + nT, h, w), np.int64)
    coef, sums = correlate_at(img, tpl, pos, nthreads=nthreads)
    return (np.ascontiguousarray(coef.T.reshape(nT, h, w)),
            np.ascontiguousarray(sums.T.reshape(2 + nT, h, w)))


def threads(nthreads: int = 0) -> int:
    """Threads the oracle's OpenMP regions use for a given request."""
    return int(_load().oracle_threads(nthreads))
