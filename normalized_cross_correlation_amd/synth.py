"""Seeded synthetic inputs for NCC template matching (numpy only).

This module makes input bytes; it holds none of the correlation or table
arithmetic, and both the GPU path's tests and the CPU oracle read what it
makes.  Every generator is deterministic for a given seed (numpy PCG64).

Workload shapes (the handbook pages time their table builds on 4096 x 4096
8-bit images and print no pixel statistics, so the values are synthetic):

* ``small``    256 x 256, uniform noise box-blurred 5 x 5; one 16 x 16
               template cut from the image at a seeded offset.
* ``sat``      4096 x 4096 uniform [0, 255]; 1 000 000 seeded box queries.
* ``medium``   1024 x 1024 smooth noise (Gaussian, sigma 40 around 128,
               9 x 9 box blur); one 32 x 32 template cut from it with
               uniform integer noise in [-8, 8] added.
* ``headline`` 4096 x 4096 smooth noise; one 16 x 16 template cut from it.
* ``bank``     4096 x 4096 smooth noise; 64 templates of 16 x 16, the first
               32 cut from the image at distinct seeded offsets, the last 32
               uniform [0, 255].

Blur: a k x k box mean with edge-replicating borders (scipy.ndimage
uniform_filter, mode "nearest"), rounded half-to-even and clipped to [0, 255].
"""
from __future__ import annotations

import numpy as np
from scipy.ndimage import uniform_filter

SEED_BASE = 1000
CONFIG_INDEX = {"small": 0, "sat": 1, "medium": 2, "headline": 3, "bank": 4}


def _rng(name: str, seed: int | None = None) -> np.random.Generator:
    if seed is None:
        seed = SEED_BASE + CONFIG_INDEX[name]
    return np.random.Generator(np.random.PCG64(seed))


def box_blur_u8(img: np.ndarray, k: int) -> np.ndarray:
    f = uniform_filter(np.asarray(img, np.float64), size=k, mode="nearest")
    return np.clip(np.rint(f), 0, 255).astype(np.uint8)


def uniform_u8(rng: np.random.Generator, H: int, W: int) -> np.ndarray:
    return rng.integers(0, 256, size=(H, W), dtype=np.uint8)


def smooth_noise_u8(rng: np.random.Generator, H: int, W: int, sigma: float = 40.0,
                    k: int = 9) -> np.ndarray:
    g = rng.normal(128.0, sigma, size=(H, W))
    f = uniform_filter(g, size=k, mode="nearest")
    return np.clip(np.rint(f), 0, 255).astype(np.uint8)


def cut(img: np.ndarray, x: int, y: int, wT: int, hT: int) -> np.ndarray:
    return np.ascontiguousarray(img[y:y + hT, x:x + wT])


def _nonconstant_cut(rng, img, wT, hT, avoid=()):
    H, W = img.shape
    for _ in range(10000):
        x = int(rng.integers(0, W - wT + 1))
        y = int(rng.integers(0, H - hT + 1))
        if (x, y) in avoid:
            continue
        t = cut(img, x, y, wT, hT)
        if t.min() != t.max():
            return t, (x, y)
    raise RuntimeError("no textured window found")


def random_rects(rng: np.random.Generator, W: int, H: int, n: int) -> np.ndarray:
    """n non-empty rectangles {x0, y0, x1, y1} (int32) inside a W x H table:
    x0 = min(a, b), x1 = max(a, b) + 1 with a, b uniform over the columns,
    and the same for rows."""
    a = rng.integers(0, W, size=n)
    b = rng.integers(0, W, size=n)
    c = rng.integers(0, H, size=n)
    d = rng.integers(0, H, size=n)
    r = np.stack([np.minimum(a, b), np.minimum(c, d),
                  np.maximum(a, b) + 1, np.maximum(c, d) + 1], axis=1)
    return np.ascontiguousarray(r.astype(np.int32))


def make(name: str, seed: int | None = None) -> dict:
    """Inputs of one named workload.

    Returns a dict with ``img`` (uint8 [H][W]) and, depending on the workload,
    ``tpl`` (uint8 [n][hT][wT]), ``cut_xy`` (offsets the cut templates came
    from, one per cut template) and ``rects`` (int32 [n][4]).
    """
    rng = _rng(name, seed)
    if name == "small":
        img = box_blur_u8(uniform_u8(rng, 256, 256), 5)
        t, xy = _nonconstant_cut(rng, img, 16, 16)
        return {"img": img, "tpl": t[None], "cut_xy": [xy]}
    if name == "sat":
        img = uniform_u8(rng, 4096, 4096)
        rects = random_rects(rng, 4096, 4096, 1_000_000)
        return {"img": img, "rects": rects}
    if name == "medium":
        img = smooth_noise_u8(rng, 1024, 1024)
        t, xy = _nonconstant_cut(rng, img, 32, 32)
        noise = rng.integers(-8, 9, size=t.shape)
        t = np.clip(t.astype(np.int64) + noise, 0, 255).astype(np.uint8)
        return {"img": img, "tpl": t[None], "cut_xy": [xy]}
    if name == "headline":
        img = smooth_noise_u8(rng, 4096, 4096)
        t, xy = _nonconstant_cut(rng, img, 16, 16)
        return {"img": img, "tpl": t[None], "cut_xy": [xy]}
    if name == "bank":
        img = smooth_noise_u8(rng, 4096, 4096)
        tpls, xys = [], []
        for _ in range(32):
            t, xy = _nonconstant_cut(rng, img, 16, 16, avoid=set(xys))
            tpls.append(t)
            xys.append(xy)
        for _ in range(32):
            tpls.append(rng.integers(0, 256, size=(16, 16), dtype=np.uint8))
        return {"img": img, "tpl": np.ascontiguousarray(np.stack(tpls)), "cut_xy": xys}
    raise KeyError(name)


def random_case(seed: int, H: int, W: int, hT: int, wT: int, nTpl: int = 1,
                kind: str = "uniform") -> dict:
    """A small seeded case for parity sweeps: image kind is one of
    'uniform', 'smooth', 'binary', 'constant', 'lowrange'."""
    rng = np.random.Generator(np.random.PCG64(seed))
    if kind == "uniform":
        img = uniform_u8(rng, H, W)
    elif kind == "smooth":
        img = smooth_noise_u8(rng, H, W)
    elif kind == "binary":
        img = (rng.integers(0, 2, size=(H, W)) * 255).astype(np.uint8)
    elif kind == "constant":
        img = np.full((H, W), int(rng.integers(0, 256)), np.uint8)
    elif kind == "lowrange":
        img = rng.integers(0, 64, size=(H, W), dtype=np.uint8)
    else:
        raise KeyError(kind)
    tpl = rng.integers(0, 256, size=(nTpl, hT, wT), dtype=np.uint8)
    # half of the templates (at least one) are cut from the image
    for t in range(0, nTpl, 2):
        x = int(rng.integers(0, W - wT + 1))
        y = int(rng.integers(0, H - hT + 1))
        tpl[t] = img[y:y + hT, x:x + wT]
    return {"img": img, "tpl": np.ascontiguousarray(tpl)}
