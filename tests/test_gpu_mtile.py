"""GPU parity of the matrix-core tile kernel (single templates up to 32 x 32:
SumIT as one banded int8 product per template row, window sums from the
tile's running column sums) against the oracle and against the vector-unit
tile kernel.

Sums bit for bit and coefficients within 1e-5 of the oracle.  Both kernels
form the same exact integers and the same float operations on them, so
their outputs must also agree bit for bit.
"""
import numpy as np
import pytest

from normalized_cross_correlation_amd import synth
from tests.gpu_util import COEF_ATOL, announce, dev, host, need_gpu, route

pytestmark = pytest.mark.gpu


def _check(oracle_mod, img, tpl, d, want_sums=True, name="single"):
    import normalized_cross_correlation_amd as ncc
    gi, gt = dev(img, d), dev(tpl, d)
    with route(name):
        coef, sums = ncc.correlate(gi, gt, want_sums=want_sums)
    co, so = oracle_mod.correlate(img, tpl, want_sums=want_sums)
    coef = host(coef)
    if want_sums:
        np.testing.assert_array_equal(host(sums), so)
    err = np.abs(coef.astype(np.float64) - co.astype(np.float64))
    assert err.max() <= COEF_ATOL, "max |coef - oracle| = %g" % err.max()
    with route("tile"):
        ct, st = ncc.correlate(gi, gt, want_sums=want_sums)
    np.testing.assert_array_equal(coef, host(ct))
    if want_sums:
        np.testing.assert_array_equal(host(sums), host(st))
    return coef, co


# H, W, hT, wT: one and several 64 x 32 workgroup tiles, ragged in both
# directions, rows not 16-byte aligned, every template width class, the
# largest template (32 x 32), one-pixel templates and templates as tall as
# the image (one output row)
@pytest.mark.parametrize("H,W,hT,wT,seed", [
    (40, 50, 1, 1, 101), (70, 90, 3, 3, 102), (100, 100, 32, 32, 103),
    (64, 200, 5, 31, 104), (20, 20, 20, 20, 105), (9, 300, 2, 29, 106),
    (65, 130, 17, 4, 107), (200, 67, 13, 30, 108), (130, 1030, 32, 32, 109),
    (97, 141, 11, 22, 110), (80, 333, 8, 25, 111), (33, 65, 32, 17, 112),
    (64, 129, 31, 32, 113), (47, 1040, 24, 20, 114), (48, 64, 16, 12, 115),
    (150, 257, 32, 1, 116), (32, 96, 32, 32, 117),
])
@pytest.mark.parametrize("want_sums", [True, False])
def test_mtile_shapes(oracle_mod, H, W, hT, wT, seed, want_sums):
    d = need_gpu()
    announce("mtile %dx%d tpl %dx%d sums=%s" % (H, W, hT, wT, want_sums))
    c = synth.random_case(seed, H, W, hT, wT, nTpl=1, kind="smooth" if seed % 2 else "uniform")
    _check(oracle_mod, c["img"], c["tpl"], d, want_sums=want_sums)


def test_mtile_several_templates(oracle_mod):
    """Three 20 x 27 templates one at a time (one launch each)."""
    d = need_gpu()
    announce("mtile 3 templates")
    c = synth.random_case(118, 90, 200, 20, 27, nTpl=3, kind="smooth")
    _check(oracle_mod, c["img"], c["tpl"], d)


def test_mtile_extremes(oracle_mod):
    """Bytes at both ends of the range: SumIT up to 1024 * 255^2, the
    numerator past 2^31 (formed exactly in double), zero-variance windows,
    a constant template, and a template cut from the image (coefficient 1)."""
    d = need_gpu()
    announce("mtile extremes")
    rng = np.random.default_rng(119)
    img = np.full((96, 160), 255, np.uint8)
    img[:, 70:] = rng.choice(np.array([0, 255], np.uint8), size=(96, 90))
    img[40:80, 100:140] = 0
    tpls = np.stack([np.full((32, 32), 255, np.uint8),
                     rng.choice(np.array([0, 255], np.uint8), size=(32, 32)),
                     np.zeros((32, 32), np.uint8)])
    coef, co = _check(oracle_mod, img, tpls, d)
    assert np.all(coef[2] == 0.0)           # constant template
    assert np.all(coef[:, :, :39] == 0.0)   # constant windows
    img2 = img.copy()
    img2[10:42, 90:122] = tpls[1]
    coef2, _ = _check(oracle_mod, img2, tpls[1], d)
    assert abs(coef2[0, 10, 90] - 1.0) <= COEF_ATOL


def test_mtile_medium_config(oracle_mod):
    """The 1024 x 1024 smooth-noise image with its 32 x 32 template cut with
    +-8 noise, on the default route (which takes this kernel), in full; the
    maximum found is the oracle's (up to the coefficient tolerance)."""
    d = need_gpu()
    announce("mtile medium 1024x1024 32x32")
    w = synth.make("medium")
    coef, co = _check(oracle_mod, w["img"], w["tpl"], d, name=None)
    i = int(np.argmax(coef[0]))
    assert co[0].flat[i] >= co[0].max() - 2 * COEF_ATOL


@pytest.mark.parametrize("layout", ["pitched_odd", "pitched16"])
def test_mtile_rects(oracle_mod, layout):
    """Search rectangles read in place from a pitched image: at an odd
    address and pitch (byte-aligned staging) and at 16-byte aligned ones,
    with output rows padded past the rectangle."""
    from tests.test_gpu_rect import _check as rect_check, _strided_image
    d = need_gpu()
    announce("mtile rects %s" % layout)
    c = synth.random_case(120, 180, 300, 24, 19, nTpl=1, kind="smooth")
    iv = (_strided_image(c["img"], d, 3, 6) if layout == "pitched_odd"
          else _strided_image(c["img"], d, 16, 20))
    with route("single"):
        for (x0, y0, w, h) in [(0, 0, 1, 1), (5, 7, 100, 60), (200, 100, 82, 57), (1, 2, 281, 155)]:
            rect_check(oracle_mod, c["img"], c["tpl"], d, x0, y0, w, h, out_pitch=w + 5, img_dev=iv)
