"""GPU parity of the vector-unit tile kernel (templates up to 32 bytes wide
and 64 rows high; window sums from the staged tile, no tables) against the
oracle and against the generic kernel (window sums from the int64 tables).

Sums bit for bit and coefficients within 1e-5 of the oracle.  Both kernels
form the same exact integers and the same float operations on them, so
their outputs must also agree bit for bit.
"""
import numpy as np
import pytest

from normalized_cross_correlation_amd import synth
from tests.gpu_util import COEF_ATOL, announce, dev, host, need_gpu, route

pytestmark = pytest.mark.gpu


def _check(oracle_mod, img, tpl, d, want_sums=True, name="tile"):
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
    with route("generic"):
        cg, sg = ncc.correlate(gi, gt, want_sums=want_sums)
    np.testing.assert_array_equal(coef, host(cg))
    if want_sums:
        np.testing.assert_array_equal(host(sums), host(sg))
    return coef, co


# H, W, hT, wT: one and several 64 x 64 tiles, ragged in both directions,
# every template width class (1 .. 8 dwords, partial last dword), the
# largest template (64 x 32)
@pytest.mark.parametrize("H,W,hT,wT,seed", [
    (40, 50, 1, 1, 81), (70, 90, 3, 3, 82), (100, 100, 32, 32, 83),
    (64, 200, 5, 31, 84), (120, 80, 40, 9, 85), (20, 20, 20, 20, 86),
    (9, 300, 2, 29, 87), (150, 257, 64, 32, 88), (65, 130, 17, 4, 89),
    (200, 67, 13, 30, 90), (130, 1030, 32, 32, 91), (66, 66, 64, 1, 92),
    (97, 141, 11, 22, 93), (80, 333, 8, 25, 94), (129, 65, 33, 17, 95),
])
@pytest.mark.parametrize("want_sums", [True, False])
def test_tile_shapes(oracle_mod, H, W, hT, wT, seed, want_sums):
    d = need_gpu()
    announce("tile %dx%d tpl %dx%d sums=%s" % (H, W, hT, wT, want_sums))
    c = synth.random_case(seed, H, W, hT, wT, nTpl=1, kind="smooth" if seed % 2 else "uniform")
    _check(oracle_mod, c["img"], c["tpl"], d, want_sums=want_sums)


def test_tile_medium_config(oracle_mod):
    """The 1024 x 1024 smooth-noise image with its 32 x 32 template cut with
    +-8 noise, on the tile kernel, in full."""
    d = need_gpu()
    announce("tile medium 1024x1024 32x32")
    w = synth.make("medium")
    _check(oracle_mod, w["img"], w["tpl"], d)


def test_tile_several_templates(oracle_mod):
    """Three templates one at a time: the window-sum planes written by the
    first launch, one SumIT plane per template."""
    d = need_gpu()
    announce("tile 3 templates 9x21")
    c = synth.random_case(96, 90, 200, 9, 21, nTpl=3, kind="smooth")
    _check(oracle_mod, c["img"], c["tpl"], d)


def test_tile_extremes(oracle_mod):
    """Bytes at both ends of the range with the largest template (K = 2048:
    SumISq = SumIT = 2048 * 255^2), constant windows and a constant
    template."""
    d = need_gpu()
    announce("tile extremes")
    rng = np.random.default_rng(97)
    img = np.full((200, 150), 255, np.uint8)
    img[:, 70:] = rng.choice(np.array([0, 255], np.uint8), size=(200, 80))
    tpls = np.stack([np.full((64, 32), 255, np.uint8),
                     rng.choice(np.array([0, 255], np.uint8), size=(64, 32)),
                     np.zeros((64, 32), np.uint8)])
    coef, _ = _check(oracle_mod, img, tpls, d)
    assert np.all(coef[2] == 0.0)           # constant template
    assert np.all(coef[:, :, :39] == 0.0)   # constant windows
    img2 = img.copy()
    img2[100:164, 90:122] = tpls[1]
    coef2, _ = _check(oracle_mod, img2, tpls[1], d)
    assert abs(coef2[0, 100, 90] - 1.0) <= COEF_ATOL


@pytest.mark.parametrize("layout", ["pitched_odd", "pitched4"])
def test_tile_rects(oracle_mod, layout):
    """Search rectangles read in place from a pitched image: at an odd
    address and pitch (byte staging) and at 4-byte aligned ones (dword
    staging), with output rows padded past the rectangle."""
    from tests.test_gpu_rect import _check as rect_check, _strided_image
    d = need_gpu()
    announce("tile rects %s" % layout)
    c = synth.random_case(98, 180, 300, 24, 19, nTpl=1, kind="smooth")
    iv = (_strided_image(c["img"], d, 3, 6) if layout == "pitched_odd"
          else _strided_image(c["img"], d, 4, 12))
    with route("tile"):
        for (x0, y0, w, h) in [(0, 0, 1, 1), (5, 7, 100, 60), (200, 100, 82, 57), (1, 2, 281, 155)]:
            rect_check(oracle_mod, c["img"], c["tpl"], d, x0, y0, w, h, out_pitch=w + 5, img_dev=iv)
