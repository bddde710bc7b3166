"""GPU parity of the single-template matrix-core kernel (SumIT of a template
16 rows high and 13 to 16 bytes wide as a banded Toeplitz product on the int8
matrix cores, SumI as the same product with an all-ones template) against the
oracle, and against the vector-unit streaming kernel.

Sums bit for bit and coefficients within 1e-5 of the oracle.  Both kernels
form the same exact integers and evaluate the coefficient with the same
float operations, so their outputs must also agree bit for bit.
"""
import numpy as np
import pytest

from normalized_cross_correlation_amd import synth
from tests.gpu_util import COEF_ATOL, announce, dev, host, need_gpu, route

pytestmark = pytest.mark.gpu


def _check(oracle_mod, img, tpl, d, want_sums=True):
    import normalized_cross_correlation_amd as ncc
    gi, gt = dev(img, d), dev(tpl, d)
    with route("single"):
        coef, sums = ncc.correlate(gi, gt, want_sums=want_sums)
    co, so = oracle_mod.correlate(img, tpl, want_sums=want_sums)
    coef = host(coef)
    if want_sums:
        np.testing.assert_array_equal(host(sums), so)
    err = np.abs(coef.astype(np.float64) - co.astype(np.float64))
    assert err.max() <= COEF_ATOL, "max |coef - oracle| = %g" % err.max()
    with route("dot4"):
        c4, s4 = ncc.correlate(gi, gt, want_sums=want_sums)
    np.testing.assert_array_equal(coef, host(c4))
    if want_sums:
        np.testing.assert_array_equal(host(sums), host(s4))
    return coef, co


# H, W, image kind, seed: workgroups take 1024 output columns x 16 or 32 rows
@pytest.mark.parametrize("H,W,kind,seed", [
    (16, 16, "uniform", 61),     # one output
    (47, 1040, "smooth", 62),    # two workgroups across (the second: 1 column)
    (100, 2064, "uniform", 63),  # three across, four row strips, ragged
    (80, 1039, "binary", 64),    # rows not 16-byte aligned: 1024 outputs per row
    (150, 257, "lowrange", 65),  # odd width
    (33, 4096, "smooth", 66),    # full headline width, two output rows
    (300, 70, "uniform", 67),    # tall and narrow
])
@pytest.mark.parametrize("want_sums", [True, False])
@pytest.mark.parametrize("strip", ["16", "32"])
def test_toeplitz_shapes(oracle_mod, ncc_opts, H, W, kind, seed, want_sums, strip):
    """Both strip heights (chosen per launch from the grid size; fixed here)."""
    d = need_gpu()
    ncc_opts(tz_strip=int(strip))
    announce("toeplitz %dx%d %s sums=%s strip=%s" % (H, W, kind, want_sums, strip))
    c = synth.random_case(seed, H, W, 16, 16, nTpl=1, kind=kind)
    _check(oracle_mod, c["img"], c["tpl"], d, want_sums=want_sums)


@pytest.mark.parametrize("wT", [13, 14, 15])
@pytest.mark.parametrize("H,W,kind,seed", [
    (60, 1104, "smooth", 71),    # two workgroups across, aligned rows
    (50, 1037, "uniform", 72),   # rows not 16-byte aligned
])
def test_toeplitz_narrow_templates(oracle_mod, wT, H, W, kind, seed):
    """16-row templates 13 to 15 bytes wide: the band and the all-ones
    operands end early and the row sums of I^2 mask the last dword."""
    d = need_gpu()
    announce("toeplitz wT=%d %dx%d %s" % (wT, H, W, kind))
    c = synth.random_case(seed + wT, H, W, 16, wT, nTpl=1, kind=kind)
    _check(oracle_mod, c["img"], c["tpl"], d)


def test_toeplitz_tall_and_wide(oracle_mod):
    """An image taller than 4096 rows and wider than 1024 columns: 132 strips
    of 32 rows, two workgroups across, a ragged last strip."""
    d = need_gpu()
    announce("toeplitz 4200x1100")
    c = synth.random_case(70, 4200, 1100, 16, 16, nTpl=1, kind="smooth")
    _check(oracle_mod, c["img"], c["tpl"], d)


def test_toeplitz_several_templates(oracle_mod):
    """Three templates one at a time (one launch each): the window-sum planes
    written once, one SumIT plane per template."""
    d = need_gpu()
    announce("toeplitz 3 templates")
    c = synth.random_case(68, 90, 1100, 16, 16, nTpl=3, kind="smooth")
    _check(oracle_mod, c["img"], c["tpl"], d)


def test_toeplitz_extremes(oracle_mod):
    """Values at the ends of the byte range: SumIT up to 256 * 255^2, the
    signed offsets of both operands at -128 and +127, zero-variance windows
    and a constant template."""
    d = need_gpu()
    announce("toeplitz extremes")
    rng = np.random.default_rng(69)
    img = np.full((64, 1100), 255, np.uint8)
    img[:, 500:] = rng.choice(np.array([0, 255], np.uint8), size=(64, 600))
    img[20:50, 700:760] = 0
    tpls = np.stack([np.full((16, 16), 255, np.uint8),
                     rng.choice(np.array([0, 255], np.uint8), size=(16, 16)),
                     np.zeros((16, 16), np.uint8)])
    coef, co = _check(oracle_mod, img, tpls, d)
    assert np.all(coef[2] == 0.0)          # constant template
    assert np.all(coef[:, :, :485] == 0.0)  # constant windows
    # the random 0/255 template cut from the image gives exactly 1 there
    img2 = img.copy()
    img2[5:21, 600:616] = tpls[1]
    coef2, _ = _check(oracle_mod, img2, tpls[1], d)
    assert abs(coef2[0, 5, 600] - 1.0) <= COEF_ATOL


def test_toeplitz_full_size_sampled(oracle_mod):
    """The 4096 x 4096 headline image with its cut template on the default
    route (the matrix-core kernel): 20 000 sampled positions, the cut and
    the corners against the oracle; the whole map against the streaming
    kernel bit for bit."""
    import normalized_cross_correlation_amd as ncc
    d = need_gpu()
    announce("toeplitz headline 4096x4096 sampled")
    w = synth.make("headline")
    img, tpl = w["img"], w["tpl"]
    gi, gt = dev(img, d), dev(tpl, d)
    coef, sums = ncc.correlate(gi, gt, want_sums=True)
    with route("dot4"):
        c4, s4 = ncc.correlate(gi, gt, want_sums=True)
    coef, sums = host(coef), host(sums)
    np.testing.assert_array_equal(coef, host(c4))
    np.testing.assert_array_equal(sums, host(s4))
    Ho, Wo = coef.shape[1:]
    rng = np.random.default_rng(97)
    (cx, cy), = w["cut_xy"]
    pos = np.concatenate([
        np.stack([rng.integers(0, Wo, 20000), rng.integers(0, Ho, 20000)], axis=1),
        [[cx, cy], [0, 0], [Wo - 1, 0], [0, Ho - 1], [Wo - 1, Ho - 1]],
    ]).astype(np.int32)
    pc, ps = oracle_mod.correlate_at(img, tpl, pos)
    xs, ys = pos[:, 0], pos[:, 1]
    np.testing.assert_array_equal(sums[:, ys, xs].T, ps)
    assert np.abs(coef[0, ys, xs] - pc[:, 0]).max() <= COEF_ATOL
    assert abs(coef[0, cy, cx] - 1.0) <= COEF_ATOL
