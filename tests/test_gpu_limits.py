"""GPU parity at the integer bounds of the method (section 15.8 width
analysis): the widest image the uint32 row partials allow, W = 66 051, filled
with values 250..255 so that the row running sums of I^2 end within 3% of
2^32, through the table builds and every correlation route;
and the largest template the int32 window sums allow, K = 33 025, against
all-255 pixels.  Tables and sums bit for bit, coefficients within 1e-5."""
import numpy as np
import pytest

from tests.gpu_util import COEF_ATOL, announce, dev, host, need_gpu, route

pytestmark = pytest.mark.gpu

MAX_W = 66051


def _near_white(seed, H, W):
    rng = np.random.default_rng(seed)
    img = rng.integers(250, 256, (H, W), dtype=np.uint8)
    img[:, -200:] = 255  # the row ends at the full 255^2 per pixel
    return img


@pytest.mark.parametrize("sat_path", ["two_pass", "single_pass"])
def test_sat_at_max_width(oracle_mod, ncc_opts, sat_path):
    import normalized_cross_correlation_amd as ncc
    d = need_gpu()
    ncc_opts(sat_build=sat_path)
    announce("sat at max width 37x%d sat=%s" % (MAX_W, sat_path))
    img = _near_white(1, 37, MAX_W)
    S, Q = ncc.sat_build(dev(img, d))
    So, Qo = oracle_mod.sat_build(img)
    np.testing.assert_array_equal(host(S), So)
    np.testing.assert_array_equal(host(Q), Qo)
    # the row partial of I^2 at the end of each row: below 2^32, within 3%
    last = np.diff(np.concatenate([[0], Qo[:, -1]]))
    assert last.max() < 2 ** 32 and last.max() > 0.97 * 2 ** 32


@pytest.mark.parametrize("rname,n,hT,wT", [
    ("single", 1, 16, 16),    # single template on the matrix cores
    ("dot4", 1, 16, 16),      # single template on the vector units
    ("generic", 1, 9, 11),    # the full tables
    (None, 3, 16, 16),        # matrix-core bank
])
def test_correlate_at_max_width(oracle_mod, rname, n, hT, wT):
    import normalized_cross_correlation_amd as ncc
    d = need_gpu()
    announce("correlate at max width route=%s n=%d %dx%d" % (rname, n, hT, wT))
    img = _near_white(2, 20, MAX_W)
    rng = np.random.default_rng(3)
    tpl = rng.integers(0, 256, (n, hT, wT), dtype=np.uint8)
    tpl[0] = img[2:2 + hT, 1000:1000 + wT]  # an exact match at (1000, 2)
    with route(rname):
        coef, sums = ncc.correlate(dev(img, d), dev(tpl, d), want_sums=True)
    co, so = oracle_mod.correlate(img, tpl)
    np.testing.assert_array_equal(host(sums), so)
    assert np.abs(host(coef).astype(np.float64) - co).max() <= COEF_ATOL
    assert abs(float(host(coef)[0, 2, 1000]) - 1.0) <= COEF_ATOL


def test_largest_template_all_255(oracle_mod):
    """K = 33 025 (a 5 x 6 605 template) of 255s over 255s: SumISq = SumIT =
    33 025 * 65 025 = 2 147 450 625, just below 2^31; zero variance
    everywhere, so every coefficient is 0."""
    import normalized_cross_correlation_amd as ncc
    d = need_gpu()
    announce("largest template all 255")
    img = np.full((7, 6700), 255, np.uint8)
    tpl = np.full((5, 6605), 255, np.uint8)
    coef, sums = ncc.correlate(dev(img, d), dev(tpl, d), want_sums=True)
    co, so = oracle_mod.correlate(img, tpl)
    np.testing.assert_array_equal(host(sums), so)
    assert int(so[1].max()) == 33025 * 65025 and int(so[2].max()) == 33025 * 65025
    assert np.all(host(coef) == 0.0) and np.all(co == 0.0)
