"""GPU parity of the FFT numerator route (large templates: SumIT as the
inverse transform of DFT(I) . conj(DFT(T)) in double precision, rounded to
the integer it equals; SumI and SumISq from the view's summed-area tables)
against the oracle.  Sums bit for bit, coefficients within 1e-5 absolute.
The route is forced with NCC_CORR_PATH=fft on small shapes (every parity of
the transform lengths' exponents) and chosen by the library itself for large
templates at the full 4096 x 4096 size."""
import numpy as np
import pytest

from normalized_cross_correlation_amd import synth
from tests.gpu_util import COEF_ATOL, announce, dev, host, need_gpu, route

pytestmark = pytest.mark.gpu


def _compare(oracle_mod, img, tpl, d, route_name="fft"):
    import normalized_cross_correlation_amd as ncc
    with route(route_name):
        coef, sums = ncc.correlate(dev(img, d), dev(tpl, d), want_sums=True)
    co, so = oracle_mod.correlate(img, tpl)
    np.testing.assert_array_equal(host(sums), so)
    err = np.abs(host(coef).astype(np.float64) - co.astype(np.float64))
    assert err.max() <= COEF_ATOL, "max |coef - oracle| = %g" % err.max()


@pytest.mark.parametrize("H,W,hT,wT,n,seed", [
    (40, 60, 9, 11, 1, 1),      # transform 64 x 64: M = 32 (odd exponent), P = 8 x 8
    (33, 47, 3, 3, 2, 2),       # two templates share the image's spectrum
    (100, 100, 32, 32, 1, 3),
    (64, 200, 5, 31, 1, 4),     # P = 64 (8 x 8), M = 128 (odd exponent)
    (120, 80, 40, 9, 1, 5),
    (20, 20, 20, 20, 1, 6),     # one output
    (9, 300, 2, 100, 1, 7),
    (5, 9, 1, 1, 3, 8),         # smallest transforms: 8 x 16
    (130, 70, 16, 16, 1, 9),    # a shape the streaming kernel would take
    (300, 257, 17, 45, 1, 10),  # P = 512 (32 x 16), Qn = 512 (M = 256)
])
def test_fft_route_shapes(oracle_mod, H, W, hT, wT, n, seed):
    d = need_gpu()
    announce("fft route %dx%d tpl %dx%d n=%d" % (H, W, hT, wT, n))
    c = synth.random_case(seed, H, W, hT, wT, nTpl=n, kind="uniform" if seed % 2 else "smooth")
    _compare(oracle_mod, c["img"], c["tpl"], d)


@pytest.mark.parametrize("sat_path", ["two_pass", "single_pass"])
def test_fft_route_both_table_builds(oracle_mod, ncc_opts, sat_path):
    d = need_gpu()
    ncc_opts(sat_build=sat_path)
    announce("fft route sat=%s" % sat_path)
    c = synth.random_case(21, 150, 170, 21, 13, nTpl=1, kind="smooth")
    _compare(oracle_mod, c["img"], c["tpl"], d)


def test_fft_route_zero_variance(oracle_mod):
    d = need_gpu()
    announce("fft route zero variance")
    rng = np.random.default_rng(8)
    img = rng.integers(0, 256, (80, 90), dtype=np.uint8)
    img[10:50, 20:70] = 99
    tpl = rng.integers(0, 256, (2, 20, 17), dtype=np.uint8)
    tpl[1] = 7
    _compare(oracle_mod, img, tpl, d)


def test_fft_route_widest_transform(oracle_mod):
    """Rows of 8192 (the longest row transform, 4096 complex in LDS) and a
    template of 16 000 pixels, all 255 against all-255 rows: the largest
    SumIT this route rounds (16 000 * 255^2 = 1 040 400 000)."""
    d = need_gpu()
    announce("fft route 3x8192, template 2x8000")
    rng = np.random.default_rng(9)
    img = rng.integers(0, 256, (3, 8192), dtype=np.uint8)
    img[:, :4000] = 255
    tpl = np.full((2, 8000), 255, np.uint8)
    tpl[1, ::7] = 3
    _compare(oracle_mod, img, tpl, d)


def test_fft_route_falls_back_beyond_its_sizes(oracle_mod):
    """A view wider than 8192 is outside the FFT route: the direct route."""
    d = need_gpu()
    announce("fft route fallback 2x9000")
    c = synth.random_case(30, 2, 9000, 2, 33, nTpl=1, kind="uniform")
    _compare(oracle_mod, c["img"], c["tpl"], d)


def test_fft_route_search_rectangle(oracle_mod):
    """A search rectangle of a pitched image through the FFT route."""
    import torch
    import normalized_cross_correlation_amd as ncc
    d = need_gpu()
    announce("fft route rectangle")
    c = synth.random_case(31, 200, 230, 25, 19, nTpl=2, kind="smooth")
    big = np.full((205, 256), 9, np.uint8)
    big[3:203, 11:241] = c["img"]
    v = torch.from_numpy(big).to(d)[3:203, 11:241]
    x0, y0, w, h = 17, 40, 150, 99
    with route("fft"):
        coef, sums = ncc.correlate_rect(v, dev(c["tpl"], d), x0, y0, w, h, want_sums=True,
                                        out_pitch=160)
    co, so = oracle_mod.correlate_rect(c["img"], c["tpl"], x0, y0, w, h)
    np.testing.assert_array_equal(host(sums).astype(np.int64), so)
    assert np.abs(host(coef).astype(np.float64) - co).max() <= COEF_ATOL


@pytest.mark.parametrize("t", [64, 128])
def test_fft_route_full_size_sampled(oracle_mod, t):
    """4096 x 4096 smooth noise with a t x t template cut from it: the
    library picks the FFT route by itself; sampled positions against the
    oracle, the cut found with gamma = 1."""
    import normalized_cross_correlation_amd as ncc
    d = need_gpu()
    announce("fft route 4096^2 tpl %dx%d (auto)" % (t, t))
    w = synth.make("headline")
    img = w["img"]
    rng = np.random.default_rng(40 + t)
    cx, cy = int(rng.integers(0, 4096 - t)), int(rng.integers(0, 4096 - t))
    tpl = np.ascontiguousarray(img[cy:cy + t, cx:cx + t])[None]
    with route(None):
        coef, sums = ncc.correlate(dev(img, d), dev(tpl, d), want_sums=True)
    coef, sums = host(coef), host(sums)
    Ho, Wo = coef.shape[1:]
    pos = np.concatenate([np.stack([rng.integers(0, Wo, 300), rng.integers(0, Ho, 300)], axis=1),
                          [[cx, cy], [0, 0], [Wo - 1, Ho - 1]]]).astype(np.int32)
    pc, ps = oracle_mod.correlate_at(img, tpl, pos)
    xs, ys = pos[:, 0], pos[:, 1]
    np.testing.assert_array_equal(sums[:, ys, xs].T, ps)
    assert np.abs(coef[0, ys, xs] - pc[:, 0]).max() <= COEF_ATOL
    assert abs(coef[0, cy, cx] - 1.0) <= COEF_ATOL
