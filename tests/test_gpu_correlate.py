"""GPU parity of ncc_correlate against the oracle.

Integer window sums must match bit for bit; float32 coefficients within
1e-5 absolute.  Each route of the library (single-template kernels on the
matrix cores and on the vector units, generic kernel on the full tables, int8
matrix-core bank kernel) is checked.
"""
import numpy as np
import pytest

from normalized_cross_correlation_amd import synth
from tests.gpu_util import COEF_ATOL, announce, dev, host, need_gpu, route

pytestmark = pytest.mark.gpu


def _compare(oracle_mod, img, tpl, d, want_sums=True, route_name=None):
    import normalized_cross_correlation_amd as ncc
    with route(route_name):
        coef, sums = ncc.correlate(dev(img, d), dev(tpl, d), want_sums=want_sums)
    co, so = oracle_mod.correlate(img, tpl, want_sums=want_sums)
    coef = host(coef)
    if want_sums:
        np.testing.assert_array_equal(host(sums), so)
    err = np.abs(coef.astype(np.float64) - co.astype(np.float64))
    assert err.max() <= COEF_ATOL, "max |coef - oracle| = %g" % err.max()
    assert np.all(np.abs(coef) <= 1.0)
    return coef, co


def test_small_config_exact_one_at_cut(oracle_mod):
    """256 x 256 box-blurred noise, 16 x 16 template cut from it."""
    d = need_gpu()
    announce("correlate small 256x256 16x16")
    w = synth.make("small")
    coef, co = _compare(oracle_mod, w["img"], w["tpl"], d)
    (x, y), = w["cut_xy"]
    assert co[0, y, x] == 1.0
    assert abs(coef[0, y, x] - 1.0) <= COEF_ATOL
    assert np.unravel_index(np.argmax(coef[0]), coef[0].shape) == (y, x)


@pytest.mark.parametrize("rname", [None, "single", "dot4", "generic"])
@pytest.mark.parametrize("H,W,hT,wT,kind,seed", [
    (16, 16, 16, 16, "uniform", 1),     # one output
    (40, 300, 16, 16, "smooth", 2),     # ragged columns past one workgroup
    (300, 70, 16, 16, "uniform", 3),    # several row strips, ragged tail
    (161, 515, 16, 13, "binary", 4),    # template width not a multiple of 4
    (150, 257, 16, 15, "lowrange", 5),
    (97, 131, 16, 14, "uniform", 6),    # odd image width
])
def test_single_template_routes(oracle_mod, rname, H, W, hT, wT, kind, seed):
    d = need_gpu()
    announce("correlate route=%s %dx%d tpl %dx%d %s" % (rname, H, W, hT, wT, kind))
    c = synth.random_case(seed, H, W, hT, wT, nTpl=1, kind=kind)
    _compare(oracle_mod, c["img"], c["tpl"], d, route_name=rname)


@pytest.mark.parametrize("rs", ["16", "32", "64"])
@pytest.mark.parametrize("H,W,hT,wT,seed", [
    (16, 40, 16, 16, 51),     # one output row
    (47, 300, 16, 16, 52),    # 32 rows: one 32-row strip or two 16-row strips
    (143, 529, 16, 15, 53),   # ragged tail at every strip height
    (96, 256, 16, 16, 54),    # 81 rows
])
def test_stream_strip_heights(oracle_mod, ncc_opts, rs, H, W, hT, wT, seed):
    """The vector-unit streaming kernel at each strip height (chosen per
    launch from the output size; fixed here)."""
    d = need_gpu()
    ncc_opts(stream_rows=int(rs))
    announce("correlate stream rs=%s %dx%d tpl %dx%d" % (rs, H, W, hT, wT))
    c = synth.random_case(seed, H, W, hT, wT, nTpl=1, kind="smooth")
    _compare(oracle_mod, c["img"], c["tpl"], d, route_name="dot4")


@pytest.mark.parametrize("H,W,hT,wT,seed", [
    (50, 60, 1, 1, 11), (33, 47, 3, 3, 12), (70, 90, 17, 17, 13),
    (100, 100, 32, 32, 14), (64, 200, 5, 31, 15), (120, 80, 40, 9, 16),
    (20, 20, 20, 20, 17), (9, 300, 2, 100, 18),
])
def test_generic_shapes(oracle_mod, H, W, hT, wT, seed):
    d = need_gpu()
    announce("correlate generic %dx%d tpl %dx%d" % (H, W, hT, wT))
    c = synth.random_case(seed, H, W, hT, wT, nTpl=1, kind="uniform")
    _compare(oracle_mod, c["img"], c["tpl"], d, route_name="generic")


@pytest.mark.parametrize("H,W,hT,wT,seed", [
    (4200, 1100, 5, 7, 41),    # over 128 table bands and two column segments
    (8230, 2100, 16, 16, 42),
    (4300000, 2, 3, 1, 43),    # a one-dimensional signal: 67 188 output tiles down
])
def test_generic_tall_and_wide(oracle_mod, H, W, hT, wT, seed):
    """Window sums from tables of images taller than 4096 rows and wider than
    1024 columns (many tile rows and strips in the table build)."""
    d = need_gpu()
    announce("correlate generic tall %dx%d tpl %dx%d" % (H, W, hT, wT))
    c = synth.random_case(seed, H, W, hT, wT, nTpl=1, kind="uniform")
    _compare(oracle_mod, c["img"], c["tpl"], d, route_name="generic")


@pytest.mark.parametrize("H,W,hT,wT,seed", [
    (40, 3000, 2, 2500, 31),   # wide: blocks of template dwords
    (2300, 40, 2200, 3, 32),   # tall: blocks of template rows
    (230, 420, 150, 200, 33),  # K = 30000, both
    (2, 33100, 1, 33025, 34),  # K at its bound, one row
    (33100, 3, 33025, 1, 35),  # K at its bound, one column
])
def test_large_templates_in_blocks(oracle_mod, H, W, hT, wT, seed):
    """Templates whose tile + halo exceed the LDS: the blocked generic kernel."""
    d = need_gpu()
    announce("correlate large template %dx%d img %dx%d" % (hT, wT, H, W))
    c = synth.random_case(seed, H, W, hT, wT, nTpl=1, kind="uniform")
    _compare(oracle_mod, c["img"], c["tpl"], d)


def test_medium_config(oracle_mod):
    """1024 x 1024 smooth noise, 32 x 32 template cut with +-8 noise."""
    d = need_gpu()
    announce("correlate medium 1024x1024 32x32")
    w = synth.make("medium")
    _compare(oracle_mod, w["img"], w["tpl"], d)


@pytest.mark.parametrize("n,hT,wT,H,W,seed", [
    (2, 16, 16, 60, 90, 21), (16, 16, 16, 80, 100, 22), (63, 16, 16, 50, 150, 23),
    (64, 16, 16, 47, 130, 24), (65, 16, 16, 40, 81, 25), (7, 8, 8, 33, 70, 26),
    (20, 16, 5, 45, 66, 27), (5, 4, 32, 30, 99, 28), (3, 1, 1, 20, 30, 29),
    (130, 16, 16, 30, 40, 30),
    (3, 8, 8, 4200, 1100, 31),   # taller than 4096 rows, wider than 1024 columns
])
def test_bank(oracle_mod, n, hT, wT, H, W, seed):
    d = need_gpu()
    announce("correlate bank n=%d %dx%d img %dx%d" % (n, hT, wT, H, W))
    c = synth.random_case(seed, H, W, hT, wT, nTpl=n, kind="smooth" if seed % 2 else "uniform")
    _compare(oracle_mod, c["img"], c["tpl"], d)


# Both staging paths of the bank kernel: widths that are multiples of 16 take
# 16-byte loads from clamped addresses (tiles past the right and bottom edges
# read repeated image bytes), other widths the byte-aligned loads.  Templates
# up to 256 bytes wide (hT = 1) need two 16-byte loads per thread for the tile
# and halo; 17 templates end in a single 16-template block.
@pytest.mark.parametrize("n,hT,wT,H,W,seed", [
    (5, 16, 16, 48, 160, 51), (3, 1, 256, 20, 512, 52), (4, 2, 128, 40, 256, 53),
    (6, 8, 32, 70, 96, 54), (17, 16, 13, 35, 64, 55), (3, 1, 256, 20, 515, 56),
    (4, 2, 128, 40, 301, 57), (2, 16, 16, 16, 16, 58),
])
@pytest.mark.parametrize("want_sums", [True, False])
def test_bank_staging_paths(oracle_mod, n, hT, wT, H, W, seed, want_sums):
    d = need_gpu()
    announce("correlate bank staging n=%d %dx%d img %dx%d sums=%s" % (n, hT, wT, H, W, want_sums))
    c = synth.random_case(seed, H, W, hT, wT, nTpl=n, kind="smooth" if seed % 2 else "uniform")
    _compare(oracle_mod, c["img"], c["tpl"], d, want_sums=want_sums)


def test_bank_equals_single_route(oracle_mod):
    """The matrix-core bank and one-template-at-a-time give identical sums."""
    import normalized_cross_correlation_amd as ncc
    d = need_gpu()
    announce("bank vs single route")
    c = synth.random_case(41, 90, 140, 16, 16, nTpl=20, kind="smooth")
    img, tpl = dev(c["img"], d), dev(c["tpl"], d)
    cb, sb = ncc.correlate(img, tpl, want_sums=True)
    with route("single"):
        cs, ss = ncc.correlate(img, tpl, want_sums=True)
    np.testing.assert_array_equal(host(sb), host(ss))
    assert np.abs(host(cb) - host(cs)).max() <= 2 * COEF_ATOL


def test_zero_variance_windows_and_templates(oracle_mod):
    d = need_gpu()
    announce("zero variance")
    rng = np.random.default_rng(8)
    img = rng.integers(0, 256, (80, 90), dtype=np.uint8)
    img[10:40, 20:60] = 99  # flat patch: windows inside it have varI = 0
    tpl = rng.integers(0, 256, (3, 16, 16), dtype=np.uint8)
    tpl[1] = 7              # constant template: varT = 0
    for rname in (None, "single", "generic"):
        coef, co = _compare(oracle_mod, img, tpl, d, route_name=rname)
        assert np.all(coef[1] == 0.0)
        assert np.all(coef[0, 10:25, 20:45] == 0.0)
    const = np.full((40, 40), 200, np.uint8)
    coef, _ = _compare(oracle_mod, const, tpl[:1], d)
    assert np.all(coef == 0.0)


def test_full_size_headline_sampled(oracle_mod):
    """4096 x 4096 smooth noise, 16 x 16 template: tables compared in full,
    coefficients and sums at 20 000 seeded positions plus the cut and the
    image corners, in the launch configuration the benchmark times."""
    import normalized_cross_correlation_amd as ncc
    d = need_gpu()
    announce("headline 4096x4096 16x16 sampled")
    w = synth.make("headline")
    img, tpl = w["img"], w["tpl"]
    gimg = dev(img, d)
    S, Q = ncc.sat_build(gimg)
    So, Qo = oracle_mod.sat_build(img)
    np.testing.assert_array_equal(host(S), So)
    np.testing.assert_array_equal(host(Q), Qo)
    coef, sums = ncc.correlate(gimg, dev(tpl, d), want_sums=True)
    coef, sums = host(coef), host(sums)
    Ho, Wo = coef.shape[1:]
    rng = np.random.default_rng(99)
    (cx, cy), = w["cut_xy"]
    pos = np.concatenate([
        np.stack([rng.integers(0, Wo, 20000), rng.integers(0, Ho, 20000)], axis=1),
        [[cx, cy], [0, 0], [Wo - 1, 0], [0, Ho - 1], [Wo - 1, Ho - 1]],
    ]).astype(np.int32)
    pc, ps = oracle_mod.correlate_at(img, tpl, pos, So, Qo)
    xs, ys = pos[:, 0], pos[:, 1]
    np.testing.assert_array_equal(sums[:, ys, xs].T, ps)
    assert np.abs(coef[0, ys, xs] - pc[:, 0]).max() <= COEF_ATOL
    assert abs(coef[0, cy, cx] - 1.0) <= COEF_ATOL
    # properties over the whole map
    assert np.all(np.abs(coef) <= 1.0) and np.isfinite(coef).all()
    # window sums agree with box queries on the full tables (another route)
    rects = np.stack([xs, ys, xs + 16, ys + 16], axis=1).astype(np.int32)
    bs = host(ncc.box(S, dev(rects, d)))
    bq = host(ncc.box(Q, dev(rects, d)))
    np.testing.assert_array_equal(sums[0, ys, xs], bs)
    np.testing.assert_array_equal(sums[1, ys, xs], bq)


def test_full_size_bank_sampled(oracle_mod):
    """4096 x 4096 smooth noise with 64 templates (32 cut, 32 random):
    every map at 4 000 seeded positions and at each cut."""
    import normalized_cross_correlation_amd as ncc
    d = need_gpu()
    announce("bank 4096x4096 x64 sampled")
    w = synth.make("bank")
    img, tpl = w["img"], w["tpl"]
    coef, sums = ncc.correlate(dev(img, d), dev(tpl, d), want_sums=True)
    Ho, Wo = coef.shape[1:]
    rng = np.random.default_rng(98)
    pos = np.stack([rng.integers(0, Wo, 4000), rng.integers(0, Ho, 4000)], axis=1)
    pos = np.concatenate([pos, np.array(w["cut_xy"])]).astype(np.int32)
    xs = __import__("torch").from_numpy(pos[:, 0].astype(np.int64)).to(d)
    ys = __import__("torch").from_numpy(pos[:, 1].astype(np.int64)).to(d)
    gc = host(coef[:, ys, xs]).T  # [n][64]
    gs = host(sums[:, ys, xs]).T
    pc, ps = oracle_mod.correlate_at(img, tpl, pos)
    np.testing.assert_array_equal(gs, ps)
    assert np.abs(gc - pc).max() <= COEF_ATOL
    for t, (x, y) in enumerate(w["cut_xy"]):
        assert abs(float(coef[t, y, x]) - 1.0) <= COEF_ATOL


def test_correlate_deterministic():
    import torch
    import normalized_cross_correlation_amd as ncc
    d = need_gpu()
    announce("correlate determinism")
    c = synth.random_case(77, 300, 600, 16, 16, nTpl=3, kind="smooth")
    img, tpl = dev(c["img"], d), dev(c["tpl"], d)
    a1, s1 = ncc.correlate(img, tpl, want_sums=True)
    a2, s2 = ncc.correlate(img, tpl, want_sums=True)
    assert torch.equal(a1, a2) and torch.equal(s1, s2)


def test_errors_from_host():
    import torch
    import normalized_cross_correlation_amd as ncc
    d = need_gpu()
    L = ncc.lib()
    img = torch.zeros((10, 10), dtype=torch.uint8, device=d)
    out = torch.zeros((1, 1, 1), dtype=torch.float32, device=d)
    assert L.ncc_correlate(img.data_ptr(), 10, 10, img.data_ptr(), 11, 1, 1, None,
                           out.data_ptr(), None, None, None) == -1
    assert L.ncc_correlate(img.data_ptr(), 70000, 1, img.data_ptr(), 1, 1, 1, None,
                           out.data_ptr(), None, None, None) == -2
    assert L.ncc_correlate(img.data_ptr(), 200, 200, img.data_ptr(), 182, 182, 1, None,
                           out.data_ptr(), None, None, None) == -2
    with pytest.raises(ValueError):
        ncc.correlate(img, torch.zeros((11, 2), dtype=torch.uint8, device=d))
