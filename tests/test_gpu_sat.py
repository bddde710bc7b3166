"""GPU parity of the summed-area table build and box queries against the oracle.

Tables and box sums are integers: they must match bit for bit.  Every test
runs on both builds of the library: the three-pass build (default) and the
single-pass look-back build (option sat_build = single_pass).
"""
import numpy as np
import pytest

from normalized_cross_correlation_amd import synth
from tests.gpu_util import announce, dev, host, need_gpu

pytestmark = pytest.mark.gpu


@pytest.fixture(autouse=True, params=["two_pass", "single_pass"])
def sat_route(request):
    import normalized_cross_correlation_amd as ncc
    with ncc.options(sat_build=request.param):
        yield request.param

SHAPES = [
    # H, W: single pixel, thin, below one tile, ragged tails in both directions,
    # widths that are not multiples of 4, several tiles
    (1, 1), (1, 300), (300, 1), (7, 5), (63, 255), (64, 256), (65, 257),
    (130, 515), (200, 1023), (129, 1030), (333, 777),
    # more than 32 tile rows, in counts that are not multiples of the 8 XCDs
    # the tile rows are spread over (33, 65, 36), and tile prologues summing
    # the column sums of many tiles above
    (4200, 1100), (8230, 1030), (4500, 2100),
    # tile rows that divide evenly over the 8 XCDs (interleaved placement)
    # with ragged tails: 8 tile rows with a partial last 4-row group and a
    # width not a multiple of 4, 16 tile rows, and 33 strips with rows wider
    # than one 4096-column chunk of a row workgroup
    (1021, 301), (2047, 129), (1024, 4100),
    # more tile rows (17 188) and row groups than one grid dimension of 65 536
    (2200000, 3),
]


@pytest.mark.parametrize("H,W", SHAPES)
def test_sat_matches_oracle(oracle_mod, H, W, sat_route):
    import normalized_cross_correlation_amd as ncc
    d = need_gpu()
    announce("sat %dx%d build=%s" % (H, W, sat_route))
    rng = np.random.default_rng(H * 10007 + W)
    img = rng.integers(0, 256, (H, W), dtype=np.uint8)
    S, Q = ncc.sat_build(dev(img, d))
    So, Qo = oracle_mod.sat_build(img)
    np.testing.assert_array_equal(host(S), So)
    np.testing.assert_array_equal(host(Q), Qo)


def test_sat_all_255_width_limits(oracle_mod):
    """All-255 4096 x 4096: the largest values the int64 tables and uint32 row
    partials take at the benchmark size."""
    import torch
    import normalized_cross_correlation_amd as ncc
    d = need_gpu()
    announce("sat all-255 4096x4096")
    img = torch.full((4096, 4096), 255, dtype=torch.uint8, device=d)
    S, Q = ncc.sat_build(img)
    ys = torch.arange(1, 4097, device=d, dtype=torch.int64)
    expect_S = 255 * ys[:, None] * ys[None, :]
    assert torch.equal(S, expect_S)
    assert torch.equal(Q, 255 * expect_S)
    assert int(Q[-1, -1]) == 4096 * 4096 * 65025


def test_sat_full_size_uniform(oracle_mod):
    """The table-build workload: 4096 x 4096 uniform bytes, compared in full,
    and 1 000 000 seeded box queries on both tables."""
    import normalized_cross_correlation_amd as ncc
    d = need_gpu()
    announce("sat 4096x4096 uniform + 1M boxes")
    w = synth.make("sat")
    img, rects = w["img"], w["rects"]
    S, Q = ncc.sat_build(dev(img, d))
    So, Qo = oracle_mod.sat_build(img)
    np.testing.assert_array_equal(host(S), So)
    np.testing.assert_array_equal(host(Q), Qo)
    r = dev(rects, d)
    bs = host(ncc.box(S, r))
    bq = host(ncc.box(Q, r))
    np.testing.assert_array_equal(bs, oracle_mod.box_batch(So, rects))
    np.testing.assert_array_equal(bq, oracle_mod.box_batch(Qo, rects))


def test_sat_deterministic():
    import torch
    import normalized_cross_correlation_amd as ncc
    d = need_gpu()
    announce("sat determinism")
    g = torch.Generator(device="cpu").manual_seed(5)
    img = torch.randint(0, 256, (1000, 1500), generator=g, dtype=torch.uint8).to(d)
    S1, Q1 = ncc.sat_build(img)
    S2, Q2 = ncc.sat_build(img)
    assert torch.equal(S1, S2) and torch.equal(Q1, Q2)


def test_box_edges(oracle_mod):
    import normalized_cross_correlation_amd as ncc
    d = need_gpu()
    announce("box edge cases")
    rng = np.random.default_rng(3)
    H, W = 37, 53
    img = rng.integers(0, 256, (H, W), dtype=np.uint8)
    S, _ = ncc.sat_build(dev(img, d))
    So, _ = oracle_mod.sat_build(img)
    rects = np.array([
        [0, 0, W, H],        # whole image
        [0, 0, 1, 1],        # first pixel
        [W - 1, H - 1, W, H],
        [5, 6, 5, 20],       # empty in x
        [5, 6, 9, 6],        # empty in y
        [0, 0, 0, 0],
        [W, H, W, H],        # empty at the far corner
        [3, 4, 10, 30],
    ], np.int32)
    bad = np.array([
        [-1, 0, 3, 3], [0, -1, 3, 3], [0, 0, W + 1, 3], [0, 0, 3, H + 1],
        [5, 0, 4, 3], [0, 5, 3, 4],
    ], np.int32)
    out = host(ncc.box(S, dev(np.concatenate([rects, bad]), d)))
    np.testing.assert_array_equal(out[:len(rects)], oracle_mod.box_batch(So, rects))
    assert out[len(rects) - 1] == img[4:30, 3:10].astype(np.int64).sum()
    assert np.all(out[len(rects):] == np.iinfo(np.int64).min)
    # n == 0 is a no-op
    import torch
    assert ncc.box(S, torch.empty((0, 4), dtype=torch.int32, device=d)).numel() == 0
