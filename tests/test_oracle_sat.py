"""Pins for the oracle's summed-area tables and box queries (CPU only).

What pins what (The CUDA Handbook ch. 15, section 15.8 "The Denominator:
Summed Area Tables"):
* the table definition (sum of every pixel above and to the left, inclusive;
  the oracle fills it by the 2-D inclusion-exclusion recurrence) ->
  brute-force definition on tiny images and numpy's cumulative sums (a
  library routine the oracle does not use);
* the four-corner box identity (Figure 15-7) -> every rectangle of tiny
  images against direct slice sums;
* the width analysis (int64 table, uint32 row running sums) -> the closed
  forms of an all-255 image.
"""
import os

import numpy as np
import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def _brute_sat(img):
    H, W = img.shape
    S = np.zeros((H, W), np.int64)
    Q = np.zeros((H, W), np.int64)
    for y in range(H):
        for x in range(W):
            blk = img[: y + 1, : x + 1].astype(np.int64)
            S[y, x] = blk.sum()
            Q[y, x] = (blk * blk).sum()
    return S, Q


@pytest.mark.parametrize("H,W,seed", [(1, 1, 0), (1, 7, 1), (6, 1, 2), (5, 9, 3), (12, 11, 4)])
def test_sat_matches_definition(oracle_mod, H, W, seed):
    rng = np.random.default_rng(seed)
    img = rng.integers(0, 256, (H, W), dtype=np.uint8)
    S, Q = oracle_mod.sat_build(img)
    Sb, Qb = _brute_sat(img)
    np.testing.assert_array_equal(S, Sb)
    np.testing.assert_array_equal(Q, Qb)


def test_sat_matches_library_cumsum(oracle_mod):
    rng = np.random.default_rng(7)
    img = rng.integers(0, 256, (37, 53), dtype=np.uint8)
    S, Q = oracle_mod.sat_build(img)
    i = img.astype(np.int64)
    np.testing.assert_array_equal(S, np.cumsum(np.cumsum(i, axis=0), axis=1))
    np.testing.assert_array_equal(Q, np.cumsum(np.cumsum(i * i, axis=1), axis=0))


def test_sat_is_not_transposed(oracle_mod):
    # a single bright pixel at (x=3, y=1) of a 4-row, 6-column image:
    # S(x,y) is 9 exactly where x >= 3 and y >= 1.
    img = np.zeros((4, 6), np.uint8)
    img[1, 3] = 9
    S, Q = oracle_mod.sat_build(img)
    ys, xs = np.mgrid[0:4, 0:6]
    np.testing.assert_array_equal(S, np.where((xs >= 3) & (ys >= 1), 9, 0))
    np.testing.assert_array_equal(Q, np.where((xs >= 3) & (ys >= 1), 81, 0))


@pytest.mark.parametrize("c", [0, 1, 17, 255])
def test_sat_constant_closed_form(oracle_mod, c):
    H, W = 13, 29
    S, Q = oracle_mod.sat_build(np.full((H, W), c, np.uint8))
    ys, xs = np.mgrid[0:H, 0:W]
    np.testing.assert_array_equal(S, c * (xs + 1) * (ys + 1))
    np.testing.assert_array_equal(Q, c * c * (xs + 1) * (ys + 1))


def _golden(name):
    vals = {}
    with open(os.path.join(ROOT, "tests", "golden", name)) as f:
        for line in f:
            line = line.split("#", 1)[0].strip()
            if line:
                k, v = line.split("=")
                vals[k.strip()] = int(v)
    return vals


def test_width_analysis_all_255(oracle_mod):
    """The pages' width analysis: sum reaches W*H*255, sum of squares
    W*H*255^2, both past int32 at 4096 x 4096, while one row's running sum of
    squares (at most W*255^2) fits uint32."""
    g = _golden("width_analysis.txt")
    W = H = 4096
    img = np.full((H, W), 255, np.uint8)
    S, Q = oracle_mod.sat_build(img)
    assert S.dtype == np.int64 and Q.dtype == np.int64
    assert int(S[-1, -1]) == g["S_full_4096_all255"] == W * H * 255
    assert int(Q[-1, -1]) == g["Q_full_4096_all255"] == W * H * 255 * 255
    assert int(Q[-1, -1]) > 2**31 and int(S[-1, -1]) > 2**31
    r1, r2 = oracle_mod.row_partials(img[:2])
    assert int(r2[0, -1]) == g["R2_row_4096_all255"] == W * 255 * 255 < 2**32
    assert int(r1[1, -1]) == W * 255
    # 512 x 512 is where the pages say the sum of squares passes 2^31
    assert 512 * 512 * 255 * 255 > 2**31


def test_row_partials_are_first_pass(oracle_mod):
    rng = np.random.default_rng(11)
    img = rng.integers(0, 256, (9, 31), dtype=np.uint8)
    r1, r2 = oracle_mod.row_partials(img)
    i = img.astype(np.int64)
    np.testing.assert_array_equal(r1, np.cumsum(i, axis=1))
    np.testing.assert_array_equal(r2, np.cumsum(i * i, axis=1))
    S, Q = oracle_mod.sat_build(img)
    # the column pass adds row partials down each column
    np.testing.assert_array_equal(np.diff(S, axis=0), r1[1:].astype(np.int64))
    np.testing.assert_array_equal(np.diff(Q, axis=0), r2[1:].astype(np.int64))


@pytest.mark.parametrize("H,W,seed", [(1, 1, 0), (1, 5, 1), (4, 1, 2), (5, 7, 3), (8, 6, 4)])
def test_box_all_rectangles(oracle_mod, H, W, seed):
    rng = np.random.default_rng(seed)
    img = rng.integers(0, 256, (H, W), dtype=np.uint8)
    S, Q = oracle_mod.sat_build(img)
    i = img.astype(np.int64)
    for y0 in range(H + 1):
        for y1 in range(y0, H + 1):
            for x0 in range(W + 1):
                for x1 in range(x0, W + 1):
                    blk = i[y0:y1, x0:x1]
                    assert oracle_mod.sat_box(S, x0, y0, x1, y1) == blk.sum()
                    assert oracle_mod.sat_box(Q, x0, y0, x1, y1) == (blk * blk).sum()


def test_box_full_and_empty(oracle_mod):
    rng = np.random.default_rng(5)
    img = rng.integers(0, 256, (10, 14), dtype=np.uint8)
    S, _ = oracle_mod.sat_build(img)
    assert oracle_mod.sat_box(S, 0, 0, 14, 10) == S[-1, -1] == img.astype(np.int64).sum()
    assert oracle_mod.sat_box(S, 3, 4, 3, 9) == 0
    assert oracle_mod.sat_box(S, 0, 10, 14, 10) == 0
    with pytest.raises(ValueError):
        oracle_mod.sat_box(S, 0, 0, 15, 10)


def test_box_batch_matches_slices(oracle_mod):
    from normalized_cross_correlation_amd import synth
    rng = np.random.default_rng(9)
    img = rng.integers(0, 256, (33, 47), dtype=np.uint8)
    S, Q = oracle_mod.sat_build(img)
    rects = synth.random_rects(rng, 47, 33, 500)
    i = img.astype(np.int64)
    out_s = oracle_mod.box_batch(S, rects)
    out_q = oracle_mod.box_batch(Q, rects)
    for k, (x0, y0, x1, y1) in enumerate(rects):
        assert out_s[k] == i[y0:y1, x0:x1].sum()
        assert out_q[k] == (i[y0:y1, x0:x1] ** 2).sum()
