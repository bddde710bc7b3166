"""Failures of the single-pass (decoupled look-back) table build reach the
caller (section 15.8: the look-back's flags; its bounded waits).

Failures are forced from the host, and every kernel still exits normally:
  - a stale build state (option sat_stale: the tile ticket counter starts past
    the last tile, as a call that never finished would leave it): every
    workgroup draws a ticket past the end, writes nothing and raises the
    failure word;
  - no waiting at all (option sat_spin = 0): a look-back that meets a word
    not yet published gives up at once.
The report comes from ncc_stream_status or the stream's next single-pass
build (NCC_EHIP, once), which also reset the state so later builds are exact.
"""
import numpy as np
import pytest

import normalized_cross_correlation_amd as ncc
from tests.gpu_util import announce, dev, host, need_gpu

pytestmark = pytest.mark.gpu
EHIP = -4
INT64_MIN = np.iinfo(np.int64).min


def _img(seed, H, W):
    return np.random.default_rng(seed).integers(0, 256, (H, W), dtype=np.uint8)


def test_stale_state_reported_by_stream_status(oracle_mod):
    import torch
    d = need_gpu()
    announce("single-pass stale state -> ncc_stream_status")
    img = _img(1, 300, 517)
    So, Qo = oracle_mod.sat_build(img)
    g = dev(img, d)
    with ncc.options(sat_build="single_pass"):
        ncc.stream_status()                      # nothing pending
        S = torch.full((300, 517), 7, dtype=torch.int64, device=d)
        Q = torch.full((300, 517), 9, dtype=torch.int64, device=d)
        ncc.set_option("sat_stale", 1)
        ncc.sat_build(g, S, Q)                   # enqueued: returns before it runs
        assert ncc.get_option("sat_stale") == 0  # the hook is one-shot
        with pytest.raises(ncc.NCCError) as e:
            ncc.stream_status()
        assert e.value.code == EHIP
        # no tile was drawn: nothing written
        assert bool((S == 7).all()) and bool((Q == 9).all())
        ncc.stream_status()                      # reported once
        S2, Q2 = ncc.sat_build(g)                # the reset state builds exactly
        ncc.stream_status()
    np.testing.assert_array_equal(host(S2), So)
    np.testing.assert_array_equal(host(Q2), Qo)


def test_stale_state_reported_by_next_build(oracle_mod):
    import torch
    d = need_gpu()
    announce("single-pass stale state -> next build")
    img = _img(2, 129, 260)
    So, Qo = oracle_mod.sat_build(img)
    g = dev(img, d)
    with ncc.options(sat_build="single_pass"):
        ncc.set_option("sat_stale", 1)
        ncc.sat_build(g)
        torch.cuda.synchronize()
        with pytest.raises(ncc.NCCError) as e:   # the next single-pass build reports it
            ncc.sat_build(g)
        assert e.value.code == EHIP
        S, Q = ncc.sat_build(g)
        ncc.stream_status()
    np.testing.assert_array_equal(host(S), So)
    np.testing.assert_array_equal(host(Q), Qo)


def test_stale_state_reported_through_correlate(oracle_mod):
    """The generic route builds its tables with the selected build: the
    failure reaches ncc_stream_status from there too."""
    import torch
    d = need_gpu()
    announce("single-pass stale state inside the generic route")
    img = _img(3, 90, 100)
    tpl = img[10:50, 20:60].copy()[None]
    with ncc.options(sat_build="single_pass", route="generic"):
        ncc.set_option("sat_stale", 1)
        ncc.correlate(dev(img, d), dev(tpl, d))
        with pytest.raises(ncc.NCCError) as e:
            ncc.stream_status()
        assert e.value.code == EHIP
        coef, sums = ncc.correlate(dev(img, d), dev(tpl, d), want_sums=True)
        ncc.stream_status()
    co, so = oracle_mod.correlate(img, tpl)
    np.testing.assert_array_equal(host(sums), so)


@pytest.mark.parametrize("H,W,seed", [(4096, 4096, 4), (2000, 3000, 5)])
def test_no_wait_gives_up_visibly(oracle_mod, H, W, seed):
    """sat_spin = 0: every entry is either the exact table value or
    INT64_MIN, and the build is reported failed exactly when an INT64_MIN
    was written (a tile that gave up, or read a word of one that did)."""
    import torch
    d = need_gpu()
    announce("single-pass no-wait %dx%d" % (H, W))
    img = _img(seed, H, W)
    So, Qo = oracle_mod.sat_build(img)
    g = dev(img, d)
    with ncc.options(sat_build="single_pass"):
        ncc.stream_status()
        fails = 0
        for rep in range(3):
            with ncc.options(sat_spin=0):
                S, Q = ncc.sat_build(g)
            try:
                ncc.stream_status()
                failed = False
            except ncc.NCCError as e:
                assert e.code == EHIP
                failed = True
            s, q = host(S), host(Q)
            bad_s, bad_q = s == INT64_MIN, q == INT64_MIN
            np.testing.assert_array_equal(s[~bad_s], So[~bad_s])
            np.testing.assert_array_equal(q[~bad_q], Qo[~bad_q])
            assert failed == bool(bad_s.any() or bad_q.any())
            fails += failed
        announce("no-wait builds that gave up: %d of 3" % fails)
        S, Q = ncc.sat_build(g)                  # default spin limit: exact
        ncc.stream_status()
    np.testing.assert_array_equal(host(S), So)
    np.testing.assert_array_equal(host(Q), Qo)
