"""Caller-supplied summed-area tables (ncc_correlate / ncc_correlate_rect with
S, Q; section 15.8: one table serves every window, every template of a bank
and every shift of an FFT search).

The generic and FFT routes read their window sums from the given full-image
tables, in place, also for a search rectangle whose windows start inside the
image (corners left of and above the rectangle are table elements there).
Every output must equal the output with the tables built internally bit for
bit (sums and coefficients: the same integers and the same float steps) and
the oracle (sums bit for bit, coefficients within 1e-5).  The specialised
kernels form the same integers on chip and ignore the tables: their outputs
are unchanged by them.  Called through the C ABI (ctypes) with raw pointers.
"""
import ctypes

import numpy as np
import pytest

from normalized_cross_correlation_amd import synth
from tests.gpu_util import COEF_ATOL, announce, dev, host, need_gpu, route

pytestmark = pytest.mark.gpu


def _abi_correlate(img, tpl, S, Q, want_sums=True):
    """ncc_correlate through ctypes; S, Q torch tensors or None."""
    import torch
    import normalized_cross_correlation_amd as ncc
    L = ncc.lib()
    H, W = img.shape
    n, hT, wT = tpl.shape
    coef = torch.full((n, H - hT + 1, W - wT + 1), -7.0, dtype=torch.float32, device=img.device)
    sums = (torch.full((2 + n, H - hT + 1, W - wT + 1), -7, dtype=torch.int32, device=img.device)
            if want_sums else None)
    rc = L.ncc_correlate(img.data_ptr(), W, H, tpl.data_ptr(), wT, hT, n,
                         sums.data_ptr() if sums is not None else None, coef.data_ptr(),
                         S.data_ptr() if S is not None else None,
                         Q.data_ptr() if Q is not None else None,
                         ctypes.c_void_p(torch.cuda.current_stream().cuda_stream))
    assert rc == 0, rc
    torch.cuda.synchronize()
    return host(coef), host(sums) if sums is not None else None


@pytest.mark.parametrize("rname,H,W,hT,wT,n,seed", [
    ("generic", 70, 90, 9, 11, 1, 1),
    ("generic", 150, 170, 40, 33, 2, 2),   # larger than the tile kernel takes
    ("generic", 33, 47, 1, 1, 1, 3),
    ("fft", 120, 100, 21, 13, 1, 4),
    ("fft", 40, 60, 9, 11, 3, 5),           # three templates share the spectrum
    (None, 300, 257, 50, 45, 1, 6),         # the library's own choice (generic)
    (None, 200, 260, 16, 16, 1, 7),         # a specialised kernel: tables not read
    (None, 200, 260, 16, 16, 5, 8),         # the bank kernel: tables not read
    (None, 90, 100, 20, 24, 1, 9),          # the tile kernel: tables not read
])
def test_correlate_with_caller_tables(oracle_mod, rname, H, W, hT, wT, n, seed):
    import normalized_cross_correlation_amd as ncc
    d = need_gpu()
    announce("caller tables route=%s %dx%d tpl %dx%d n=%d" % (rname, H, W, hT, wT, n))
    c = synth.random_case(100 + seed, H, W, hT, wT, nTpl=n, kind="smooth" if seed % 2 else "uniform")
    img, tpl = dev(c["img"], d), dev(c["tpl"], d)
    S, Q = ncc.sat_build(img)
    with route(rname):
        c_own, s_own = _abi_correlate(img, tpl, None, None)
        c_tab, s_tab = _abi_correlate(img, tpl, S, Q)
        c_tab2, _ = _abi_correlate(img, tpl, S, Q, want_sums=False)
    np.testing.assert_array_equal(s_tab, s_own)
    np.testing.assert_array_equal(c_tab, c_own)
    np.testing.assert_array_equal(c_tab2, c_own)
    co, so = oracle_mod.correlate(c["img"], c["tpl"])
    np.testing.assert_array_equal(s_tab, so)
    assert np.abs(c_tab.astype(np.float64) - co).max() <= COEF_ATOL


@pytest.mark.parametrize("rname,x0,y0,w,h", [
    ("generic", 0, 0, 5, 4),      # the image's corner: table edges read as zero
    ("generic", 13, 9, 31, 17),   # inside: corners above and left are table elements
    ("generic", 0, 21, 40, 3),    # left edge only
    ("generic", 17, 0, 1, 30),    # top edge only
    ("generic", 70, 50, 12, 11),  # the bottom-right corner of the valid positions
    ("fft", 13, 9, 31, 17),
    ("fft", 0, 0, 82, 61),        # every position
    ("fft", 41, 33, 1, 1),
])
def test_rect_with_caller_tables(oracle_mod, rname, x0, y0, w, h):
    """A pitched image and pitched output; the tables are of the whole image."""
    import torch
    import normalized_cross_correlation_amd as ncc
    d = need_gpu()
    announce("rect caller tables route=%s (%d,%d) %dx%d" % (rname, x0, y0, w, h))
    H, W, hT, wT = 70, 90, 10, 9  # valid positions 82 x 61
    c = synth.random_case(131, H, W, hT, wT, nTpl=2, kind="smooth")
    big = torch.zeros((H, W + 13), dtype=torch.uint8, device=d)
    big[:, 5:5 + W] = dev(c["img"], d)
    img = big[:, 5:5 + W]                       # row pitch W + 13, odd address
    S, Q = ncc.sat_build(dev(c["img"], d))      # tables of the dense copy: [H][W]
    tpl = dev(c["tpl"], d)
    with route(rname):
        c_own, s_own = ncc.correlate_rect(img, tpl, x0, y0, w, h, want_sums=True, out_pitch=w + 3)
        c_tab, s_tab = ncc.correlate_rect(img, tpl, x0, y0, w, h, want_sums=True, out_pitch=w + 3,
                                          tables=(S, Q))
    torch.cuda.synchronize()
    np.testing.assert_array_equal(host(s_tab), host(s_own))
    np.testing.assert_array_equal(host(c_tab), host(c_own))
    co, so = oracle_mod.correlate_rect(c["img"], c["tpl"], x0, y0, w, h)
    np.testing.assert_array_equal(host(s_tab), so)
    assert np.abs(host(c_tab).astype(np.float64) - co).max() <= COEF_ATOL


def test_caller_tables_skip_the_build(oracle_mod):
    """With caller tables the generic route launches no table-build kernel:
    poisoned workspace tables would show if it read them, and the build's
    option (the single-pass build with a stale state) would report a failure
    if it ran."""
    import normalized_cross_correlation_amd as ncc
    d = need_gpu()
    announce("caller tables: no build")
    c = synth.random_case(140, 120, 130, 20, 40, nTpl=1, kind="smooth")
    img, tpl = dev(c["img"], d), dev(c["tpl"], d)
    S, Q = ncc.sat_build(img)
    ncc.stream_status()
    with ncc.options(route="generic", sat_build="single_pass", sat_stale=1):
        coef, sums = ncc.correlate(img, tpl, want_sums=True, tables=(S, Q))
        ncc.stream_status()                      # no single-pass build ran: nothing to report
        assert ncc.get_option("sat_stale") == 1  # still armed: no build consumed it
        ncc.set_option("sat_stale", 0)
    co, so = oracle_mod.correlate(c["img"], c["tpl"])
    np.testing.assert_array_equal(host(sums), so)
    assert np.abs(host(coef).astype(np.float64) - co).max() <= COEF_ATOL
