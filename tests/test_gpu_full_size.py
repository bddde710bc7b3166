"""The 4096 x 4096 workloads compared with the oracle in full, in the launch
configurations the benchmark times.

Headline (16 x 16 template cut from smooth noise): every coefficient and
every sums plane of the 4081 x 4081 map on the default route (the int8
matrix-core kernel), computed with the sums planes, without them (the
configuration the benchmark times) and given the tables, plus both tables.
Bank (64 templates, 32 cut and 32 uniform): all 64 maps of one 64-template
call (the benchmark's call), with and without sums, every coefficient and
every sums plane; the oracle runs 16 templates per test.  Sums bit for bit,
coefficients within 1e-5 absolute ("Image in shared memory": the per-window
sums; section 15.8: the tables)."""
import numpy as np
import pytest

from normalized_cross_correlation_amd import synth
from tests.gpu_util import COEF_ATOL, announce, dev, host, need_gpu

pytestmark = pytest.mark.gpu


def _coef_close(got, want):
    err = np.abs(got.astype(np.float64) - want.astype(np.float64))
    assert err.max() <= COEF_ATOL, "max |coef - oracle| = %g" % err.max()


def test_headline_full_map(oracle_mod):
    import torch
    import normalized_cross_correlation_amd as ncc
    d = need_gpu()
    announce("headline 4096x4096 16x16 full map")
    w = synth.make("headline")
    img, tpl = w["img"], w["tpl"]
    gi, gt = dev(img, d), dev(tpl, d)
    S, Q = ncc.sat_build(gi)
    coef_s, sums = ncc.correlate(gi, gt, want_sums=True)
    coef_n, _ = ncc.correlate(gi, gt)                       # no sums: as the benchmark times it
    coef_t, _ = ncc.correlate(gi, gt, tables=(S, Q))        # given the tables: the benchmark's step
    torch.cuda.synchronize()
    So, Qo = oracle_mod.sat_build(img)
    np.testing.assert_array_equal(host(S), So)
    np.testing.assert_array_equal(host(Q), Qo)
    del S, Q, So, Qo
    co, so = oracle_mod.correlate(img, tpl)
    np.testing.assert_array_equal(host(sums), so)           # SumI, SumISq, SumIT: every position
    for c in (coef_s, coef_n, coef_t):
        _coef_close(host(c), co)
    np.testing.assert_array_equal(host(coef_n), host(coef_s))
    np.testing.assert_array_equal(host(coef_t), host(coef_s))
    (cx, cy), = w["cut_xy"]
    assert abs(float(coef_s[0, cy, cx]) - 1.0) <= COEF_ATOL


@pytest.fixture(scope="module")
def bank_outputs():
    """The 64-template 4096 x 4096 call, with and without sums, on the host."""
    import torch
    import normalized_cross_correlation_amd as ncc
    d = need_gpu()
    announce("bank 4096x4096 x64: GPU maps")
    w = synth.make("bank")
    gi, gt = dev(w["img"], d), dev(w["tpl"], d)
    coef_s, sums = ncc.correlate(gi, gt, want_sums=True)
    coef_n, _ = ncc.correlate(gi, gt)
    torch.cuda.synchronize()
    out = {"w": w, "coef_s": host(coef_s), "sums": host(sums), "coef_n": host(coef_n)}
    del coef_s, sums, coef_n
    torch.cuda.empty_cache()
    return out


@pytest.mark.parametrize("part", [0, 1, 2, 3])
def test_bank_full_maps(oracle_mod, bank_outputs, part):
    b = bank_outputs
    w = b["w"]
    t0, t1 = 16 * part, 16 * (part + 1)
    announce("bank 4096x4096 maps %d..%d in full" % (t0, t1 - 1))
    co, so = oracle_mod.correlate(w["img"], w["tpl"][t0:t1])
    np.testing.assert_array_equal(b["sums"][:2], so[:2])              # SumI, SumISq
    np.testing.assert_array_equal(b["sums"][2 + t0:2 + t1], so[2:])   # SumIT of these templates
    _coef_close(b["coef_s"][t0:t1], co)
    np.testing.assert_array_equal(b["coef_n"][t0:t1], b["coef_s"][t0:t1])
    for t, (x, y) in enumerate(w["cut_xy"]):
        if t0 <= t < t1:
            assert abs(float(b["coef_s"][t, y, x]) - 1.0) <= COEF_ATOL
