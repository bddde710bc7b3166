"""The library on several streams and under HIP graph capture.

Each (device, stream) has its own workspace, so calls on different streams
may run concurrently; a call whose workspace is already sized records into a
graph like any other kernel launch (no memory set or copy nodes), and every
replay reads the current contents of its input buffers.  Results are compared
with eager calls on one stream: tables and sums bit for bit, coefficients
bit for bit as well (the same kernels on the same data).
"""
import numpy as np
import pytest

from normalized_cross_correlation_amd import synth
from tests.gpu_util import announce, dev, host, need_gpu

pytestmark = pytest.mark.gpu


def _eager(ncc, img, tpl):
    import torch
    S, Q = ncc.sat_build(img)
    coef, sums = ncc.correlate(img, tpl, want_sums=True)
    torch.cuda.synchronize()
    return host(S), host(Q), host(coef), host(sums)


@pytest.mark.parametrize("tshape,sat_path,corr_path", [
    ((16, 16, 1), "two_pass", None), ((16, 16, 1), "two_pass", "single"),
    ((16, 16, 20), "two_pass", None), ((9, 11, 1), "two_pass", None), ((9, 11, 1), "two_pass", "generic"),
    ((16, 16, 1), "single_pass", None)])
def test_graph_capture_replays(tshape, sat_path, corr_path, ncc_opts):
    """Table build + correlation captured once, replayed on changing images
    (the 16 x 16 single template on both of its kernels: vector units by
    default at this size, matrix cores forced; a 9 x 11 template on the tile
    kernel by default and on the generic kernel, which reads the tables).  The single-pass table build
    keeps its call counters on the device, so its replays need nothing from
    the host either."""
    import torch
    import normalized_cross_correlation_amd as ncc
    d = need_gpu()
    ncc_opts(sat_build=sat_path)
    if corr_path:
        ncc_opts(route=corr_path)
    hT, wT, n = tshape
    announce("graph capture tpl %dx%d n=%d sat=%s corr=%s" % (hT, wT, n, sat_path, corr_path))
    cases = [synth.random_case(60 + i, 173, 301, hT, wT, nTpl=n, kind="smooth") for i in range(3)]
    img = dev(cases[0]["img"], d)
    tpl = dev(cases[0]["tpl"], d)
    s = torch.cuda.Stream(device=d)
    with torch.cuda.stream(s):
        # eager calls on the capture stream size its workspace
        ncc.sat_build(img)
        ncc.correlate(img, tpl, want_sums=True)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g, stream=s):
        S, Q = ncc.sat_build(img)
        coef, sums = ncc.correlate(img, tpl, want_sums=True)
    torch.cuda.synchronize()
    for rep in range(6):
        c = cases[rep % 3]
        img.copy_(dev(c["img"], d))  # eager work between replays
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        eS, eQ, ecoef, esums = _eager(ncc, img, tpl)
        np.testing.assert_array_equal(host(S), eS)
        np.testing.assert_array_equal(host(Q), eQ)
        np.testing.assert_array_equal(host(sums), esums)
        np.testing.assert_array_equal(host(coef), ecoef)


def test_two_streams_concurrent():
    """Table builds on one stream while correlations run on another."""
    import torch
    import normalized_cross_correlation_amd as ncc
    d = need_gpu()
    announce("two streams")
    a = synth.random_case(70, 520, 1100, 16, 16, nTpl=1, kind="smooth")
    b = synth.random_case(71, 300, 700, 16, 16, nTpl=5, kind="uniform")
    ia, ta = dev(a["img"], d), dev(a["tpl"], d)
    ib, tb = dev(b["img"], d), dev(b["tpl"], d)
    ref_a = _eager(ncc, ia, ta)
    ref_b = _eager(ncc, ib, tb)
    s1, s2 = torch.cuda.Stream(device=d), torch.cuda.Stream(device=d)
    outs = []
    for it in range(4):
        with torch.cuda.stream(s1):
            Sa, Qa = ncc.sat_build(ia)
            cb, sb = ncc.correlate(ib, tb, want_sums=True)
        with torch.cuda.stream(s2):
            Sb, Qb = ncc.sat_build(ib)
            ca, sa = ncc.correlate(ia, ta, want_sums=True)
        outs.append((Sa, Qa, ca, sa, Sb, Qb, cb, sb))
    torch.cuda.synchronize()
    for Sa, Qa, ca, sa, Sb, Qb, cb, sb in outs:
        np.testing.assert_array_equal(host(Sa), ref_a[0])
        np.testing.assert_array_equal(host(Qa), ref_a[1])
        np.testing.assert_array_equal(host(ca), ref_a[2])
        np.testing.assert_array_equal(host(sa), ref_a[3])
        np.testing.assert_array_equal(host(Sb), ref_b[0])
        np.testing.assert_array_equal(host(Qb), ref_b[1])
        np.testing.assert_array_equal(host(cb), ref_b[2])
        np.testing.assert_array_equal(host(sb), ref_b[3])


@pytest.mark.parametrize("sat_path", ["two_pass", "single_pass"])
def test_workspace_regrowth_between_calls(sat_path, ncc_opts):
    """Sizes that grow and shrink on one stream reuse or regrow its workspace
    (and, for the single-pass table build, its call state)."""
    import normalized_cross_correlation_amd as ncc
    d = need_gpu()
    ncc_opts(sat_build=sat_path)
    announce("workspace regrowth sat=%s" % sat_path)
    refs = []
    shapes = [(40, 70, 16, 16, 3), (400, 900, 16, 16, 1), (33, 50, 5, 7, 2), (500, 1000, 16, 16, 64),
              (20, 20, 4, 4, 1)]
    for i, (H, W, hT, wT, n) in enumerate(shapes):
        c = synth.random_case(80 + i, H, W, hT, wT, nTpl=n, kind="smooth")
        refs.append((c, _eager(ncc, dev(c["img"], d), dev(c["tpl"], d))))
    ncc.release()
    for c, ref in refs[::-1] + refs:
        got = _eager(ncc, dev(c["img"], d), dev(c["tpl"], d))
        for g_, r_ in zip(got, ref):
            np.testing.assert_array_equal(g_, r_)


@pytest.mark.parametrize("sat_path", ["two_pass", "single_pass"])
def test_graph_replay_after_workspace_growth(sat_path, ncc_opts):
    """A graph captured on a stream, then an eager call on the same stream
    that needs a larger workspace (and single-pass state): the block the
    graph recorded is retired, not freed, so every later replay still matches
    the eager results (generic route: the workspace holds the tables)."""
    import torch
    import normalized_cross_correlation_amd as ncc
    d = need_gpu()
    ncc_opts(sat_build=sat_path, route="generic")
    announce("graph replay after workspace growth sat=%s" % sat_path)
    small = [synth.random_case(90 + i, 150, 170, 9, 11, nTpl=2, kind="smooth") for i in range(2)]
    large = synth.random_case(95, 900, 1300, 9, 11, nTpl=2, kind="uniform")
    img = dev(small[0]["img"], d)
    tpl = dev(small[0]["tpl"], d)
    s = torch.cuda.Stream(device=d)
    with torch.cuda.stream(s):
        ncc.sat_build(img)
        ncc.correlate(img, tpl, want_sums=True)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g, stream=s):
        S, Q = ncc.sat_build(img)
        coef, sums = ncc.correlate(img, tpl, want_sums=True)
    torch.cuda.synchronize()
    limg, ltpl = dev(large["img"], d), dev(large["tpl"], d)
    for rep in range(4):
        with torch.cuda.stream(s):  # grows the stream's workspace on the first pass
            lS, lQ = ncc.sat_build(limg)
            lc, ls = ncc.correlate(limg, ltpl, want_sums=True)
        torch.cuda.synchronize()
        c = small[rep % 2]
        img.copy_(dev(c["img"], d))
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        eS, eQ, ecoef, esums = _eager(ncc, img, tpl)
        np.testing.assert_array_equal(host(S), eS)
        np.testing.assert_array_equal(host(Q), eQ)
        np.testing.assert_array_equal(host(sums), esums)
        np.testing.assert_array_equal(host(coef), ecoef)
    ncc.stream_status()
