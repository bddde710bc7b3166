"""ncc_sat_build_noalloc, the table build that allocates nothing (its scratch
is a fixed device array), against ncc_sat_build on the same inputs: tables
bit for bit, on two calls in a row, the second with a smaller image (the
array keeps the first call's contents; nothing in it needs to start at zero),
and against the oracle.  Images past the fixed scratch are rejected before
any launch, leaving the outputs untouched.  Called through the C ABI."""
import ctypes

import numpy as np
import pytest

from tests.gpu_util import announce, dev, host, need_gpu

pytestmark = pytest.mark.gpu
ERANGE = -2


def _noalloc(L, img, S, Q):
    import torch
    H, W = img.shape
    return L.ncc_sat_build_noalloc(img.data_ptr(), W, H, S.data_ptr(), Q.data_ptr(),
                                   ctypes.c_void_p(torch.cuda.current_stream().cuda_stream))


def test_noalloc_matches_sat_build(oracle_mod):
    import torch
    import normalized_cross_correlation_amd as ncc
    d = need_gpu()
    L = ncc.lib()
    rng = np.random.default_rng(31)
    # the headline size, then a smaller ragged image
    for H, W in ((4096, 4096), (300, 517)):
        announce("noalloc table build %dx%d" % (H, W))
        img = rng.integers(0, 256, (H, W), dtype=np.uint8)
        g = dev(img, d)
        S_ref, Q_ref = ncc.sat_build(g)
        S = torch.full((H, W), -1, dtype=torch.int64, device=d)
        Q = torch.full((H, W), -1, dtype=torch.int64, device=d)
        assert _noalloc(L, g, S, Q) == 0
        torch.cuda.synchronize()
        np.testing.assert_array_equal(host(S), host(S_ref))
        np.testing.assert_array_equal(host(Q), host(Q_ref))
        if H * W < 10 ** 6:
            So, Qo = oracle_mod.sat_build(img)
            np.testing.assert_array_equal(host(S), So)
            np.testing.assert_array_equal(host(Q), Qo)


def test_noalloc_rejects_past_its_scratch():
    import torch
    import normalized_cross_correlation_amd as ncc
    d = need_gpu()
    L = ncc.lib()
    announce("noalloc rejects 11600 x 11600")
    H = W = 11600  # build scratch ~16.8 MB > 16 MiB
    img = torch.zeros((1, 1), dtype=torch.uint8, device=d)  # never read: rejected first
    S = torch.full((1,), 5, dtype=torch.int64, device=d)
    rc = L.ncc_sat_build_noalloc(img.data_ptr(), W, H, S.data_ptr(), S.data_ptr(),
                                 ctypes.c_void_p(torch.cuda.current_stream().cuda_stream))
    assert rc == ERANGE
    assert int(S[0]) == 5
