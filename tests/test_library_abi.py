"""The C ABI of libncc.so without a GPU: the library loads, exports every
function include/ncc.h declares, and rejects bad arguments on the host before
any HIP call (those paths never touch a device, so they run here).

Pointers passed below are never dereferenced: every call is one the host
checks reject.  A call that passed them would reach the HIP runtime and, with
no device, return NCC_EHIP; the tests assert the specific rejection codes.
"""
import ctypes
import os
import re

import pytest

import normalized_cross_correlation_amd as ncc

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "ncc.h")

OK, EINVAL, ERANGE = 0, -1, -2
FAKE = ctypes.c_void_p(0x1000)  # stands for a device buffer; never read


def _declared():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(ncc_\w+)\s*\(", text)))


@pytest.fixture(scope="module")
def L():
    if not os.path.exists(ncc.LIB_PATH):
        from normalized_cross_correlation_amd import build
        build.build()
    return ncc.lib()


def test_exports_every_declared_function(L):
    decl = _declared()
    assert decl == sorted(ncc.ABI_FUNCTIONS)
    for name in decl:
        assert hasattr(L, name), name


def test_header_constants_match_binding():
    text = open(HEADER).read()
    consts = dict(re.findall(r"#define (NCC_\w+) \(?(-?[\w<\s]+?)\)?\s*(?:/\*|$)", text, flags=re.M))
    assert int(consts["NCC_MAX_WIDTH"]) == ncc.MAX_WIDTH
    assert int(consts["NCC_MAX_TEMPLATE_PIXELS"]) == ncc.MAX_TEMPLATE_PIXELS
    assert eval(consts["NCC_MAX_OUT_PITCH"]) == ncc.MAX_OUT_PITCH
    # the width bound is the largest W with W * 255^2 < 2^32, the template
    # bound the largest K with K * 255^2 < 2^31
    assert ncc.MAX_WIDTH * 65025 < 2 ** 32 <= (ncc.MAX_WIDTH + 1) * 65025
    assert ncc.MAX_TEMPLATE_PIXELS * 65025 < 2 ** 31 <= (ncc.MAX_TEMPLATE_PIXELS + 1) * 65025


def test_version_and_strerror(L):
    assert L.ncc_version() == ncc.ABI_VERSION == 201
    for code in (0, -1, -2, -3, -4, -5):
        assert L.ncc_strerror(code)
    assert L.ncc_strerror(-99) == b"unknown status"


def test_sat_build_rejects(L):
    assert L.ncc_sat_build(None, 4, 4, FAKE, FAKE, None) == EINVAL
    assert L.ncc_sat_build(FAKE, 0, 4, FAKE, FAKE, None) == EINVAL
    assert L.ncc_sat_build(FAKE, ncc.MAX_WIDTH + 1, 4, FAKE, FAKE, None) == ERANGE
    assert L.ncc_sat_build(FAKE, 65536, 1 << 25, FAKE, FAKE, None) == ERANGE


def test_sat_build_noalloc_rejects(L):
    f = L.ncc_sat_build_noalloc
    assert f(None, 4, 4, FAKE, FAKE, None) == EINVAL
    assert f(FAKE, 4, 0, FAKE, FAKE, None) == EINVAL
    assert f(FAKE, ncc.MAX_WIDTH + 1, 4, FAKE, FAKE, None) == ERANGE
    # past the fixed scratch: about W*H/8 bytes against 16 MiB
    assert f(FAKE, 16384, 16384, FAKE, FAKE, None) == ERANGE
    assert f(FAKE, 60000, 2300, FAKE, FAKE, None) == ERANGE


def test_box_rejects_and_empty(L):
    assert L.ncc_box(FAKE, 4, 4, FAKE, 0, FAKE, None) == OK  # nothing to do
    assert L.ncc_box(FAKE, 4, 4, FAKE, -1, FAKE, None) == EINVAL
    assert L.ncc_box(None, 4, 4, FAKE, 3, FAKE, None) == EINVAL
    assert L.ncc_box(FAKE, 0, 4, FAKE, 3, FAKE, None) == EINVAL


def test_correlate_rejects(L):
    def c(img, W, H, tpl, wT, hT, n, sums, coef, S=None, Q=None):
        return L.ncc_correlate(img, W, H, tpl, wT, hT, n, sums, coef, S, Q, None)
    assert c(None, 8, 8, FAKE, 3, 3, 1, None, FAKE) == EINVAL
    assert c(FAKE, 8, 8, FAKE, 9, 3, 1, None, FAKE) == EINVAL  # wT > W
    assert c(FAKE, 8, 8, FAKE, 3, 3, 0, None, FAKE) == EINVAL
    assert c(FAKE, 8, 8, FAKE, 3, 3, 1, None, None) == EINVAL
    assert c(FAKE, 8, 8, FAKE, 3, 3, 1, None, FAKE, S=FAKE) == EINVAL  # S without Q
    assert c(FAKE, 8, 8, FAKE, 3, 3, 1, None, FAKE, Q=FAKE) == EINVAL  # Q without S
    assert c(FAKE, ncc.MAX_WIDTH + 1, 8, FAKE, 3, 3, 1, None, FAKE) == ERANGE
    assert c(FAKE, 300, 300, FAKE, 182, 182, 1, None, FAKE) == ERANGE  # K > 33025


def _rect(L, W=40, H=30, ip=40, wT=5, hT=4, n=1, x0=0, y0=0, w=1, h=1, op=1, coef=FAKE,
          img=FAKE, S=None, Q=None):
    return L.ncc_correlate_rect(img, W, H, ip, FAKE, wT, hT, n, x0, y0, w, h, op, None, coef,
                                S, Q, None)


def test_correlate_rect_rejects(L):
    Wo, Ho = 36, 27  # 40 - 5 + 1, 30 - 4 + 1
    assert _rect(L, img=None) == EINVAL
    assert _rect(L, ip=39) == EINVAL                    # pitch below the width
    assert _rect(L, w=-1) == EINVAL
    assert _rect(L, w=5, op=4) == EINVAL                # output pitch below w
    assert _rect(L, coef=None) == EINVAL                # outputs needed for w, h > 0
    assert _rect(L, S=FAKE) == EINVAL                   # S without Q
    assert _rect(L, Q=FAKE) == EINVAL
    assert _rect(L, x0=-1) == ERANGE
    assert _rect(L, x0=Wo - 3, w=4, op=4) == ERANGE     # last window past the right edge
    assert _rect(L, y0=Ho - 2, h=3) == ERANGE
    assert _rect(L, x0=Wo, w=1) == ERANGE
    assert _rect(L, op=ncc.MAX_OUT_PITCH + 1) == ERANGE
    assert _rect(L, W=300, H=300, ip=300, wT=182, hT=182) == ERANGE
    big = ncc.MAX_WIDTH + 10
    assert _rect(L, W=big, H=4, ip=big, wT=1, hT=1, w=ncc.MAX_WIDTH + 1,
                 op=ncc.MAX_WIDTH + 1) == ERANGE        # the view past the width bound


def test_correlate_rect_empty_is_noop(L):
    # no positions: nothing launched, outputs may be null
    assert _rect(L, w=0, op=0, coef=None) == OK
    assert _rect(L, x0=36, w=0, op=0, coef=None) == OK  # empty at the right edge
    assert _rect(L, h=0, w=3, op=3, coef=None) == OK
    assert _rect(L, x0=40, w=0, op=0, coef=None) == ERANGE  # still validated


def test_options(L):
    """ncc_set_option / ncc_get_option: defaults, accepted values, rejected
    options and values (which leave the setting unchanged)."""
    v = ctypes.c_int()
    defaults = {1: 0, 2: 0, 3: 0, 4: 0, 5: 1 << 22, 6: 0}
    for opt, want in defaults.items():
        assert L.ncc_get_option(opt, ctypes.byref(v)) == OK
        assert v.value == want, (opt, v.value)
    assert L.ncc_get_option(0, ctypes.byref(v)) == EINVAL
    assert L.ncc_get_option(7, ctypes.byref(v)) == EINVAL
    assert L.ncc_get_option(1, None) == EINVAL
    good = {1: [0, 1, 2, 3, 4, 5], 2: [0, 1], 3: [0, 16, 32], 4: [0, 16, 32, 64], 5: [0, 7, 1 << 22],
            6: [0, 1]}
    bad = {1: [-1, 6], 2: [-1, 2], 3: [8, 64], 4: [8, 128], 5: [-1], 6: [2, -1]}
    for opt in good:
        for val in good[opt]:
            assert L.ncc_set_option(opt, val) == OK
            assert L.ncc_get_option(opt, ctypes.byref(v)) == OK and v.value == val
        last = good[opt][-1]
        for val in bad[opt]:
            assert L.ncc_set_option(opt, val) == EINVAL
            assert L.ncc_get_option(opt, ctypes.byref(v)) == OK and v.value == last
        assert L.ncc_set_option(opt, defaults[opt]) == OK
    assert L.ncc_set_option(99, 0) == EINVAL
    # the binding's names and context manager
    with ncc.options(route="generic", sat_build="single_pass", stream_rows=32):
        assert ncc.get_option("route") == 1
        assert ncc.get_option("sat_build") == 1
        assert ncc.get_option("stream_rows") == 32
    assert ncc.get_option("route") == 0 and ncc.get_option("sat_build") == 0
    assert ncc.get_option("stream_rows") == 0
    with pytest.raises(ncc.NCCError):
        ncc.set_option("tz_strip", 24)
    # every option and value name the header defines matches the binding
    text = open(HEADER).read()
    header_name = {"route": "CORR_ROUTE"}
    for name, num in ncc.OPTIONS.items():
        hn = header_name.get(name, name.upper())
        assert re.search(r"#define NCC_OPT_%s %d\b" % (hn, num), text), name
    for name, num in ncc.ROUTES.items():
        assert re.search(r"#define NCC_ROUTE_%s %d\b" % (name.upper(), num), text), name


def test_library_reads_no_environment():
    """Routes are chosen by ncc_set_option only: the library's sources call
    no getenv (a caller's environment cannot change what a call does)."""
    csrc = os.path.join(ROOT, "normalized_cross_correlation_amd", "csrc")
    for f in sorted(os.listdir(csrc)):
        text = open(os.path.join(csrc, f)).read()
        assert "getenv" not in text, f


def test_peaks_library_exports():
    """The benchmark's microbenchmark library (not part of the C ABI)."""
    from normalized_cross_correlation_amd import build
    if not os.path.exists(build.PEAKS_LIB):
        build.build()
    P = ctypes.CDLL(build.PEAKS_LIB)
    for name in ("ncc_peak_props", "ncc_peak_write", "ncc_peak_dot4", "ncc_peak_mfma_i8"):
        assert hasattr(P, name), name
    P.ncc_peak_write.argtypes = [ctypes.c_void_p, ctypes.c_size_t, ctypes.c_int, ctypes.c_void_p]
    # shapes it cannot tile are refused before any launch
    assert P.ncc_peak_write(FAKE, 1 << 20, 1000, None) == -1
    assert P.ncc_peak_write(None, 1 << 20, 1024, None) == -1
