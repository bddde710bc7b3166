// C ABI of libncc.so (declared in include/ncc.h): argument validation,
// options, the per-device, per-stream workspace cache, and dispatch to the
// kernels.
#include "ncc.h"
#include "ncc_internal.h"

#include <atomic>
#include <climits>
#include <cstring>
#include <map>
#include <mutex>
#include <utility>
#include <vector>

namespace ncc {

namespace {
// Process-wide options, indexed by NCC_OPT_*.
std::atomic<int> g_opt[7] = {0, NCC_ROUTE_AUTO, NCC_SAT_TWO_PASS, 0, 0, 1 << 22, 0};
}  // namespace

int opt_get(int option) {
    return option >= 1 && option <= 6 ? g_opt[option].load(std::memory_order_relaxed) : 0;
}

}  // namespace ncc

// ncc_sat_build_noalloc's build scratch: one fixed array per device, held
// until the process ends and shared by every call on that device.  Host code
// uses its device address from hipGetSymbolAddress, never the symbol itself.
static __device__ __align__(256) unsigned char scratch[NCC_NOALLOC_SCRATCH_BYTES];

namespace {

using namespace ncc;

std::mutex g_scratch_mu;
void *g_scratch[NCC_MAX_DEVICES];  // device address of `scratch` on each device

// The address of `scratch` on the current device, looked up at the first
// call there (with that device current).
int scratch_address(void **out) {
    int dev = 0;
    if (hipGetDevice(&dev) != hipSuccess) return NCC_EHIP;
    if (dev < 0 || dev >= NCC_MAX_DEVICES) return NCC_EHIP;
    std::lock_guard<std::mutex> lock(g_scratch_mu);
    if (!g_scratch[dev]) {
        void *p = nullptr;
        if (hipGetSymbolAddress(&p, HIP_SYMBOL(scratch)) != hipSuccess || !p) {
            (void)hipGetLastError();
            return NCC_EHIP;
        }
        g_scratch[dev] = p;
    }
    *out = g_scratch[dev];
    return NCC_OK;
}

struct Block {
    void *ptr = nullptr;
    size_t bytes = 0;
};

// What the library keeps for one (device, stream): the workspace, the
// single-pass build state with its pinned failure word, and the blocks that
// calls have outgrown.  Outgrown blocks are not freed before ncc_release: a
// HIP graph captured earlier on the stream may still replay kernels that use
// them.
struct StreamRec {
    Block work;
    Block state;
    uint32_t *hostflag = nullptr;  // pinned host word (host address)
    uint32_t *devflag = nullptr;   // its device address
    std::vector<void *> retired;
};

std::mutex g_mu;
std::map<std::pair<int, hipStream_t>, StreamRec> g_rec;

int capturing(hipStream_t st, bool *yes) {
    hipStreamCaptureStatus cs = hipStreamCaptureStatusNone;
    if (hipStreamIsCapturing(st, &cs) != hipSuccess) return NCC_EHIP;
    *yes = cs != hipStreamCaptureStatusNone;
    return NCC_OK;
}

// The record of (current device, st); the caller holds g_mu.
int rec_of(hipStream_t st, StreamRec **out) {
    int dev = 0;
    if (hipGetDevice(&dev) != hipSuccess) return NCC_EHIP;
    *out = &g_rec[std::make_pair(dev, st)];
    return NCC_OK;
}

// A block of at least `bytes` in b (grown by a quarter beyond the request
// against repeated small growth); a zero-filled one when `zero`.  Growing is
// refused during stream capture (NCC_EUNSUPPORTED: call once outside the
// capture to size the stream's blocks).  The caller holds g_mu.
int grow(StreamRec &r, Block &b, size_t bytes, bool zero, hipStream_t st) {
    if (b.ptr && b.bytes >= bytes) return NCC_OK;
    bool cap = false;
    int rc = capturing(st, &cap);
    if (rc != NCC_OK) return rc;
    if (cap) return NCC_EUNSUPPORTED;
    size_t want = zero ? bytes : bytes + bytes / 4;
    void *p = nullptr;
    if (hipMalloc(&p, want) != hipSuccess) {
        (void)hipGetLastError();
        want = bytes;
        if (hipMalloc(&p, want) != hipSuccess) {
            (void)hipGetLastError();
            return NCC_ENOMEM;
        }
    }
    if (zero && hipMemsetAsync(p, 0, want, st) != hipSuccess) {
        (void)hipFree(p);
        return NCC_EHIP;
    }
    if (b.ptr) r.retired.push_back(b.ptr);
    b.ptr = p;
    b.bytes = want;
    return NCC_OK;
}

int get_work(hipStream_t st, size_t bytes, void **out) {
    std::lock_guard<std::mutex> lock(g_mu);
    StreamRec *r = nullptr;
    int rc = rec_of(st, &r);
    if (rc != NCC_OK) return rc;
    rc = grow(*r, r->work, bytes, false, st);
    if (rc == NCC_OK) *out = r->work.ptr;
    return rc;
}

// A reported single-pass failure: waits for the stream, zero-fills its build
// state and clears the word.  Not possible during capture (the failure stays
// pending).  The caller holds g_mu.
int take_failure(StreamRec &r, hipStream_t st) {
    if (!r.hostflag || __atomic_load_n(r.hostflag, __ATOMIC_ACQUIRE) == 0) return NCC_OK;
    bool cap = false;
    if (capturing(st, &cap) != NCC_OK || cap) return NCC_EHIP;
    if (hipStreamSynchronize(st) != hipSuccess) return NCC_EHIP;
    if (r.state.ptr && (hipMemsetAsync(r.state.ptr, 0, r.state.bytes, st) != hipSuccess ||
                        hipStreamSynchronize(st) != hipSuccess))
        return NCC_EHIP;
    __atomic_store_n(r.hostflag, 0u, __ATOMIC_RELEASE);
    return NCC_EHIP;
}

// The single-pass build state of (current device, st): at least `bytes`,
// zero-filled when (re)allocated, with the pinned failure word.  Reports (and
// clears) a failure of an earlier single-pass build on the stream.
int get_state(hipStream_t st, size_t bytes, SatState *fs) {
    std::lock_guard<std::mutex> lock(g_mu);
    StreamRec *r = nullptr;
    int rc = rec_of(st, &r);
    if (rc != NCC_OK) return rc;
    rc = take_failure(*r, st);
    if (rc != NCC_OK) return rc;
    if (!r->hostflag) {
        bool cap = false;
        rc = capturing(st, &cap);
        if (rc != NCC_OK) return rc;
        if (cap) return NCC_EUNSUPPORTED;
        void *h = nullptr, *d = nullptr;
        if (hipHostMalloc(&h, 256, hipHostMallocMapped | hipHostMallocCoherent) != hipSuccess) {
            (void)hipGetLastError();
            return NCC_ENOMEM;
        }
        if (hipHostGetDevicePointer(&d, h, 0) != hipSuccess) {
            (void)hipHostFree(h);
            return NCC_EHIP;
        }
        std::memset(h, 0, 256);
        r->hostflag = (uint32_t *)h;
        r->devflag = (uint32_t *)d;
    }
    rc = grow(*r, r->state, bytes, true, st);
    if (rc != NCC_OK) return rc;
    *fs = sat_state_view(r->state.ptr, r->state.bytes);
    fs->hostflag = r->devflag;
    fs->spin = opt_get(NCC_OPT_SAT_SPIN);
    return NCC_OK;
}

int hip_status(hipError_t e) {
    if (e == hipSuccess) return NCC_OK;
    if (e == hipErrorNotSupported) return NCC_EUNSUPPORTED;
    return NCC_EHIP;
}

// Builds S and Q of the H x W image with row pitch ip on `st`, with `wk`
// (two-pass scratch) carved by the caller; the single-pass build when the
// option selects it.
int build_tables(const uint8_t *img, int W, int H, size_t ip, int64_t *S, int64_t *Q,
                 const SatWork &wk, hipStream_t st) {
    SatState fs{nullptr, nullptr, 0, nullptr, 0};
    if (opt_get(NCC_OPT_SAT_BUILD) == NCC_SAT_SINGLE_PASS) {
        int rc = get_state(st, sat_state_bytes(W, H), &fs);
        if (rc != NCC_OK) return rc;
        int stale = 1;
        if (g_opt[NCC_OPT_SAT_STALE].compare_exchange_strong(stale, 0)) {
            rc = hip_status(sat_state_poison_launch(fs, st));
            if (rc != NCC_OK) return rc;
        }
    }
    return hip_status(sat_build_launch(img, W, H, ip, S, Q, wk, fs, st));
}

size_t round256(size_t n) { return (n + 255) & ~(size_t)255; }

// Whether a template that no specialised kernel takes goes through the FFT
// numerator rather than the direct generic kernel: estimated times from the
// measured rates of both on this part (direct: ~55 T MAC/s for large
// templates; FFT: ~10 spectrum passes per template and 3 for the image, each
// pass moving the spectrum twice at ~5.3 TB/s).  At 4096 x 4096 the two
// meet near a 48 x 48 template (0.73 ms each).
bool fft_chosen(int route, int Wv, int Hv, int Wo, int Ho, int wT, int hT, int nTpl) {
    if (!corr_fft_supported(Wv, Hv)) return false;
    if (route == NCC_ROUTE_FFT) return true;
    if (route != NCC_ROUTE_AUTO) return false;
    const double spec = (double)corr_fft_bytes(Wv, Hv) / 3.0;
    const double t_fft = 20e-6 + (3.0 + 10.0 * nTpl) * 2.0 * spec / 5.3e12;
    const double t_direct = (double)nTpl * Wo * (double)Ho * wT * (double)hT / 55e12;
    return t_fft < t_direct;
}

// One correlation: positions x0 <= x < x0 + w, y0 <= y < y0 + h of the H x W
// image at img (row pitch ip bytes); output planes of h rows with pitch op
// elements; S, Q the caller's tables of the whole image (pitch W) or null.
// Arguments are validated by the caller; w, h >= 1.
struct Request {
    const uint8_t *img;
    int W, H;
    size_t ip;
    const uint8_t *tpl;
    int wT, hT, nTpl;
    int x0, y0, w, h;
    size_t op;
    int32_t *sums;
    float *coef;
    const int64_t *S, *Q;
};

int correlate_request(const Request &r, hipStream_t st) {
    const int wT = r.wT, hT = r.hT, nTpl = r.nTpl;
    const int route = opt_get(NCC_OPT_CORR_ROUTE);
    const bool autor = route == NCC_ROUTE_AUTO;
    const bool bank = autor && corr_bank_supported(wT, hT, nTpl);
    // single-template kernels: the matrix-core strip kernel for 16-row
    // templates (small launches, e.g. a local search, take the matrix-core
    // tile kernel below; NCC_ROUTE_SINGLE forces the strip kernel where it
    // applies); the vector-unit stream only when forced (NCC_ROUTE_DOT4)
    const bool single_route = autor || route == NCC_ROUTE_SINGLE;
    const bool toep_ok = single_route && corr_toeplitz_supported(wT, hT) &&
                         (route == NCC_ROUTE_SINGLE || corr_toeplitz_preferred(r.w, r.h));
    const bool stream_ok = toep_ok || (route == NCC_ROUTE_DOT4 && corr_stream_supported(wT, hT));
    // templates up to 32 x 32 that no kernel above takes: the matrix-core
    // tile kernel; then the vector-unit tile kernel (up to 32 x 64, or
    // forced by NCC_ROUTE_TILE)
    const bool mtile_ok = !bank && !stream_ok && single_route && corr_mtile_supported(wT, hT);
    const bool tile_ok = !bank && !stream_ok && !mtile_ok && (autor || route == NCC_ROUTE_TILE) &&
                         corr_tile_supported(wT, hT);
    const bool need_tables = !bank && !stream_ok && !mtile_ok && !tile_ok;  // the generic and FFT routes
    if (need_tables && !corr_generic_supported(wT, hT)) return NCC_EUNSUPPORTED;
    const bool fft = need_tables && fft_chosen(route, r.w + wT - 1, r.h + hT - 1, r.w, r.h, wT,
                                               hT, nTpl);
    const bool own_tables = need_tables && !r.S;  // tables built here, of the view

    // The view the kernels see: the rows and columns the positions' windows
    // cover.  For the streaming kernel on an image with 16-byte aligned rows,
    // the view starts at the 16-byte boundary at or left of x0 and its width
    // is rounded up to 16 bytes: x0 - xs and W are multiples of 16, so the
    // rounded width still ends inside the image row.
    int xs = 0, Wv = r.w + wT - 1;
    if (!bank && stream_ok && ((uintptr_t)r.img & 15) == 0 && r.ip % 16 == 0 && r.W % 16 == 0) {
        xs = r.x0 & 15;
        Wv = (xs + r.w + wT - 1 + 15) & ~15;
    }
    CorrArgs a;
    a.img = r.img + (size_t)r.y0 * r.ip + (size_t)(r.x0 - xs);
    a.tpl = r.tpl;
    a.W = Wv;
    a.H = r.h + hT - 1;
    a.wT = wT;
    a.hT = hT;
    a.nTpl = nTpl;
    a.Wo = xs + r.w;
    a.Ho = r.h;
    a.xs = xs;
    a.ip = r.ip;
    a.op = r.op;
    a.oplane = (size_t)r.h * r.op;
    a.rows = nullptr;
    a.mfma = nullptr;
    a.stats = nullptr;
    a.sums = r.sums;
    a.coef = r.coef;

    // the streaming and tile kernels derive everything from the caller's buffers
    if (!bank && (stream_ok || mtile_ok || tile_ok)) {
        for (int t = 0; t < nTpl; t++) {
            hipError_t e = tile_ok    ? corr_tile_launch(a, t, st)
                           : mtile_ok ? corr_mtile_launch(a, t, st)
                           : toep_ok  ? corr_toeplitz_launch(a, t, st)
                                      : corr_stream_launch(a, t, st);
            if (e != hipSuccess) return hip_status(e);
        }
        return NCC_OK;
    }

    // workspace: packed templates, per-template constants, and (table routes
    // without caller tables) the tables of the view and their build scratch,
    // and (FFT) the spectra
    const int W = a.W, H = a.H;
    size_t off_rows = 0;
    size_t off_mfma = round256(off_rows + tpl_rows_bytes(wT, hT, nTpl));
    size_t off_stats = round256(off_mfma + (bank ? tpl_mfma_bytes(wT, hT, nTpl) : 0));
    size_t off_S = round256(off_stats + sizeof(TStat) * (size_t)nTpl);
    size_t tbl = own_tables ? (size_t)W * H * sizeof(int64_t) : 0;
    size_t off_Q = round256(off_S + tbl);
    size_t off_sat = round256(off_Q + tbl);
    size_t off_fft = round256(off_sat + (own_tables ? sat_work_bytes(W, H) : 0));
    size_t total = off_fft + (fft ? corr_fft_bytes(W, H) : 0);

    void *ws = nullptr;
    int rc = get_work(st, total, &ws);
    if (rc != NCC_OK) return rc;
    char *base = (char *)ws;
    a.rows = (const uint32_t *)(base + off_rows);
    a.mfma = bank ? (const int8_t *)(base + off_mfma) : nullptr;
    a.stats = (const TStat *)(base + off_stats);

    hipError_t e = tpl_prep_launch(r.tpl, wT, hT, nTpl, (uint32_t *)(base + off_rows),
                                   bank ? (int8_t *)(base + off_mfma) : nullptr,
                                   (TStat *)(base + off_stats), st);
    if (e != hipSuccess) return hip_status(e);

    if (bank) return hip_status(corr_bank_launch(a, st));

    Tables tb;
    if (own_tables) {
        int64_t *Sm = (int64_t *)(base + off_S), *Qm = (int64_t *)(base + off_Q);
        SatWork wk = sat_work_carve(base + off_sat, W, H);
        rc = build_tables(a.img, W, H, a.ip, Sm, Qm, wk, st);
        if (rc != NCC_OK) return rc;
        tb = Tables{Sm, Qm, (size_t)W, 0, 0};
    } else {
        // the caller's tables of the whole image: the view starts at (x0, y0)
        const size_t o = (size_t)r.y0 * (size_t)r.W + (size_t)r.x0;
        tb = Tables{r.S + o, r.Q + o, (size_t)r.W, r.x0, r.y0};
    }
    if (fft) return hip_status(corr_fft_launch(a, tb, base + off_fft, st));
    for (int t = 0; t < nTpl; t++) {
        e = corr_generic_launch(a, t, tb, st);
        if (e != hipSuccess) return hip_status(e);
    }
    return NCC_OK;
}

}  // namespace

extern "C" {

int ncc_version(void) { return 201; }

const char *ncc_strerror(int status) {
    switch (status) {
        case NCC_OK: return "ok";
        case NCC_EINVAL: return "invalid argument";
        case NCC_ERANGE: return "size outside the integer widths of the method";
        case NCC_ENOMEM: return "workspace allocation failed";
        case NCC_EHIP: return "HIP runtime or kernel launch error";
        case NCC_EUNSUPPORTED: return "shape not supported by this build";
        default: return "unknown status";
    }
}

int ncc_set_option(int option, int value) {
    bool ok = false;
    switch (option) {
        case NCC_OPT_CORR_ROUTE: ok = value >= NCC_ROUTE_AUTO && value <= NCC_ROUTE_TILE; break;
        case NCC_OPT_SAT_BUILD: ok = value == NCC_SAT_TWO_PASS || value == NCC_SAT_SINGLE_PASS; break;
        case NCC_OPT_TZ_STRIP: ok = value == 0 || value == 16 || value == 32; break;
        case NCC_OPT_STREAM_ROWS: ok = value == 0 || value == 16 || value == 32 || value == 64; break;
        case NCC_OPT_SAT_SPIN: ok = value >= 0; break;
        case NCC_OPT_SAT_STALE: ok = value == 0 || value == 1; break;
        default: break;
    }
    if (!ok) return NCC_EINVAL;
    g_opt[option].store(value, std::memory_order_relaxed);
    return NCC_OK;
}

int ncc_get_option(int option, int *value) {
    if (!value || option < 1 || option > 6) return NCC_EINVAL;
    *value = g_opt[option].load(std::memory_order_relaxed);
    return NCC_OK;
}

int ncc_stream_status(void *stream) {
    hipStream_t st = (hipStream_t)stream;
    if (hipStreamSynchronize(st) != hipSuccess) return NCC_EHIP;
    std::lock_guard<std::mutex> lock(g_mu);
    StreamRec *r = nullptr;
    int rc = rec_of(st, &r);
    if (rc != NCC_OK) return rc;
    return take_failure(*r, st);
}

int ncc_sat_build(const uint8_t *img, int W, int H, int64_t *S, int64_t *Q, void *stream) {
    if (!img || !S || !Q || W < 1 || H < 1) return NCC_EINVAL;
    if (W > NCC_MAX_WIDTH) return NCC_ERANGE;
    // Q's corner is W*H*65025; keep it, and every byte offset, inside int64
    if ((unsigned long long)W * (unsigned long long)H > (1ull << 40)) return NCC_ERANGE;
    hipStream_t st = (hipStream_t)stream;
    void *ws = nullptr;
    int rc = get_work(st, sat_work_bytes(W, H), &ws);
    if (rc != NCC_OK) return rc;
    SatWork wk = sat_work_carve(ws, W, H);
    return build_tables(img, W, H, (size_t)W, S, Q, wk, st);
}

int ncc_sat_build_noalloc(const uint8_t *img, int W, int H, int64_t *S, int64_t *Q, void *stream) {
    if (!img || !S || !Q || W < 1 || H < 1) return NCC_EINVAL;
    if (W > NCC_MAX_WIDTH) return NCC_ERANGE;
    if ((unsigned long long)W * (unsigned long long)H > (1ull << 40)) return NCC_ERANGE;
    if (sat_work_bytes(W, H) > (size_t)NCC_NOALLOC_SCRATCH_BYTES) return NCC_ERANGE;
    void *ws = nullptr;
    int rc = scratch_address(&ws);
    if (rc != NCC_OK) return rc;
    const SatState none{nullptr, nullptr, 0, nullptr, 0};  // the two-pass build
    return hip_status(sat_build_launch(img, W, H, (size_t)W, S, Q, sat_work_carve(ws, W, H), none,
                                       (hipStream_t)stream));
}

int ncc_box(const int64_t *S, int W, int H, const int32_t *rects, int64_t n, int64_t *out,
            void *stream) {
    if (W < 1 || H < 1 || n < 0) return NCC_EINVAL;
    if (n == 0) return NCC_OK;
    if (!S || !rects || !out) return NCC_EINVAL;
    if ((unsigned long long)W * (unsigned long long)H > (1ull << 40)) return NCC_ERANGE;
    return hip_status(box_launch(S, W, H, rects, n, out, (hipStream_t)stream));
}

int ncc_correlate(const uint8_t *img, int W, int H, const uint8_t *tpl, int wT, int hT,
                  int nTpl, int32_t *sums_out, float *coef_out, const int64_t *S,
                  const int64_t *Q, void *stream) {
    if (!img || !tpl || !coef_out) return NCC_EINVAL;
    if (!S != !Q) return NCC_EINVAL;
    if (W < 1 || H < 1 || wT < 1 || hT < 1 || nTpl < 1 || wT > W || hT > H) return NCC_EINVAL;
    if (W > NCC_MAX_WIDTH) return NCC_ERANGE;
    if ((long long)wT * hT > NCC_MAX_TEMPLATE_PIXELS) return NCC_ERANGE;
    if ((unsigned long long)W * (unsigned long long)H > (1ull << 40)) return NCC_ERANGE;
    const int Wo = W - wT + 1, Ho = H - hT + 1;
    const unsigned long long planes = (unsigned long long)nTpl + 2;
    if ((unsigned long long)Wo * Ho * planes * 4ull > (1ull << 62)) return NCC_ERANGE;

    Request r;
    r.img = img;
    r.W = W;
    r.H = H;
    r.ip = (size_t)W;
    r.tpl = tpl;
    r.wT = wT;
    r.hT = hT;
    r.nTpl = nTpl;
    r.x0 = 0;
    r.y0 = 0;
    r.w = Wo;
    r.h = Ho;
    r.op = (size_t)Wo;
    r.sums = sums_out;
    r.coef = coef_out;
    r.S = S;
    r.Q = Q;
    return correlate_request(r, (hipStream_t)stream);
}

int ncc_correlate_rect(const uint8_t *img, int W, int H, size_t img_pitch, const uint8_t *tpl,
                       int wT, int hT, int nTpl, int x0, int y0, int w, int h,
                       size_t out_pitch, int32_t *sums_out, float *coef_out, const int64_t *S,
                       const int64_t *Q, void *stream) {
    if (!img || !tpl) return NCC_EINVAL;
    if (!S != !Q) return NCC_EINVAL;
    if (W < 1 || H < 1 || wT < 1 || hT < 1 || nTpl < 1 || wT > W || hT > H) return NCC_EINVAL;
    if (img_pitch < (size_t)W || w < 0 || h < 0 || out_pitch < (size_t)w) return NCC_EINVAL;
    if ((long long)wT * hT > NCC_MAX_TEMPLATE_PIXELS) return NCC_ERANGE;
    if (img_pitch > (1ull << 40) || (unsigned long long)img_pitch * (unsigned long long)H > (1ull << 48))
        return NCC_ERANGE;
    const int Wo = W - wT + 1, Ho = H - hT + 1;
    if (x0 < 0 || y0 < 0 || x0 > Wo - w || y0 > Ho - h) return NCC_ERANGE;
    // the view the windows cover obeys the width bound of the tables, and
    // its table corners stay inside int64
    if ((long long)w + wT - 1 > NCC_MAX_WIDTH) return NCC_ERANGE;
    if ((unsigned long long)(w + wT - 1) * (unsigned long long)(h + hT - 1) > (1ull << 40))
        return NCC_ERANGE;
    // caller tables cover the whole image: the same bounds as ncc_sat_build's
    if (S && (W > NCC_MAX_WIDTH || (unsigned long long)W * (unsigned long long)H > (1ull << 40)))
        return NCC_ERANGE;
    if (out_pitch > NCC_MAX_OUT_PITCH) return NCC_ERANGE;
    const unsigned long long planes = (unsigned long long)nTpl + 2;
    if ((unsigned long long)h * out_pitch * planes * 4ull > (1ull << 62)) return NCC_ERANGE;
    if (w == 0 || h == 0) return NCC_OK;  // no positions: nothing to write
    if (!coef_out) return NCC_EINVAL;

    Request r;
    r.img = img;
    r.W = W;
    r.H = H;
    r.ip = img_pitch;
    r.tpl = tpl;
    r.wT = wT;
    r.hT = hT;
    r.nTpl = nTpl;
    r.x0 = x0;
    r.y0 = y0;
    r.w = w;
    r.h = h;
    r.op = out_pitch;
    r.sums = sums_out;
    r.coef = coef_out;
    r.S = S;
    r.Q = Q;
    return correlate_request(r, (hipStream_t)stream);
}

void ncc_release(void) {
    std::lock_guard<std::mutex> lock(g_mu);
    int cur = 0;
    (void)hipGetDevice(&cur);
    for (auto &kv : g_rec) {
        StreamRec &r = kv.second;
        if (hipSetDevice(kv.first.first) != hipSuccess) continue;
        (void)hipDeviceSynchronize();
        if (r.work.ptr) (void)hipFree(r.work.ptr);
        if (r.state.ptr) (void)hipFree(r.state.ptr);
        for (void *p : r.retired) (void)hipFree(p);
        if (r.hostflag) (void)hipHostFree(r.hostflag);
    }
    g_rec.clear();
    (void)hipSetDevice(cur);
}

}  // extern "C"
