// C ABI of libncc.so (declared in include/ncc.h): argument validation,
// the per-device, per-stream workspace cache, and dispatch to the kernels.
#include "ncc.h"
#include "ncc_internal.h"

#include <climits>
#include <cstdlib>
#include <cstring>
#include <map>
#include <mutex>
#include <utility>

namespace {

using namespace ncc;

struct Work {
    void *ptr = nullptr;
    size_t bytes = 0;
};

std::mutex g_mu;
std::map<std::pair<int, hipStream_t>, Work> g_work;

// A workspace of at least `bytes` for (current device, stream).  Growing
// waits for the stream so that kernels still reading the old block finish
// first; that is not allowed under stream capture, which gets
// NCC_EUNSUPPORTED (call once outside the capture to size the workspace).
int get_work(hipStream_t st, size_t bytes, void **out) {
    int dev = 0;
    if (hipGetDevice(&dev) != hipSuccess) return NCC_EHIP;
    std::lock_guard<std::mutex> lock(g_mu);
    Work &w = g_work[std::make_pair(dev, st)];
    if (w.bytes >= bytes && w.ptr) {
        *out = w.ptr;
        return NCC_OK;
    }
    hipStreamCaptureStatus cs = hipStreamCaptureStatusNone;
    if (hipStreamIsCapturing(st, &cs) != hipSuccess) return NCC_EHIP;
    if (cs != hipStreamCaptureStatusNone) return NCC_EUNSUPPORTED;
    if (w.ptr) {
        if (hipStreamSynchronize(st) != hipSuccess) return NCC_EHIP;
        if (hipFree(w.ptr) != hipSuccess) return NCC_EHIP;
        w.ptr = nullptr;
        w.bytes = 0;
    }
    size_t want = bytes + bytes / 4;  // headroom against repeated small growth
    if (hipMalloc(&w.ptr, want) != hipSuccess) {
        (void)hipGetLastError();
        w.ptr = nullptr;
        if (hipMalloc(&w.ptr, bytes) != hipSuccess) {
            (void)hipGetLastError();
            w.ptr = nullptr;
            return NCC_ENOMEM;
        }
        want = bytes;
    }
    w.bytes = want;
    *out = w.ptr;
    return NCC_OK;
}

// State of the single-pass table build for (current device, stream): kept
// between calls and zero-filled when (re)allocated.  Same growth rules as
// the workspace.
std::map<std::pair<int, hipStream_t>, Work> g_state;

int get_state(hipStream_t st, size_t bytes, void **out, size_t *have) {
    int dev = 0;
    if (hipGetDevice(&dev) != hipSuccess) return NCC_EHIP;
    std::lock_guard<std::mutex> lock(g_mu);
    Work &w = g_state[std::make_pair(dev, st)];
    if (w.bytes >= bytes && w.ptr) {
        *out = w.ptr;
        *have = w.bytes;
        return NCC_OK;
    }
    hipStreamCaptureStatus cs = hipStreamCaptureStatusNone;
    if (hipStreamIsCapturing(st, &cs) != hipSuccess) return NCC_EHIP;
    if (cs != hipStreamCaptureStatusNone) return NCC_EUNSUPPORTED;
    if (w.ptr) {
        if (hipStreamSynchronize(st) != hipSuccess) return NCC_EHIP;
        if (hipFree(w.ptr) != hipSuccess) return NCC_EHIP;
        w.ptr = nullptr;
        w.bytes = 0;
    }
    if (hipMalloc(&w.ptr, bytes) != hipSuccess) {
        (void)hipGetLastError();
        w.ptr = nullptr;
        return NCC_ENOMEM;
    }
    if (hipMemsetAsync(w.ptr, 0, bytes, st) != hipSuccess) {
        (void)hipFree(w.ptr);
        w.ptr = nullptr;
        return NCC_EHIP;
    }
    w.bytes = bytes;
    *out = w.ptr;
    *have = bytes;
    return NCC_OK;
}

// Table build route: NCC_SAT_PATH = "fused" (single pass) or "passes".
bool sat_fused_from_env() {
    const char *e = std::getenv("NCC_SAT_PATH");
    return e && !std::strcmp(e, "fused");
}

// Builds S and Q on `st`, with `wk` (three-pass scratch) carved by the caller.
int build_tables(const uint8_t *img, int W, int H, int64_t *S, int64_t *Q, const SatWork &wk,
                 hipStream_t st) {
    SatState fs{nullptr, nullptr, 0};
    if (sat_fused_from_env()) {
        void *p = nullptr;
        size_t have = 0;
        int rc = get_state(st, sat_state_bytes(W, H), &p, &have);
        if (rc != NCC_OK) return rc;
        fs = sat_state_view(p, have);
    }
    hipError_t e = sat_build_launch(img, W, H, S, Q, wk, fs, st);
    return e == hipSuccess ? NCC_OK : (e == hipErrorNotSupported ? NCC_EUNSUPPORTED : NCC_EHIP);
}

size_t round256(size_t n) { return (n + 255) & ~(size_t)255; }

int hip_status(hipError_t e) {
    if (e == hipSuccess) return NCC_OK;
    if (e == hipErrorNotSupported) return NCC_EUNSUPPORTED;
    return NCC_EHIP;
}

// Which correlation route to take; NCC_CORR_PATH selects one explicitly
// ("generic", "single" for one template at a time, default "auto").
enum class Route { Auto, Generic, Single };
Route route_from_env() {
    const char *e = std::getenv("NCC_CORR_PATH");
    if (!e) return Route::Auto;
    if (!std::strcmp(e, "generic")) return Route::Generic;
    if (!std::strcmp(e, "single")) return Route::Single;
    return Route::Auto;
}

}  // namespace

extern "C" {

int ncc_version(void) { return 100; }

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
    return build_tables(img, W, H, S, Q, wk, st);
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
                  int nTpl, int32_t *sums_out, float *coef_out, void *stream) {
    if (!img || !tpl || !coef_out) return NCC_EINVAL;
    if (W < 1 || H < 1 || wT < 1 || hT < 1 || nTpl < 1 || wT > W || hT > H) return NCC_EINVAL;
    if (W > NCC_MAX_WIDTH) return NCC_ERANGE;
    if ((long long)wT * hT > NCC_MAX_TEMPLATE_PIXELS) return NCC_ERANGE;
    if ((unsigned long long)W * (unsigned long long)H > (1ull << 40)) return NCC_ERANGE;
    const int Wo = W - wT + 1, Ho = H - hT + 1;
    const unsigned long long planes = (unsigned long long)nTpl + 2;
    if ((unsigned long long)Wo * Ho * planes * 4ull > (1ull << 62)) return NCC_ERANGE;

    const Route route = route_from_env();
    const bool bank = route == Route::Auto && corr_bank_supported(wT, hT, nTpl);
    const bool stream_ok = route != Route::Generic && corr_stream_supported(wT, hT);
    const bool need_tables = !bank && !stream_ok;  // the generic route
    if (need_tables && !corr_generic_supported(wT, hT)) return NCC_EUNSUPPORTED;

    hipStream_t st = (hipStream_t)stream;
    CorrArgs a;
    a.img = img;
    a.tpl = tpl;
    a.W = W;
    a.H = H;
    a.wT = wT;
    a.hT = hT;
    a.nTpl = nTpl;
    a.Wo = Wo;
    a.Ho = Ho;
    a.rows = nullptr;
    a.mfma = nullptr;
    a.stats = nullptr;
    a.sums = sums_out;
    a.coef = coef_out;

    // the streaming kernel derives everything from the caller's buffers
    if (!bank && stream_ok) {
        for (int t = 0; t < nTpl; t++) {
            hipError_t e = corr_stream_launch(a, t, st);
            if (e != hipSuccess) return hip_status(e);
        }
        return NCC_OK;
    }

    // workspace: packed templates, per-template constants, and (generic
    // route only) the full tables and their build scratch
    size_t off_rows = 0;
    size_t off_mfma = round256(off_rows + tpl_rows_bytes(wT, hT, nTpl));
    size_t off_stats = round256(off_mfma + (bank ? tpl_mfma_bytes(wT, hT, nTpl) : 0));
    size_t off_S = round256(off_stats + sizeof(TStat) * (size_t)nTpl);
    size_t tbl = need_tables ? (size_t)W * H * sizeof(int64_t) : 0;
    size_t off_Q = round256(off_S + tbl);
    size_t off_sat = round256(off_Q + tbl);
    size_t total = off_sat + (need_tables ? sat_work_bytes(W, H) : 0);

    void *ws = nullptr;
    int rc = get_work(st, total, &ws);
    if (rc != NCC_OK) return rc;
    char *base = (char *)ws;
    a.rows = (const uint32_t *)(base + off_rows);
    a.mfma = bank ? (const int8_t *)(base + off_mfma) : nullptr;
    a.stats = (const TStat *)(base + off_stats);

    hipError_t e = tpl_prep_launch(tpl, wT, hT, nTpl, (uint32_t *)(base + off_rows),
                                   bank ? (int8_t *)(base + off_mfma) : nullptr,
                                   (TStat *)(base + off_stats), st);
    if (e != hipSuccess) return hip_status(e);

    if (bank) return hip_status(corr_bank_launch(a, st));

    const int64_t *S = nullptr, *Q = nullptr;
    if (need_tables) {
        int64_t *Sm = (int64_t *)(base + off_S), *Qm = (int64_t *)(base + off_Q);
        SatWork wk = sat_work_carve(base + off_sat, W, H);
        rc = build_tables(img, W, H, Sm, Qm, wk, st);
        if (rc != NCC_OK) return rc;
        S = Sm;
        Q = Qm;
    }
    for (int t = 0; t < nTpl; t++) {
        e = corr_generic_launch(a, t, S, Q, st);
        if (e != hipSuccess) return hip_status(e);
    }
    return NCC_OK;
}

void ncc_release(void) {
    std::lock_guard<std::mutex> lock(g_mu);
    int cur = 0;
    (void)hipGetDevice(&cur);
    for (auto &kv : g_work) {
        if (!kv.second.ptr) continue;
        if (hipSetDevice(kv.first.first) == hipSuccess) {
            (void)hipDeviceSynchronize();
            (void)hipFree(kv.second.ptr);
        }
    }
    g_work.clear();
    for (auto &kv : g_state) {
        if (!kv.second.ptr) continue;
        if (hipSetDevice(kv.first.first) == hipSuccess) {
            (void)hipDeviceSynchronize();
            (void)hipFree(kv.second.ptr);
        }
    }
    g_state.clear();
    (void)hipSetDevice(cur);
}

}  // extern "C"
