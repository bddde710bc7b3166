// Internal declarations shared by the HIP sources of libncc.so.
// Written for gfx950 (CDNA4): 64-lane wavefronts, DPP row operations.
#pragma once

#include <hip/hip_runtime.h>
#include <cstddef>
#include <cstdint>

#include "ncc.h"

namespace ncc {

// Current value of a process-wide option (NCC_OPT_* of ncc.h).
int opt_get(int option);

// ---------------------------------------------------------------- tables ---
// Table build tiling: tiles of SAT_SW columns x SAT_TR rows (strip s, tile
// row g); the downsweep walks a tile in SAT_SUB bands of SAT_BH rows, a lane
// owning 2 adjacent columns and each of the 4 wavefronts SAT_BH / 4 rows of
// every band.
constexpr int SAT_SW = 128;
constexpr int SAT_BH = 32;
constexpr int SAT_SUB = 4;
constexpr int SAT_TR = SAT_BH * SAT_SUB;

struct SatWork {
    int nS, nG, nS4;   // strips, tile rows, strips rounded up to 4
    uint32_t *colsum;  // [2][nG][nS*SAT_SW] each tile's column sums
    uint32_t *btot;    // [2][nG][nS4]       each tile's total
    uint32_t *lcar;    // [2][H][nS]         each row's sum over the columns left of each strip
};

// State of the single-pass build, kept per (device, stream) between calls:
// ctl = {next tile ticket, finished tiles, call epoch, failure flag} and two
// parity buffers of published tile words ([2][capTiles][SAT_FWORDS] uint64).
// A call works in buffer epoch & 1 and clears the other one for the next
// call; the last tile to finish resets the counters and advances the epoch.
// Zero-filled when allocated and after a reported failure.  A workgroup whose
// bounded wait gives up, or that draws a ticket past the last tile, also
// stores 1 into *hostflag (pinned host memory, read by the host at the
// stream's next single-pass build and by ncc_stream_status).
struct SatState {
    uint32_t *ctl;
    uint64_t *words;
    int capTiles;
    uint32_t *hostflag;  // device address of the pinned host word
    int spin;            // polls of a wait before it gives up
};
constexpr int SAT_FW = 128;          // single-pass tile: columns
constexpr int SAT_FSUB = 4;          // ... bands of SAT_BH rows
constexpr int SAT_FWORDS = 4 * 128;  // words per tile: rows [2][128], columns [2][128]
size_t sat_state_bytes(int W, int H);
SatState sat_state_view(void *base, size_t bytes);

size_t sat_work_bytes(int W, int H);
SatWork sat_work_carve(void *base, int W, int H);
// Sets the state's ticket counter past the last tile (the state a call that
// never finished would leave): the failure path of ncc_stream_status' tests.
hipError_t sat_state_poison_launch(const SatState &fs, hipStream_t st);
// Tables of the H x W image whose row y starts at img + y * ip (ip >= W).
// fs.ctl == nullptr: the three-pass build; else the single-pass build
hipError_t sat_build_launch(const uint8_t *img, int W, int H, size_t ip, int64_t *S,
                            int64_t *Q, const SatWork &wk, const SatState &fs,
                            hipStream_t st);

hipError_t box_launch(const int64_t *S, int W, int H, const int32_t *rects,
                      int64_t n, int64_t *out, hipStream_t st);

// ------------------------------------------------------------- templates ---
// Per-template constants computed on the device.
struct TStat {
    long long sumT;    // sum of T
    long long sumTSq;  // sum of T^2
    long long varT;    // K*sumTSq - sumT^2 (exact)
    float varTf;       // (float)varT
    float rT;          // 1/sqrt(varT), 0 when varT == 0
};

// Packed forms of a template bank written by tpl_prep_launch:
//  rows: [nTpl][hT][WT4] uint32, each template row zero-padded to WT4 = ceil(wT/4)
//        dwords (little-endian bytes).
//  mfma: for banks eligible for the matrix-core kernel,
//        [nGroups of 16 templates][KSTEPS][64 lanes][16 bytes] int8 with
//        T' = T - 128; chunk c = 4*kstep + lane/16 is template row c / NB16,
//        bytes 16*(c % NB16) .. +15 (NB16 = ceil(wT/16)); padding is 0.
size_t tpl_rows_bytes(int wT, int hT, int nTpl);
size_t tpl_mfma_bytes(int wT, int hT, int nTpl);
hipError_t tpl_prep_launch(const uint8_t *tpl, int wT, int hT, int nTpl,
                           uint32_t *rows, int8_t *mfma, TStat *stats,
                           hipStream_t st);

// ----------------------------------------------------------- correlation ---
// A correlation over a view of the image: rows 0..H-1 of W bytes each, row y
// at img + y * ip, and positions (x, y), xs <= x < Wo, 0 <= y < Ho, whose
// windows lie inside the view (Wo + wT - 1 <= W, Ho + hT - 1 <= H).  Output
// of position (x, y) in plane p sits at element p * oplane + y * op + x - xs.
// Columns below xs are not outputs: a view may start left of the first
// position so that its rows start on an aligned address (streaming kernel
// only; the others take xs == 0).
struct CorrArgs {
    const uint8_t *img;
    const uint8_t *tpl;    // [nTpl][hT][wT] as given by the caller
    int W, H, wT, hT, nTpl, Wo, Ho;
    int xs;                // first output column of the view
    size_t ip;             // image row pitch (bytes)
    size_t op;             // output row pitch (elements)
    size_t oplane;         // output plane stride (elements)
    const uint32_t *rows;  // packed template rows
    const int8_t *mfma;    // packed bank operands (bank kernel only)
    const TStat *stats;
    int32_t *sums;         // nullable
    float *coef;
};

// Specialised single-template kernels (an on-chip table of each image strip
// supplies SumI / SumISq).  Returns hipErrorNotSupported when no kernel fits
// the shape.
bool corr_stream_supported(int wT, int hT);
hipError_t corr_stream_launch(const CorrArgs &a, int t, hipStream_t st);

// Single template up to 32 x 32 on the int8 matrix cores in 16 x 16 output
// tiles (one banded product per template row; window sums from running
// column sums of the tile's row sums).
bool corr_mtile_supported(int wT, int hT);
hipError_t corr_mtile_launch(const CorrArgs &a, int t, hipStream_t st);

// Single template on the int8 matrix cores (SumIT as a banded Toeplitz
// product; window sums from the strip's running column sums).
bool corr_toeplitz_supported(int wT, int hT);
bool corr_toeplitz_preferred(int Wo, int Ho);  // over the vector-unit kernel
hipError_t corr_toeplitz_launch(const CorrArgs &a, int t, hipStream_t st);

// Templates up to 32 bytes wide and 64 rows high on the vector units, window
// sums from the staged tile (no tables, no template preparation).
bool corr_tile_supported(int wT, int hT);
hipError_t corr_tile_launch(const CorrArgs &a, int t, hipStream_t st);

// Summed-area tables as the generic and FFT routes read them: view position
// (x, y) is table element (tx + x, ty + y), S and Q point at element
// (tx, ty), rows are `pitch` elements apart, and corners left of column 0 or
// above row 0 of the table read as zero.
struct Tables {
    const int64_t *S, *Q;
    size_t pitch;
    int tx, ty;
};

// Any shape: window sums from the full int64 tables.
bool corr_generic_supported(int wT, int hT);
hipError_t corr_generic_launch(const CorrArgs &a, int t, const Tables &tb, hipStream_t st);

// SumIT by 2-D FFT in double precision (large templates), SumI and SumISq
// from the full int64 tables.  Supported while the view's padded transform
// sizes stay within 8192 x 8192; needs corr_fft_bytes(W, H) of workspace (the
// spectra and the twiddle table).
bool corr_fft_supported(int W, int H);
size_t corr_fft_bytes(int W, int H);
hipError_t corr_fft_launch(const CorrArgs &a, const Tables &tb, void *work, hipStream_t st);

// Template bank on the int8 matrix cores.
bool corr_bank_supported(int wT, int hT, int nTpl);
hipError_t corr_bank_launch(const CorrArgs &a, hipStream_t st);

// ------------------------------------------------------ host utilities ---
// Kernel attributes (the dynamic LDS limit above 64 KB) are set once per
// device: set_once(flags, fn) runs fn on the current device unless it has
// already succeeded there.  Running it twice from racing threads is harmless.
constexpr int NCC_MAX_DEVICES = 64;
template <class F>
hipError_t set_once(bool (&flags)[NCC_MAX_DEVICES], F fn) {
    int dev = 0;
    hipError_t e = hipGetDevice(&dev);
    if (e != hipSuccess) return e;
    if (dev < 0 || dev >= NCC_MAX_DEVICES) return hipErrorInvalidDevice;
    if (flags[dev]) return hipSuccess;
    e = fn();
    if (e == hipSuccess) flags[dev] = true;
    return e;
}

// ---------------------------------------------------- device utilities ---
#ifdef __HIP_DEVICE_COMPILE__
#define NCC_DEV __device__ __forceinline__
#else
#define NCC_DEV __device__ inline
#endif

// DPP control codes (GFX9 encoding).
constexpr int DPP_ROW_SHR1 = 0x111;
constexpr int DPP_ROW_SHR2 = 0x112;
constexpr int DPP_ROW_SHR4 = 0x114;
constexpr int DPP_ROW_SHR8 = 0x118;
constexpr int DPP_ROW_ROR8 = 0x128;
constexpr int DPP_ROW_BCAST15 = 0x142;
constexpr int DPP_ROW_BCAST31 = 0x143;

// Inclusive prefix sum over the 64 lanes of a wavefront (Hillis-Steele on
// DPP: shifts within 16-lane rows, then the two row broadcasts).
NCC_DEV uint32_t wave_incl_scan_u32(uint32_t x) {
    x += (uint32_t)__builtin_amdgcn_update_dpp(0, (int)x, DPP_ROW_SHR1, 0xf, 0xf, false);
    x += (uint32_t)__builtin_amdgcn_update_dpp(0, (int)x, DPP_ROW_SHR2, 0xf, 0xf, false);
    x += (uint32_t)__builtin_amdgcn_update_dpp(0, (int)x, DPP_ROW_SHR4, 0xf, 0xf, false);
    x += (uint32_t)__builtin_amdgcn_update_dpp(0, (int)x, DPP_ROW_SHR8, 0xf, 0xf, false);
    x += (uint32_t)__builtin_amdgcn_update_dpp(0, (int)x, DPP_ROW_BCAST15, 0xa, 0xf, false);
    x += (uint32_t)__builtin_amdgcn_update_dpp(0, (int)x, DPP_ROW_BCAST31, 0xc, 0xf, false);
    return x;
}

template <int CTRL, int ROWMASK>
NCC_DEV uint64_t dpp_u64(uint64_t v) {
    uint32_t lo = (uint32_t)v, hi = (uint32_t)(v >> 32);
    lo = (uint32_t)__builtin_amdgcn_update_dpp(0, (int)lo, CTRL, ROWMASK, 0xf, false);
    hi = (uint32_t)__builtin_amdgcn_update_dpp(0, (int)hi, CTRL, ROWMASK, 0xf, false);
    return ((uint64_t)hi << 32) | lo;
}

NCC_DEV uint64_t wave_incl_scan_u64(uint64_t x) {
    x += dpp_u64<DPP_ROW_SHR1, 0xf>(x);
    x += dpp_u64<DPP_ROW_SHR2, 0xf>(x);
    x += dpp_u64<DPP_ROW_SHR4, 0xf>(x);
    x += dpp_u64<DPP_ROW_SHR8, 0xf>(x);
    x += dpp_u64<DPP_ROW_BCAST15, 0xa>(x);
    x += dpp_u64<DPP_ROW_BCAST31, 0xc>(x);
    return x;
}

// Sum over the wavefront, returned in every lane (uniform).
NCC_DEV uint32_t wave_sum_u32(uint32_t x) {
    return (uint32_t)__builtin_amdgcn_readlane((int)wave_incl_scan_u32(x), 63);
}

// Workgroups are handed to the 8 XCDs of the chip round-robin in launch
// order.  Launching ceil(ntiles/8)*8 workgroups and mapping launch index k to
// tile (k % 8) * ceil(ntiles/8) + k / 8 gives each XCD one contiguous run of
// tiles, so each XCD's L2 writes back one compact stretch of the output;
// indices past ntiles (returned as -1) do nothing.
constexpr int NUM_XCD = 8;
NCC_DEV int xcd_tile(int k, int ntiles) {
    const int per = (ntiles + NUM_XCD - 1) / NUM_XCD;
    const int t = (k % NUM_XCD) * per + k / NUM_XCD;
    return t < ntiles ? t : -1;
}
inline unsigned xcd_grid(int ntiles) {
    return (unsigned)((ntiles + NUM_XCD - 1) / NUM_XCD * NUM_XCD);
}

NCC_DEV uint32_t dot4u(uint32_t a, uint32_t b, uint32_t c) {
    return __builtin_amdgcn_udot4(a, b, c, false);
}

// Bytes s .. s+3 of the 8-byte little-endian value hi:lo (s in 0..3).
NCC_DEV uint32_t align_bytes(uint32_t hi, uint32_t lo, uint32_t s) {
    return __builtin_amdgcn_alignbyte(hi, lo, s);
}

// Mask keeping the low nb bytes of a dword (nb in 1..4).
NCC_DEV uint32_t byte_mask(int nb) {
    return nb >= 4 ? 0xffffffffu : ((1u << (8 * nb)) - 1u);
}

// Bytes x .. x+15 of row y (row y at img + y * ip) for images without
// 16-byte aligned rows: five aligned dwords, byte-aligned.  Each dword
// address is clamped to the dword holding the row's last byte, so every read
// touches an image byte (an aligned dword never straddles a page).  Bytes
// past the last row or column are then arbitrary: they feed only positions
// past Ho or Wo, which are not stored.
NCC_DEV uint4 load16_any(const uint8_t *img, size_t ip, int W, int H, int x, int y) {
    const uint8_t *row = img + (size_t)min(y, H - 1) * ip;
    const uint8_t *first = row + min(x, W - 1), *lastb = row + W - 1;
    const uint32_t sh = (uint32_t)((uintptr_t)first & 3);
    const uint32_t *base = (const uint32_t *)(first - sh);
    const uint32_t *last = (const uint32_t *)(lastb - ((uintptr_t)lastb & 3));
    uint32_t d[5];
#pragma unroll
    for (int k = 0; k < 5; k++) d[k] = *(base + k <= last ? base + k : last);
    return make_uint4(align_bytes(d[1], d[0], sh), align_bytes(d[2], d[1], sh),
                      align_bytes(d[3], d[2], sh), align_bytes(d[4], d[3], sh));
}

// The coefficient from exact integer numerator and window variance and the
// template's variance as float.  A zero variance yields 0: varI == 0 forces
// num == 0 (every window pixel equal), varT == 0 likewise.  For nonzero
// integer variances the product is >= 1 and 1/sqrt of it <= 1, so clamping
// 1/sqrt to [0, 1] (the instruction's clamp modifier) changes nothing but
// turns 1/sqrt(0) = inf into 1, and 0 * 1 = 0.
NCC_DEV float ncc_coef(float numf, float varIf, float varTf) {
    const float r = __builtin_amdgcn_fmed3f(__builtin_amdgcn_rsqf(varIf * varTf), 0.0f, 1.0f);
    return __builtin_amdgcn_fmed3f(numf * r, -1.0f, 1.0f);
}

}  // namespace ncc
