// SumIT of large templates through the frequency domain: the correlation
// numerator as a product of Fourier transforms, with SumI and SumISq from the
// summed-area tables as on every other route (The CUDA Handbook ch. 15,
// section 15.8: the tables serve the denominator of any numerator, the FFT
// one included; the pages name that numerator without giving its method).
//
// SumIT(x, y) = sum_{j,i} I(y+j, x+i) T(j, i) is the cyclic cross-correlation
// of I with T zero-padded to P x Qn (P >= H, Qn >= W, powers of two): at a
// valid position no index wraps.  It is the inverse 2-D DFT of
// DFT(I) . conj(DFT(T)), evaluated here in double precision.  SumIT is an
// integer below 2^31 and the round-off of the double evaluation is of order
// eps * log2(P Qn) * |I|_2 * |T|_2 <= 2e-3 at every size this route takes
// (P, Qn <= 8192, K <= 33025), so rounding to the nearest integer gives it
// exactly.
//
// Layout: a row's real transform of length Qn is taken as a complex one of
// length M = Qn / 2 (even samples real, odd imaginary) and split into the
// M + 1 half-spectrum columns; columns are transformed in two in-place passes
// of lengths P1 x P2 = P over rows n1 * P2 + n2 (the four-step split).
// Forward transforms run decimation in frequency (natural order in, digit-
// reversed order out) and inverse ones decimation in time (that order in,
// natural order out), so no pass reorders data, and the product of the two
// spectra is taken in whatever order both are stored.  Each transform runs in
// LDS; a pass reads and writes the spectrum once.
#include "ncc_internal.h"

namespace ncc {

namespace {

constexpr int TW_LOG = 14;
constexpr int TWN = 1 << TW_LOG;  // twiddle table: exp(-2 pi i k / TWN), k < TWN
constexpr int FFT_T = 256;        // threads per workgroup of the column passes
constexpr int ROW_T = 1024;       // ... of the row transforms (one row per workgroup: enough
                                  //   wavefronts per CU at up to 96 KB of LDS each)
constexpr int ROW_MAXX = 8;       // outputs per lane in the last row pass (8192 / ROW_T)
constexpr int FFT_TB = 32;        // columns per workgroup in the column passes
constexpr int FFT_MAX_LOG = 13;   // transform lengths up to 8192 per dimension

__device__ __forceinline__ double2 cadd(double2 a, double2 b) { return make_double2(a.x + b.x, a.y + b.y); }
__device__ __forceinline__ double2 csub(double2 a, double2 b) { return make_double2(a.x - b.x, a.y - b.y); }
__device__ __forceinline__ double2 cmul(double2 a, double2 b) {
    return make_double2(a.x * b.x - a.y * b.y, a.x * b.y + a.y * b.x);
}
__device__ __forceinline__ double2 cmulc(double2 a, double2 b) {  // a * conj(b)
    return make_double2(a.x * b.x + a.y * b.y, a.y * b.x - a.x * b.y);
}
__device__ __forceinline__ double2 conjd(double2 a) { return make_double2(a.x, -a.y); }
__device__ __forceinline__ double2 mul_i(double2 a) { return make_double2(-a.y, a.x); }   // i a
__device__ __forceinline__ double2 mul_mi(double2 a) { return make_double2(a.y, -a.x); }  // -i a
__device__ __forceinline__ double2 scaled(double2 a, double s) { return make_double2(a.x * s, a.y * s); }

// W_N^x = exp(-2 pi i x / N) for N = 2^e, 0 <= x < N.
__device__ __forceinline__ double2 tw_at(const double2 *__restrict__ tw, int x, int e) {
    return tw[x << (TW_LOG - e)];
}

// Twiddles from the global table.
struct TwGlobal {
    const double2 *__restrict__ tw;
    __device__ __forceinline__ double2 operator()(int x, int e) const { return tw_at(tw, x, e); }
};

// Twiddles from a quarter table in LDS: q[r] = W_NT^r for r < NT/4 (NT =
// 2^eNT), and W_NT^(r + m NT/4) = (-i)^m W_NT^r.
struct TwLds {
    const double2 *q;
    int eNT;
    __device__ __forceinline__ double2 operator()(int x, int e) const {
        const int y = x << (eNT - e);
        const int m = y >> (eNT - 2), r = y & ((1 << (eNT - 2)) - 1);
        const double2 w = q[r];
        // (-i)^m w: m = 1 -> (w.y, -w.x), 2 -> -w, 3 -> (-w.y, w.x)
        const double re = (m & 1) ? w.y : w.x, im = (m & 1) ? w.x : w.y;
        const double sr = (m < 2) ? 1.0 : -1.0, si = (m == 0 || m == 3) ? 1.0 : -1.0;
        return make_double2(sr * re, si * im);
    }
};

// Fills q[r] = W_NT^r, r < NT/4, from the global table.
__device__ __forceinline__ void load_quarter(double2 *q, int eNT, const double2 *__restrict__ tw) {
    for (int r = threadIdx.x; r < (1 << (eNT - 2)); r += blockDim.x) q[r] = tw_at(tw, r, eNT);
}

// Position of frequency k after a length-2^e decimation-in-frequency
// transform: its mixed-radix digits (a radix-2 digit first when e is odd,
// then base-4 digits), lowest first, read back highest first.
__device__ __forceinline__ int fft_pos(int k, int e) {
    int n = 1 << e, p = 0;
    if (e & 1) {
        n >>= 1;
        p = (k & 1) * n;
        k >>= 1;
    }
    while (n > 1) {
        n >>= 2;
        p += (k & 3) * n;
        k >>= 2;
    }
    return p;
}

// The frequency stored at position p (the inverse of fft_pos).
__device__ __forceinline__ int fft_freq(int p, int e) {
    const bool odd = e & 1;
    int h = 0;
    if (odd) {
        h = p >> (e - 1);
        p &= (1 << (e - 1)) - 1;
        e -= 1;
    }
    int k = 0;
    for (int d = 0; d < e; d += 2) {  // reverse the base-4 digits of p
        k = (k << 2) | (p & 3);
        p >>= 2;
    }
    return odd ? ((k << 1) | h) : k;
}

// In-place forward DFT (unnormalised, kernel exp(-2 pi i nk / N)) of B
// sequences of length N = 2^e held in LDS as buf[n * B + b]: decimation in
// frequency, a radix-2 stage first when e is odd, then radix-4 stages; the
// output of frequency k sits at position fft_pos(k, e).  Ends with a barrier.
template <class TW>
__device__ void lds_dif(double2 *buf, int e, int B, const TW tw) {
    const int N = 1 << e;
    int L = N, eL = e;
    if (e & 1) {
        const int s = N >> 1;
        for (int idx = threadIdx.x; idx < s * B; idx += blockDim.x) {
            const int j = idx / B, b = idx - j * B;
            const double2 a0 = buf[j * B + b], a1 = buf[(j + s) * B + b];
            buf[j * B + b] = cadd(a0, a1);
            buf[(j + s) * B + b] = cmul(csub(a0, a1), tw(j, e));
        }
        __syncthreads();
        L = s;
        eL = e - 1;
    }
    for (; L >= 4; L >>= 2, eL -= 2) {
        const int s = L >> 2;
        for (int idx = threadIdx.x; idx < (N >> 2) * B; idx += blockDim.x) {
            const int bf = idx / B, b = idx - bf * B;
            const int g = bf / s, j = bf - g * s;
            const int i0 = (g * L + j) * B + b;
            const double2 a0 = buf[i0], a1 = buf[i0 + s * B], a2 = buf[i0 + 2 * s * B],
                          a3 = buf[i0 + 3 * s * B];
            const double2 t0 = cadd(a0, a2), t1 = csub(a0, a2), t2 = cadd(a1, a3),
                          t3 = mul_mi(csub(a1, a3));
            buf[i0] = cadd(t0, t2);
            buf[i0 + s * B] = cmul(cadd(t1, t3), tw(j, eL));
            buf[i0 + 2 * s * B] = cmul(csub(t0, t2), tw(2 * j, eL));
            buf[i0 + 3 * s * B] = cmul(csub(t1, t3), tw(3 * j, eL));
        }
        __syncthreads();
    }
}

// The exact reverse of lds_dif with conjugate twiddles: input at positions
// fft_pos(k, e), output in natural order, N times the inverse DFT.  Ends
// with a barrier.
template <class TW>
__device__ void lds_dit_inv(double2 *buf, int e, int B, const TW tw) {
    const int N = 1 << e;
    const int eTop = (e & 1) ? e - 1 : e;
    for (int eL = 2; eL <= eTop; eL += 2) {
        const int L = 1 << eL, s = L >> 2;
        for (int idx = threadIdx.x; idx < (N >> 2) * B; idx += blockDim.x) {
            const int bf = idx / B, b = idx - bf * B;
            const int g = bf / s, j = bf - g * s;
            const int i0 = (g * L + j) * B + b;
            const double2 x0 = buf[i0];
            const double2 x1 = cmulc(buf[i0 + s * B], tw(j, eL));
            const double2 x2 = cmulc(buf[i0 + 2 * s * B], tw(2 * j, eL));
            const double2 x3 = cmulc(buf[i0 + 3 * s * B], tw(3 * j, eL));
            const double2 t0 = cadd(x0, x2), t1 = csub(x0, x2), t2 = cadd(x1, x3),
                          t3 = mul_i(csub(x1, x3));
            buf[i0] = cadd(t0, t2);
            buf[i0 + s * B] = cadd(t1, t3);
            buf[i0 + 2 * s * B] = csub(t0, t2);
            buf[i0 + 3 * s * B] = csub(t1, t3);
        }
        __syncthreads();
    }
    if (e & 1) {
        const int s = N >> 1;
        for (int idx = threadIdx.x; idx < s * B; idx += blockDim.x) {
            const int j = idx / B, b = idx - j * B;
            const double2 y = buf[j * B + b];
            const double2 z = cmulc(buf[(j + s) * B + b], tw(j, e));
            buf[j * B + b] = cadd(y, z);
            buf[(j + s) * B + b] = csub(y, z);
        }
        __syncthreads();
    }
}

__global__ __launch_bounds__(FFT_T) void fft_twiddles(double2 *__restrict__ tw) {
    const int k = blockIdx.x * FFT_T + threadIdx.x;
    if (k < TWN) {
        double s, c;
        sincospi(2.0 * (double)k / (double)TWN, &s, &c);
        tw[k] = make_double2(c, -s);
    }
}

// Rows 0 .. rows-1 of the half spectrum of a real u8 plane (src rows of srcW
// bytes srcPitch apart, zero beyond srcW and below srcRows): row r's real DFT
// of length Qn = 2M, columns 0 .. M, zeros in columns M+1 .. pitch-1.
__global__ __launch_bounds__(ROW_T) void fft_rows_r2c(const uint8_t *__restrict__ src, int srcW,
                                                      int srcRows, size_t srcPitch, int eM,
                                                      double2 *__restrict__ spec, int pitch,
                                                      const double2 *__restrict__ tw) {
    extern __shared__ double2 z[];  // [M] samples, then the quarter table of W_2M
    const int M = 1 << eM, r = blockIdx.x;
    const TwLds tq{z + M, eM + 1};
    load_quarter(z + M, eM + 1, tw);
    const uint8_t *row = src + (size_t)r * srcPitch;
    for (int n = threadIdx.x; n < M; n += ROW_T) {
        const int x = 2 * n;
        const double v0 = (r < srcRows && x < srcW) ? (double)row[x] : 0.0;
        const double v1 = (r < srcRows && x + 1 < srcW) ? (double)row[x + 1] : 0.0;
        z[n] = make_double2(v0, v1);
    }
    __syncthreads();
    lds_dif(z, eM, 1, tq);
    // X[k] = E[k] + W_Qn^k O[k]: E = (Z[k] + conj Z[M-k]) / 2 the even
    // samples' DFT, O = -i (Z[k] - conj Z[M-k]) / 2 the odd samples'
    double2 *out = spec + (size_t)r * pitch;
    for (int k = threadIdx.x; k < pitch; k += ROW_T) {
        if (k > M) {
            out[k] = make_double2(0.0, 0.0);
            continue;
        }
        const double2 zk = z[fft_pos(k & (M - 1), eM)];
        const double2 zm = conjd(z[fft_pos((M - k) & (M - 1), eM)]);
        const double2 E = scaled(cadd(zk, zm), 0.5);
        const double2 O = scaled(mul_mi(csub(zk, zm)), 0.5);
        out[k] = cadd(E, cmul(tq(k, eM + 1), O));
    }
}

// Column pass 1: for column tile blockIdx.x (FFT_TB columns) and n2 =
// blockIdx.y, the length-P1 transform over rows n1 * P2 + n2, with the
// four-step twiddle W_P^(n2 k1).  Forward: transform, then twiddle (rows at
// or below nzRows hold zeros and are not read).  Inverse: conjugate twiddle,
// then inverse transform; only rows below outRows are written.
template <bool INV>
__global__ __launch_bounds__(FFT_T) void fft_cols_pass1(double2 *__restrict__ spec, int pitch,
                                                        int eP1, int eP2, int nzRows, int outRows,
                                                        const double2 *__restrict__ tw) {
    extern __shared__ double2 buf[];
    const int P1 = 1 << eP1, P2 = 1 << eP2, eP = eP1 + eP2;
    const int c0 = blockIdx.x * FFT_TB, n2 = blockIdx.y;
    for (int idx = threadIdx.x; idx < P1 * FFT_TB; idx += FFT_T) {
        const int p = idx / FFT_TB, c = idx - p * FFT_TB;
        const int row = p * P2 + n2;
        double2 v = make_double2(0.0, 0.0);
        if (INV || row < nzRows) v = spec[(size_t)row * pitch + c0 + c];
        if (INV) v = cmulc(v, tw_at(tw, (n2 * fft_freq(p, eP1)) & ((1 << eP) - 1), eP));
        buf[idx] = v;
    }
    __syncthreads();
    if (INV)
        lds_dit_inv(buf, eP1, FFT_TB, TwGlobal{tw});
    else
        lds_dif(buf, eP1, FFT_TB, TwGlobal{tw});
    for (int idx = threadIdx.x; idx < P1 * FFT_TB; idx += FFT_T) {
        const int p = idx / FFT_TB, c = idx - p * FFT_TB;
        const int row = p * P2 + n2;
        double2 v = buf[idx];
        if (!INV) v = cmul(v, tw_at(tw, (n2 * fft_freq(p, eP1)) & ((1 << eP) - 1), eP));
        if (!INV || row < outRows) spec[(size_t)row * pitch + c0 + c] = v;
    }
}

// Column pass 2: for column tile blockIdx.x and the block of rows
// blockIdx.y * P2 .. + P2 - 1, the length-P2 transform.  CORR: multiply by
// the conjugate of tspec (the template's spectrum, stored by this same pass)
// and transform back, writing dst; else write the forward transform to dst.
template <bool CORR>
__global__ __launch_bounds__(FFT_T) void fft_cols_pass2(const double2 *__restrict__ src,
                                                        const double2 *__restrict__ tspec,
                                                        double2 *__restrict__ dst, int pitch,
                                                        int eP2, const double2 *__restrict__ tw) {
    extern __shared__ double2 buf[];
    const int P2 = 1 << eP2;
    const int c0 = blockIdx.x * FFT_TB;
    const size_t r0 = (size_t)blockIdx.y * P2;
    for (int idx = threadIdx.x; idx < P2 * FFT_TB; idx += FFT_T) {
        const int q = idx / FFT_TB, c = idx - q * FFT_TB;
        buf[idx] = src[(r0 + q) * pitch + c0 + c];
    }
    __syncthreads();
    lds_dif(buf, eP2, FFT_TB, TwGlobal{tw});
    if (CORR) {
        for (int idx = threadIdx.x; idx < P2 * FFT_TB; idx += FFT_T) {
            const int q = idx / FFT_TB, c = idx - q * FFT_TB;
            buf[idx] = cmulc(buf[idx], tspec[(r0 + q) * pitch + c0 + c]);
        }
        __syncthreads();
        lds_dit_inv(buf, eP2, FFT_TB, TwGlobal{tw});
    }
    for (int idx = threadIdx.x; idx < P2 * FFT_TB; idx += FFT_T) {
        const int q = idx / FFT_TB, c = idx - q * FFT_TB;
        dst[(r0 + q) * pitch + c0 + c] = buf[idx];
    }
}

// Output row y = blockIdx.x: the inverse real transform of spectrum row y
// (E = (X[k] + conj X[M-k]) / 2, O = W_Qn^-k (X[k] - conj X[M-k]) / 2,
// Z = E + i O, z = M x IDFT(Z)), SumIT = round(scale * sample), then SumI and
// SumISq by the four-corner rule on the tables and the coefficient, as the
// generic route does.  The four corners are taken as differences of two
// table rows staged once in LDS: cS[x + 1] = S(x, y+hT-1) - S(x, y-1) for
// view columns x = -1 .. W-1 (mod 2^32; every window sum is below 2^32, so
// its difference of two cS is exact; column -1 and row -1 are table elements
// when the view starts inside the table, zero at its edges).  cS and cQ reuse
// the LDS of the samples and the twiddle quarter table (8 (W + 1) <= 24 M
// bytes) once each lane holds its SumIT values (at most ROW_MAXX of them:
// Wo <= 8192).
__global__ __launch_bounds__(ROW_T) void fft_rows_c2r_coef(const double2 *__restrict__ spec,
                                                           int pitch, int eM, double scale,
                                                           CorrArgs a, int t, Tables tb,
                                                           const double2 *__restrict__ tw) {
    extern __shared__ double2 z[];  // [M] samples (later cS, cQ [W] each), [M/2] quarter table
    const int M = 1 << eM, y = blockIdx.x;
    const TwLds tq{z + M, eM + 1};
    load_quarter(z + M, eM + 1, tw);
    __syncthreads();  // the quarter table is read below
    const double2 *in = spec + (size_t)y * pitch;
    for (int k = threadIdx.x; k < M; k += ROW_T) {
        const double2 xk = in[k], xm = conjd(in[M - k]);
        const double2 E = scaled(cadd(xk, xm), 0.5);
        const double2 O = scaled(cmulc(csub(xk, xm), tq(k, eM + 1)), 0.5);
        z[fft_pos(k, eM)] = cadd(E, mul_i(O));
    }
    __syncthreads();
    lds_dit_inv(z, eM, 1, tq);
    long long sit[ROW_MAXX];
#pragma unroll
    for (int i = 0; i < ROW_MAXX; i++) {
        const int x = threadIdx.x + i * ROW_T;
        const double2 zz = z[(x < a.Wo ? x : 0) >> 1];
        sit[i] = __double2ll_rn(((x & 1) ? zz.y : zz.x) * scale);
    }
    __syncthreads();  // the samples and the quarter table are read; their LDS takes cS, cQ
    uint32_t *cS = (uint32_t *)z, *cQ = cS + a.W + 1;
    {
        const ptrdiff_t pt = (ptrdiff_t)tb.pitch;
        const int64_t *sb = tb.S + (ptrdiff_t)(y + a.hT - 1) * pt, *qb = tb.Q + (ptrdiff_t)(y + a.hT - 1) * pt;
        const bool above = tb.ty + y > 0;  // the row above the windows is a table row
        const int64_t *st = tb.S + (above ? (ptrdiff_t)(y - 1) * pt : 0);
        const int64_t *qt = tb.Q + (above ? (ptrdiff_t)(y - 1) * pt : 0);
        for (int i = threadIdx.x; i <= a.W; i += ROW_T) {
            const int x = i - 1;
            uint32_t vs = 0, vq = 0;
            if (tb.tx + x >= 0) {
                vs = (uint32_t)(sb[x] - (above ? st[x] : 0));
                vq = (uint32_t)(qb[x] - (above ? qt[x] : 0));
            }
            cS[i] = vs;
            cQ[i] = vq;
        }
    }
    __syncthreads();
    const TStat ts = a.stats[t];
    const long long K = (long long)a.wT * a.hT;
    const size_t o_row = (size_t)y * a.op;
#pragma unroll
    for (int i = 0; i < ROW_MAXX; i++) {
        const int x = threadIdx.x + i * ROW_T;
        if (x >= a.Wo) break;
        const long long sumIT = sit[i];
        const long long sumI = (long long)(cS[x + a.wT] - cS[x]);
        const long long sumISq = (long long)(cQ[x + a.wT] - cQ[x]);
        const long long num = K * sumIT - sumI * ts.sumT;
        const long long varI = K * sumISq - sumI * sumI;
        const size_t o = o_row + x;
        __builtin_nontemporal_store(ncc_coef((float)num, (float)varI, ts.varTf),
                                    a.coef + (size_t)t * a.oplane + o);
        if (a.sums) {
            if (t == 0) {
                __builtin_nontemporal_store((int32_t)sumI, a.sums + o);
                __builtin_nontemporal_store((int32_t)sumISq, a.sums + a.oplane + o);
            }
            __builtin_nontemporal_store((int32_t)sumIT, a.sums + (size_t)(2 + t) * a.oplane + o);
        }
    }
}

int ilog2_ceil(int n) {
    int e = 0;
    while ((1 << e) < n) e++;
    return e;
}

struct FftGeom {
    int eQ, eM, eP, eP1, eP2, pitch, tiles;
};

bool fft_geometry(int W, int H, FftGeom *g) {
    g->eQ = ilog2_ceil(W < 8 ? 8 : W);
    g->eP = ilog2_ceil(H < 4 ? 4 : H);
    if (g->eQ > FFT_MAX_LOG || g->eP > FFT_MAX_LOG) return false;
    g->eM = g->eQ - 1;
    g->eP1 = (g->eP + 1) / 2;
    g->eP2 = g->eP / 2;
    const int cols = (1 << g->eM) + 1;
    g->tiles = (cols + FFT_TB - 1) / FFT_TB;
    g->pitch = g->tiles * FFT_TB;
    return true;
}

hipError_t set_lds(const void *fn, size_t bytes) {
    return hipFuncSetAttribute(fn, hipFuncAttributeMaxDynamicSharedMemorySize, (int)bytes);
}

}  // namespace

bool corr_fft_supported(int W, int H) {
    FftGeom g;
    return fft_geometry(W, H, &g);
}

size_t corr_fft_bytes(int W, int H) {
    FftGeom g;
    if (!fft_geometry(W, H, &g)) return 0;
    const size_t spec = ((size_t)g.pitch << g.eP) * sizeof(double2);
    return 3 * spec + (size_t)TWN * sizeof(double2) + 3 * 256;
}

hipError_t corr_fft_launch(const CorrArgs &a, const Tables &tb, void *work, hipStream_t st) {
    FftGeom g;
    if (!fft_geometry(a.W, a.H, &g)) return hipErrorNotSupported;
    static bool attr_set[NCC_MAX_DEVICES] = {};
    hipError_t ea = set_once(attr_set, [] {
        const size_t mx = 160 * 1024;
        hipError_t e;
        if ((e = set_lds((const void *)fft_rows_r2c, mx)) != hipSuccess) return e;
        if ((e = set_lds((const void *)fft_rows_c2r_coef, mx)) != hipSuccess) return e;
        if ((e = set_lds((const void *)fft_cols_pass1<false>, mx)) != hipSuccess) return e;
        if ((e = set_lds((const void *)fft_cols_pass1<true>, mx)) != hipSuccess) return e;
        if ((e = set_lds((const void *)fft_cols_pass2<false>, mx)) != hipSuccess) return e;
        return set_lds((const void *)fft_cols_pass2<true>, mx);
    });
    if (ea != hipSuccess) return ea;
    const size_t spec = ((size_t)g.pitch << g.eP) * sizeof(double2);
    char *base = (char *)work;
    double2 *ispec = (double2 *)base;
    double2 *tspec = (double2 *)(base + spec);
    double2 *wspec = (double2 *)(base + 2 * spec);
    double2 *tw = (double2 *)(base + 3 * spec);
    const int M = 1 << g.eM, P = 1 << g.eP, P1 = 1 << g.eP1, P2 = 1 << g.eP2;
    const size_t rowLds = (size_t)(M + M / 2) * sizeof(double2);
    const size_t c2rLds = rowLds;  // cS, cQ (8 (W + 1) <= 24 M bytes) reuse it
    const size_t c1Lds = (size_t)P1 * FFT_TB * sizeof(double2);
    const size_t c2Lds = (size_t)P2 * FFT_TB * sizeof(double2);
    const dim3 blk(FFT_T);

    hipLaunchKernelGGL(fft_twiddles, dim3(TWN / FFT_T), blk, 0, st, tw);
    // the image's spectrum: rows of the view, then both column passes
    hipLaunchKernelGGL(fft_rows_r2c, dim3(a.H), dim3(ROW_T), rowLds, st, a.img, a.W, a.H, a.ip, g.eM, ispec,
                       g.pitch, (const double2 *)tw);
    hipLaunchKernelGGL(fft_cols_pass1<false>, dim3(g.tiles, P2), blk, c1Lds, st, ispec, g.pitch,
                       g.eP1, g.eP2, a.H, P, (const double2 *)tw);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
    const double scale = 1.0 / ((double)M * (double)P);
    for (int t = 0; t < a.nTpl; t++) {
        const uint8_t *T = a.tpl + (size_t)t * a.hT * a.wT;
        hipLaunchKernelGGL(fft_rows_r2c, dim3(a.hT), dim3(ROW_T), rowLds, st, T, a.wT, a.hT, (size_t)a.wT,
                           g.eM, tspec, g.pitch, (const double2 *)tw);
        hipLaunchKernelGGL(fft_cols_pass1<false>, dim3(g.tiles, P2), blk, c1Lds, st, tspec, g.pitch,
                           g.eP1, g.eP2, a.hT, P, (const double2 *)tw);
        hipLaunchKernelGGL(fft_cols_pass2<false>, dim3(g.tiles, P1), blk, c2Lds, st,
                           (const double2 *)tspec, (const double2 *)nullptr, tspec, g.pitch, g.eP2,
                           (const double2 *)tw);
        // the image's second column pass, the product and its inverse in one
        hipLaunchKernelGGL(fft_cols_pass2<true>, dim3(g.tiles, P1), blk, c2Lds, st,
                           (const double2 *)ispec, (const double2 *)tspec, wspec, g.pitch, g.eP2,
                           (const double2 *)tw);
        hipLaunchKernelGGL(fft_cols_pass1<true>, dim3(g.tiles, P2), blk, c1Lds, st, wspec, g.pitch,
                           g.eP1, g.eP2, P, a.Ho, (const double2 *)tw);
        hipLaunchKernelGGL(fft_rows_c2r_coef, dim3(a.Ho), dim3(ROW_T), c2rLds, st, (const double2 *)wspec,
                           g.pitch, g.eM, scale, a, t, tb, (const double2 *)tw);
        e = hipGetLastError();
        if (e != hipSuccess) return e;
    }
    return hipSuccess;
}

}  // namespace ncc
