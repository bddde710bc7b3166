// Single-template normalized cross-correlation on the vector units.
//
// What is computed follows The CUDA Handbook ch. 15 "Image in shared
// memory" (corrShared_kernel: for each window, SumI, SumISq and SumIT over a
// wT x hT template, from an image tile plus a (wT-1) x (hT-1) halo staged in
// on-chip memory, then the coefficient) and section 15.8 (SumI and SumISq
// from summed-area tables by the four-corner rule).
//
// corr_stream (specialised template sizes): a workgroup owns 64*WAVES
// adjacent output columns and RS output rows.  Each lane owns one output
// column and streams down the image rows; rows are staged through a
// double-buffered LDS ring of HT rows.  For every image row a lane:
//   - reads WT4+1 aligned dwords of its window from LDS and byte-aligns them
//     (v_alignbyte_b32) to its window start;
//   - forms the row's window sums of I and I^2 (v_dot4_u32_u8 against ones /
//     against itself) and adds them to running column sums: these are the
//     differences S(x+wT-1, y) - S(x-1, y) of the strip's summed-area table,
//     so SumI of an output row is the difference of two of them (the
//     four-corner rule with its horizontal difference taken first);
//   - adds the row's products with template row j into the SumIT
//     accumulator of output row y-j (v_dot4_u32_u8, template in SGPRs),
//     for all HT template rows: a ring of HT accumulators;
//   - finishes the output row whose window ends at this image row.
// The template's last partial dword is zero-padded, so SumIT needs no mask.
//
// corr_generic (any shape): 64 x 64 output tile per workgroup, 4 x 4 outputs
// per lane, dot4 over an LDS-staged tile + halo; SumI and SumISq by satBox on
// the full int64 tables.
#include "ncc_internal.h"

namespace ncc {

namespace {

// ------------------------------------------------------ staging helpers --
// Loads bytes [x, x+16) of row y as 4 dwords; bytes outside the image are 0.
template <int ALIGN>
__device__ __forceinline__ uint4 load16(const uint8_t *img, int W, int H, int x, int y) {
    uint4 v = make_uint4(0, 0, 0, 0);
    if (y >= H || x >= W) return v;
    const uint8_t *row = img + (size_t)y * W;
    if (ALIGN == 16 && x + 15 < W) return *(const uint4 *)(row + x);
    if (ALIGN >= 4 && x + 15 < W) {
        const uint32_t *p = (const uint32_t *)(row + x);
        return make_uint4(p[0], p[1], p[2], p[3]);
    }
    uint32_t w[4] = {0, 0, 0, 0};
#pragma unroll
    for (int b = 0; b < 16; b++)
        if (x + b < W) w[b >> 2] |= (uint32_t)row[x + b] << (8 * (b & 3));
    return make_uint4(w[0], w[1], w[2], w[3]);
}

__device__ __forceinline__ void store_coef(float *p, float v) {
    __builtin_nontemporal_store(v, p);
}
__device__ __forceinline__ void store_sum(int32_t *p, int32_t v) {
    __builtin_nontemporal_store(v, p);
}

// ------------------------------------------------------------- streaming --
template <int WT4, int HT, int WAVES, int RS, int ALIGN>
__global__ __launch_bounds__(WAVES * 64) void corr_stream(CorrArgs a, int t) {
    constexpr int NT = WAVES * 64;                     // output columns per workgroup
    constexpr int SEGB = NT + 4 * WT4 + 4;             // staged bytes per row
    constexpr int CH = (SEGB + 15) / 16;               // 16-byte chunks per row
    constexpr int PITCH = CH * 4 + 4;                  // dwords per LDS row
    constexpr int LOADS = (HT * CH + NT - 1) / NT;     // chunk loads per thread per batch
    __shared__ uint32_t buf[2][HT][PITCH];

    const int tid = threadIdx.x;
    const int x0 = blockIdx.x * NT, y0 = blockIdx.y * RS;
    const int x = x0 + tid;
    const int db = tid >> 2;
    const uint32_t sh = (uint32_t)(tid & 3);
    const int rowsOut = min(RS, a.Ho - y0);
    const int rowsIn = rowsOut + HT - 1;
    const int nb = (rowsIn + HT - 1) / HT;

    // template rows (wave-uniform), each zero-padded to WT4 dwords, and the
    // template constants SumT, SumTSq, varT computed from them
    const int wT = a.wT;
    const uint32_t mlast = byte_mask(wT - 4 * (WT4 - 1));
    const uint8_t *T = a.tpl + (size_t)t * HT * wT;
    uint32_t tp[HT][WT4];
    if (wT == 4 * WT4 && (((uintptr_t)T & 3) == 0)) {
#pragma unroll
        for (int j = 0; j < HT; j++)
#pragma unroll
            for (int k = 0; k < WT4; k++) tp[j][k] = ((const uint32_t *)(T + j * wT))[k];
    } else {
#pragma unroll
        for (int j = 0; j < HT; j++)
#pragma unroll
            for (int k = 0; k < WT4; k++) {
                uint32_t v = 0;
#pragma unroll
                for (int b = 0; b < 4; b++)
                    if (4 * k + b < wT) v |= (uint32_t)T[j * wT + 4 * k + b] << (8 * b);
                tp[j][k] = v;
            }
    }
    uint32_t sumT = 0, sumTSq = 0;
#pragma unroll
    for (int j = 0; j < HT; j++)
#pragma unroll
        for (int k = 0; k < WT4; k++) {
            sumT = dot4u(tp[j][k], 0x01010101u, sumT);
            sumTSq = dot4u(tp[j][k], tp[j][k], sumTSq);
        }
    const uint32_t K = (uint32_t)(wT * HT);
    // varT <= K^2 * 127.5^2 < 2^32 for K <= 514
    const float varTf = (float)(K * sumTSq - sumT * sumT);

    // staging: chunk i of the batch -> row i / CH, bytes 16 * (i % CH)
    uint4 pre[LOADS];
    auto fetch = [&](int bt) {
#pragma unroll
        for (int u = 0; u < LOADS; u++) {
            const int i = tid + u * NT;
            const int r = i / CH, c = i % CH;
            pre[u] = (i < HT * CH) ? load16<ALIGN>(a.img, a.W, a.H, x0 + 16 * c, y0 + bt * HT + r)
                                   : make_uint4(0, 0, 0, 0);
        }
    };
    auto put = [&](int bt) {
#pragma unroll
        for (int u = 0; u < LOADS; u++) {
            const int i = tid + u * NT;
            if (i < HT * CH) {
                const int r = i / CH, c = i % CH;
                *(uint4 *)&buf[bt & 1][r][4 * c] = pre[u];
            }
        }
    };

    uint32_t acc[HT], pI[HT], pQ[HT];
#pragma unroll
    for (int i = 0; i < HT; i++) acc[i] = pI[i] = pQ[i] = 0;
    uint32_t PI = 0, PQ = 0;

    fetch(0);
    put(0);
    __syncthreads();
    for (int bt = 0; bt < nb; bt++) {
        if (bt + 1 < nb) fetch(bt + 1);
#pragma unroll
        for (int q = 0; q < HT; q++) {
            const uint32_t *rowp = &buf[bt & 1][q][db];
            uint32_t d[WT4 + 1];
#pragma unroll
            for (int k = 0; k <= WT4; k++) d[k] = rowp[k];
            uint32_t v[WT4];
#pragma unroll
            for (int k = 0; k < WT4; k++) v[k] = align_bytes(d[k + 1], d[k], sh);
            // window row sums of I and I^2
            uint32_t hs = 0, hs2 = 0;
#pragma unroll
            for (int k = 0; k < WT4; k++) {
                const uint32_t m = (k == WT4 - 1) ? mlast : 0xffffffffu;
                hs = dot4u(v[k], 0x01010101u & m, hs);
                hs2 = dot4u(v[k], v[k] & m, hs2);
            }
            PI += hs;
            PQ += hs2;
            // products with every template row
#pragma unroll
            for (int j = 0; j < HT; j++) {
                const int slot = (q - j + HT) % HT;
                uint32_t s = acc[slot];
#pragma unroll
                for (int k = 0; k < WT4; k++) s = dot4u(v[k], tp[j][k], s);
                acc[slot] = s;
            }
            // output row whose window ends at this image row
            const int fin = (q + 1) % HT;
            const uint32_t sumIT = acc[fin];
            acc[fin] = 0;
            const uint32_t sumI = PI - pI[q];
            const uint32_t sumISq = PQ - pQ[q];
            pI[q] = PI;
            pQ[q] = PQ;
            const int rho = bt * HT + q;  // image row relative to y0
            const int yo = y0 + rho - (HT - 1);
            if (rho >= HT - 1 && rho - (HT - 1) < rowsOut && x < a.Wo) {
                float g;
                if (HT * 4 * WT4 <= 363) {
                    // |num| <= K^2 * 127.5^2 < 2^31 and varI < 2^32: exact mod 2^32
                    const int32_t num = (int32_t)(K * sumIT - sumI * sumT);
                    const uint32_t varI = K * sumISq - sumI * sumI;
                    g = ncc_coef((float)num, (float)varI, varTf);
                } else {
                    const long long num = (long long)K * sumIT - (long long)sumI * (long long)sumT;
                    const long long varI = (long long)K * sumISq - (long long)sumI * (long long)sumI;
                    g = ncc_coef((float)num, (float)varI, varTf);
                }
                const size_t plane = (size_t)a.Ho * a.Wo;
                const size_t o = (size_t)yo * a.Wo + x;
                store_coef(a.coef + (size_t)t * plane + o, g);
                if (a.sums) {
                    if (t == 0) {
                        store_sum(a.sums + o, (int32_t)sumI);
                        store_sum(a.sums + plane + o, (int32_t)sumISq);
                    }
                    store_sum(a.sums + (size_t)(2 + t) * plane + o, (int32_t)sumIT);
                }
            }
        }
        if (bt + 1 < nb) put(bt + 1);
        __syncthreads();
    }
}

// --------------------------------------------------------------- generic --
constexpr int GT = 64;  // output tile edge

__device__ __forceinline__ long long sat_box(const int64_t *S, int W, int x0, int y0, int x1,
                                             int y1) {
    // 0 <= x0 < x1 <= W, 0 <= y0 < y1 <= H guaranteed by the caller
    const int64_t *rb = S + (size_t)(y1 - 1) * W;
    long long D = rb[x1 - 1];
    long long C = x0 > 0 ? rb[x0 - 1] : 0;
    long long B = 0, A = 0;
    if (y0 > 0) {
        const int64_t *rt = S + (size_t)(y0 - 1) * W;
        B = rt[x1 - 1];
        A = x0 > 0 ? rt[x0 - 1] : 0;
    }
    return D - B - C + A;
}

__global__ __launch_bounds__(256) void corr_generic(CorrArgs a, int t, const int64_t *__restrict__ S,
                                                    const int64_t *__restrict__ Q, int pitch,
                                                    int rowsT) {
    extern __shared__ uint32_t tile[];  // rowsT x pitch bytes
    const int tid = threadIdx.x;
    const int x0 = blockIdx.x * GT, y0 = blockIdx.y * GT;
    const int wt4 = (a.wT + 3) / 4;
    const int pw = pitch / 4;

    // stage the tile + halo
    for (int i = tid; i < rowsT * pw; i += 256) {
        const int r = i / pw, c = i % pw;
        const int y = y0 + r, xb = x0 + 4 * c;
        uint32_t v = 0;
        if (y < a.H) {
            const uint8_t *row = a.img + (size_t)y * a.W;
#pragma unroll
            for (int b = 0; b < 4; b++)
                if (xb + b < a.W) v |= (uint32_t)row[xb + b] << (8 * b);
        }
        tile[i] = v;
    }
    __syncthreads();

    const int tx = tid & 15, ty = tid >> 4;
    uint32_t acc[4][4];
#pragma unroll
    for (int dy = 0; dy < 4; dy++)
#pragma unroll
        for (int s = 0; s < 4; s++) acc[dy][s] = 0;
    const uint32_t *trow = a.rows + (size_t)t * a.hT * wt4;

    for (int r = 0; r < a.hT + 3; r++) {
        const uint32_t *rowp = tile + (4 * ty + r) * pw + tx;
        uint32_t lo = rowp[0];
        for (int k = 0; k < wt4; k++) {
            const uint32_t hi = rowp[k + 1];
            const uint32_t v0 = lo, v1 = align_bytes(hi, lo, 1), v2 = align_bytes(hi, lo, 2),
                           v3 = align_bytes(hi, lo, 3);
#pragma unroll
            for (int dy = 0; dy < 4; dy++) {
                const int j = r - dy;
                if (j >= 0 && j < a.hT) {
                    const uint32_t tv = trow[j * wt4 + k];
                    acc[dy][0] = dot4u(v0, tv, acc[dy][0]);
                    acc[dy][1] = dot4u(v1, tv, acc[dy][1]);
                    acc[dy][2] = dot4u(v2, tv, acc[dy][2]);
                    acc[dy][3] = dot4u(v3, tv, acc[dy][3]);
                }
            }
            lo = hi;
        }
    }

    const TStat ts = a.stats[t];
    const long long K = (long long)a.wT * a.hT;
    const size_t plane = (size_t)a.Ho * a.Wo;
#pragma unroll
    for (int dy = 0; dy < 4; dy++) {
        const int y = y0 + 4 * ty + dy;
        if (y >= a.Ho) break;
#pragma unroll
        for (int s = 0; s < 4; s++) {
            const int x = x0 + 4 * tx + s;
            if (x >= a.Wo) break;
            const long long sumI = sat_box(S, a.W, x, y, x + a.wT, y + a.hT);
            const long long sumISq = sat_box(Q, a.W, x, y, x + a.wT, y + a.hT);
            const long long sumIT = acc[dy][s];
            const long long num = K * sumIT - sumI * ts.sumT;
            const long long varI = K * sumISq - sumI * sumI;
            const float g = ncc_coef((float)num, (float)varI, ts.varTf);
            const size_t o = (size_t)y * a.Wo + x;
            store_coef(a.coef + (size_t)t * plane + o, g);
            if (a.sums) {
                if (t == 0) {
                    store_sum(a.sums + o, (int32_t)sumI);
                    store_sum(a.sums + plane + o, (int32_t)sumISq);
                }
                store_sum(a.sums + (size_t)(2 + t) * plane + o, (int32_t)sumIT);
            }
        }
    }
}

constexpr int STREAM_WAVES = 4;
constexpr int STREAM_RS = 128;

template <int WT4, int HT>
hipError_t launch_stream(const CorrArgs &a, int t, hipStream_t st) {
    constexpr int NT = STREAM_WAVES * 64;
    dim3 grid((a.Wo + NT - 1) / NT, (a.Ho + STREAM_RS - 1) / STREAM_RS);
    if (a.W % 16 == 0 && ((uintptr_t)a.img & 15) == 0)
        hipLaunchKernelGGL((corr_stream<WT4, HT, STREAM_WAVES, STREAM_RS, 16>), grid, dim3(NT), 0,
                           st, a, t);
    else if (a.W % 4 == 0 && ((uintptr_t)a.img & 3) == 0)
        hipLaunchKernelGGL((corr_stream<WT4, HT, STREAM_WAVES, STREAM_RS, 4>), grid, dim3(NT), 0,
                           st, a, t);
    else
        hipLaunchKernelGGL((corr_stream<WT4, HT, STREAM_WAVES, STREAM_RS, 1>), grid, dim3(NT), 0,
                           st, a, t);
    return hipGetLastError();
}

void generic_geometry(int wT, int hT, int *pitch, int *rowsT) {
    const int wt4 = (wT + 3) / 4;
    *pitch = ((GT + 4 * wt4 + 4) + 15) / 16 * 16;
    *rowsT = GT + hT + 2;
}

}  // namespace

bool corr_stream_supported(int wT, int hT) {
    return hT == 16 && wT > 12 && wT <= 16;
}

hipError_t corr_stream_launch(const CorrArgs &a, int t, hipStream_t st) {
    if (a.hT == 16 && a.wT > 12 && a.wT <= 16) return launch_stream<4, 16>(a, t, st);
    return hipErrorNotSupported;
}

bool corr_generic_supported(int wT, int hT) {
    int pitch, rowsT;
    generic_geometry(wT, hT, &pitch, &rowsT);
    return (size_t)pitch * rowsT <= 160 * 1024;
}

hipError_t corr_generic_launch(const CorrArgs &a, int t, const int64_t *S, const int64_t *Q,
                               hipStream_t st) {
    int pitch, rowsT;
    generic_geometry(a.wT, a.hT, &pitch, &rowsT);
    size_t lds = (size_t)pitch * rowsT;
    if (lds > 160 * 1024) return hipErrorNotSupported;
    static bool attr_set = false;
    if (!attr_set) {
        hipError_t e = hipFuncSetAttribute((const void *)corr_generic,
                                           hipFuncAttributeMaxDynamicSharedMemorySize, 160 * 1024);
        if (e != hipSuccess) return e;
        attr_set = true;
    }
    dim3 grid((a.Wo + GT - 1) / GT, (a.Ho + GT - 1) / GT);
    hipLaunchKernelGGL(corr_generic, grid, dim3(256), lds, st, a, t, S, Q, pitch, rowsT);
    return hipGetLastError();
}

}  // namespace ncc
