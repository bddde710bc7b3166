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
// the full int64 tables.  A template whose tile + halo exceeds the LDS is
// taken in blocks of rows x dwords, each block staging its part of the image.
#include "ncc_internal.h"


namespace ncc {

namespace {

// ------------------------------------------------------ staging helpers --
// Loads bytes [x, x+16) of row y (at img + y * ip) as 4 dwords; bytes
// outside the image are 0.  ALIGN: the alignment of img and ip (and of x,
// a multiple of 16).
template <int ALIGN>
__device__ __forceinline__ uint4 load16(const uint8_t *img, size_t ip, int W, int H, int x, int y) {
    uint4 v = make_uint4(0, 0, 0, 0);
    if (y >= H || x >= W) return v;
    const uint8_t *row = img + (size_t)y * ip;
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
// Registers of one lane of the streaming kernel, which owns POS adjacent
// output columns.  MASK: the template's last dword is partial (wT < 4 WT4);
// WSUM: the window sums are written too.
template <int WT4_, int HT_, int POS_, bool MASK_, bool WSUM_>
struct StreamState {
    static constexpr int WT4 = WT4_, HT = HT_, POS = POS_;
    static constexpr bool MASK = MASK_, WSUM = WSUM_;
    uint32_t tp[HT][WT4];      // template rows (zero-padded dwords)
    uint32_t acc[POS][HT];     // SumIT rings: slot (row mod HT) of the output row
    uint32_t pI[POS][HT];      // running column sums of HT rows ago
    uint32_t pQ[POS][HT];
    uint32_t PI[POS], PQ[POS]; // running column sums of window row sums
    uint32_t sh[POS];          // byte offset of each window in the lane's first dword
    uint32_t mlast, K, sumT;
    float varTf;
    float *out;                // the strip's first output row (workgroup-uniform) ...
    int32_t *s0, *s1, *s2;     // ... and its sums planes
    uint32_t off;              // + this offset (elements): the lane's first column of the
                               //   next finished row
    bool wfirst;               // SumI / SumISq planes written by this call
    bool pairs;                // wave-uniform: every lane's POS columns are distinct
    int yrel;                  // output row (relative to the strip) finished next
};

// A wave-uniform value copied into a vector register: the template does not
// fit the scalar register file, and uses of a spilled scalar cost a
// v_readlane each.
__device__ __forceinline__ uint32_t to_vgpr(uint32_t x) {
    uint32_t r;
    __asm__("v_mov_b32 %0, %1" : "=v"(r) : "s"(x));
    return r;
}

typedef float f2u __attribute__((ext_vector_type(2), aligned(4)));
typedef int i2u __attribute__((ext_vector_type(2), aligned(4)));

// nI = -SumI (mod 2^32), as the running sums give it.
template <class ST>
__device__ __forceinline__ float stream_coef(const ST &st, uint32_t nI, uint32_t sumISq,
                                             uint32_t sumIT) {
    if (ST::HT * 4 * ST::WT4 <= 256) {
        // K*SumIT < 2^24 and SumISq < 2^24 (unsigned 24-bit products); SumI,
        // SumT < 2^16 (signed 24-bit); |num| <= K^2 * 127.5^2 < 2^31: exact mod 2^32
        const int32_t num = __mul24((int)st.sumT, (int)nI) + (int32_t)__umul24(st.K, sumIT);
        const uint32_t varI = __umul24(st.K, sumISq) - (uint32_t)__mul24((int)nI, (int)nI);
        return ncc_coef((float)num, (float)varI, st.varTf);
    } else {
        const long long sumI = -(long long)(int32_t)nI;
        const long long num = (long long)st.K * sumIT - sumI * st.sumT;
        const long long varI = (long long)st.K * sumISq - sumI * sumI;
        return ncc_coef((float)num, (float)varI, st.varTf);
    }
}

// One image row: window row sums, products with all template rows, and the
// output row whose window ends here.  PHASE 0: the strip's first HT image
// rows, where template rows j > Q land above the strip and are skipped;
// PHASE 2: the HT rows after the strip's last output row starts, where
// template rows j <= Q land below the strip and are skipped (the windows of
// the strip's last HT-1 output rows still end here); PHASE 1: all.  CHECK:
// the strip may end before this row's output (a strip cut by the image
// bottom); op: output row pitch in elements.
template <class ST, int Q, int PHASE, bool CHECK>
__device__ __forceinline__ void stream_row(ST &st, const uint32_t (&d)[ST::WT4 + 1], int rowsOut,
                                           uint32_t op) {
    constexpr int WT4 = ST::WT4, HT = ST::HT, POS = ST::POS;
    uint32_t v[POS][WT4];
#pragma unroll
    for (int p = 0; p < POS; p++)
#pragma unroll
        for (int k = 0; k < WT4; k++) v[p][k] = align_bytes(d[k + 1], d[k], st.sh[p]);
#pragma unroll
    for (int p = 0; p < POS; p++) {
        uint32_t hs = 0, hs2 = 0;
#pragma unroll
        for (int k = 0; k < WT4; k++) {
            const uint32_t vm = (ST::MASK && k == WT4 - 1) ? (v[p][k] & st.mlast) : v[p][k];
            hs = dot4u(vm, 0x01010101u, hs);
            hs2 = dot4u(vm, vm, hs2);
        }
        st.PI[p] += hs;
        st.PQ[p] += hs2;
    }
    // k outer, j inner: consecutive dot4s feed different accumulators
#pragma unroll
    for (int k = 0; k < WT4; k++)
#pragma unroll
        for (int j = 0; j < HT; j++) {
            if (PHASE == 0 && j > Q) continue;
            if (PHASE == 2 && j <= Q) continue;
            const int slot = (Q - j + HT) % HT;
#pragma unroll
            for (int p = 0; p < POS; p++)
                st.acc[p][slot] = dot4u(v[p][k], st.tp[j][k], st.acc[p][slot]);
        }
    // Empty asm statements that read and "write" every accumulator close the
    // row: without them the compiler defers each output's dot4s to where its
    // sum is consumed, which serialises them into one chain per output and
    // keeps 16 rows of image words live.
#pragma unroll
    for (int p = 0; p < POS; p++)
#pragma unroll
        for (int i = 0; i < HT; i++) __asm__ volatile("" : "+v"(st.acc[p][i]));
    // nor may later rows' loads and byte shifts be hoisted into this one
    __builtin_amdgcn_sched_barrier(0);
    constexpr int fin = (Q + 1) % HT;
    uint32_t sumIT[POS], nI[POS], sumISq[POS];
#pragma unroll
    for (int p = 0; p < POS; p++) {
        sumIT[p] = st.acc[p][fin];
        st.acc[p][fin] = 0;
        nI[p] = st.pI[p][Q] - st.PI[p];
        sumISq[p] = st.PQ[p] - st.pQ[p][Q];
        st.pI[p][Q] = st.PI[p];
        st.pQ[p][Q] = st.PQ[p];
    }
    if (PHASE == 0 && Q != HT - 1) return;  // no window ends here yet
    // every lane holds real columns (lanes past the last one repeat it), so
    // only the wave-uniform row test guards the stores
    if (!CHECK || st.yrel < rowsOut) {
        float g[POS];
#pragma unroll
        for (int p = 0; p < POS; p++) g[p] = stream_coef(st, nI[p], sumISq[p], sumIT[p]);
        if (POS == 2 && st.pairs) {
            __builtin_nontemporal_store((f2u){g[0], g[POS - 1]}, (f2u *)(st.out + st.off));
            if (ST::WSUM) {
                if (st.wfirst) {
                    __builtin_nontemporal_store((i2u){-(int)nI[0], -(int)nI[POS - 1]},
                                                (i2u *)(st.s0 + st.off));
                    __builtin_nontemporal_store((i2u){(int)sumISq[0], (int)sumISq[POS - 1]},
                                                (i2u *)(st.s1 + st.off));
                }
                __builtin_nontemporal_store((i2u){(int)sumIT[0], (int)sumIT[POS - 1]},
                                            (i2u *)(st.s2 + st.off));
            }
        } else {
            // edge lanes: column p of this lane is min(first + p, Wo - 1)
#pragma unroll
            for (int p = 0; p < POS; p++) {
                const uint32_t o = st.off + (st.sh[p] - st.sh[0]);
                store_coef(st.out + o, g[p]);
                if (ST::WSUM) {
                    if (st.wfirst) {
                        store_sum(st.s0 + o, -(int32_t)nI[p]);
                        store_sum(st.s1 + o, (int32_t)sumISq[p]);
                    }
                    store_sum(st.s2 + o, (int32_t)sumIT[p]);
                }
            }
        }
    }
    st.yrel++;
    st.off += op;
}

// Rows Q .. HT-1 of a batch; the LDS reads of row Q+1 are issued before row
// Q's arithmetic.
template <class ST, int Q, int PHASE, bool CHECK>
__device__ __forceinline__ void stream_rows(ST &st, const uint32_t *rowbase, int pitch,
                                            uint32_t (&d)[ST::WT4 + 1], int rowsOut,
                                            uint32_t op) {
    constexpr int WT4 = ST::WT4, HT = ST::HT;
    uint32_t dn[WT4 + 1];
    if constexpr (Q + 1 < HT) {
#pragma unroll
        for (int k = 0; k <= WT4; k++) dn[k] = rowbase[(Q + 1) * pitch + k];
    }
    stream_row<ST, Q, PHASE, CHECK>(st, d, rowsOut, op);
    if constexpr (Q + 1 < HT) {
#pragma unroll
        for (int k = 0; k <= WT4; k++) d[k] = dn[k];
        stream_rows<ST, Q + 1, PHASE, CHECK>(st, rowbase, pitch, d, rowsOut, op);
    }
}

template <int WT4, int HT, int POS, int WAVES, int RS, int ALIGN, bool TALIGN, bool WSUM>
#ifndef NCC_STREAM_WPE
#define NCC_STREAM_WPE 3
#endif
__global__ __launch_bounds__(WAVES * 64) __attribute__((amdgpu_waves_per_eu(NCC_STREAM_WPE)))
void corr_stream(CorrArgs a, int t, int ntx, int nty) {
    static_assert(RS % HT == 0, "strip height must be whole batches");
    static_assert(POS == 1 || POS == 2, "one or two columns per lane");
    constexpr int NT = WAVES * 64;                     // lanes per workgroup
    constexpr int NC = NT * POS;                       // output columns per workgroup
    constexpr int SEGB = NC + 4 * WT4 + 4;             // staged bytes per row
    constexpr int CH = (SEGB + 15) / 16;               // 16-byte chunks per row
    constexpr int PITCH = CH * 4 + 4;                  // dwords per LDS row
    constexpr int LOADS = (HT * CH + NT - 1) / NT;     // chunk loads per thread per batch
    __shared__ uint32_t buf[2][HT][PITCH];

    const int tix = xcd_tile((int)blockIdx.x, ntx * nty);
    if (tix < 0) return;
    const int tid = threadIdx.x;
    const int x0 = (tix % ntx) * NC, y0 = (tix / ntx) * RS;
    const int rowsOut = min(RS, a.Ho - y0);

    // a template row-aligned in whole dwords (TALIGN) needs no mask
    typedef StreamState<WT4, HT, POS, !TALIGN, WSUM> ST;
    ST st;
    // the lane's columns; lanes past the last output column compute (and
    // store) that column again, lanes before the first one (xs) the first
    const int xf = x0 + POS * tid;
    const int xa = max(min(xf, a.Wo - 1), a.xs);
    const int lxa = xa - x0;   // byte offset of the first window in a staged row
#pragma unroll
    for (int p = 0; p < POS; p++)
        st.sh[p] = (uint32_t)(max(min(xf + p, a.Wo - 1), a.xs) - x0 - (lxa & ~3));
    st.pairs = x0 >= a.xs && x0 + NC <= a.Wo;

    const int wT = a.wT;
    st.mlast = byte_mask(wT - 4 * (WT4 - 1));
    // template rows, zero-padded to WT4 dwords (wave-uniform)
    const uint8_t *T = a.tpl + (size_t)t * HT * wT;
#pragma unroll
    for (int j = 0; j < HT; j++)
#pragma unroll
        for (int k = 0; k < WT4; k++) {
            if (TALIGN) {
                st.tp[j][k] = to_vgpr(((const uint32_t *)(T + j * 4 * WT4))[k]);
            } else {
                uint32_t v = 0;
#pragma unroll
                for (int b = 0; b < 4; b++)
                    if (4 * k + b < wT) v |= (uint32_t)T[j * wT + 4 * k + b] << (8 * b);
                st.tp[j][k] = v;
            }
        }
    uint32_t sumT = 0, sumTSq = 0;
#pragma unroll
    for (int j = 0; j < HT; j++)
#pragma unroll
        for (int k = 0; k < WT4; k++) {
            sumT = dot4u(st.tp[j][k], 0x01010101u, sumT);
            sumTSq = dot4u(st.tp[j][k], st.tp[j][k], sumTSq);
        }
    st.K = (uint32_t)(wT * HT);
    st.sumT = sumT;
    // varT <= K^2 * 127.5^2 < 2^32 for K <= 514
    st.varTf = (float)(st.K * sumTSq - sumT * sumT);
#pragma unroll
    for (int p = 0; p < POS; p++) {
        st.PI[p] = st.PQ[p] = 0;
#pragma unroll
        for (int i = 0; i < HT; i++) st.acc[p][i] = st.pI[p][i] = st.pQ[p][i] = 0;
    }
    st.yrel = 0;
    const size_t plane = a.oplane;
    // per-strip bases keep the per-lane offset within 32 bits
    const size_t o0 = (size_t)y0 * a.op;
    st.off = (uint32_t)(xa - a.xs);
    st.out = a.coef + (size_t)t * plane + o0;
    st.wfirst = t == 0;
    // only dereferenced when WSUM (and st.wfirst for s0, s1)
    int32_t *sb = WSUM ? a.sums : (int32_t *)a.coef;
    st.s0 = sb + o0;
    st.s1 = sb + plane + o0;
    st.s2 = sb + (size_t)(2 + t) * plane + o0;

    // staging: chunk i of the batch -> row i / CH, bytes 16 * (i % CH); a
    // batch whose staged rectangle lies inside the image loads without any
    // per-byte test (wave-uniform choice)
    uint4 pre[LOADS];
    const bool colsIn = ALIGN == 16 && x0 + 16 * CH <= a.W;
    auto fetch = [&](int bt) {
        if (ALIGN == 16) {
            // W, ip % 16 == 0: a chunk lies wholly inside or wholly outside
            // the image; load from a clamped in-bounds address and zero what
            // lies outside (a select, not a branch)
#pragma unroll
            for (int u = 0; u < LOADS; u++) {
                const int i = tid + u * NT;
                const int r = i / CH, c = i % CH;
                const int y = y0 + bt * HT + r, x = x0 + 16 * c;
                const uint4 v = *(const uint4 *)(a.img + (size_t)min(y, a.H - 1) * a.ip + min(x, a.W - 16));
                const bool ok = i < HT * CH && y < a.H && x < a.W;
                pre[u] = ok ? v : make_uint4(0, 0, 0, 0);
            }
            return;
        }
        const bool inside = colsIn && y0 + (bt + 1) * HT <= a.H;
        if (inside) {
#pragma unroll
            for (int u = 0; u < LOADS; u++) {
                const int i = tid + u * NT;
                const int r = i / CH, c = i % CH;
                pre[u] = (i < HT * CH)
                             ? *(const uint4 *)(a.img + (size_t)(y0 + bt * HT + r) * a.ip + x0 + 16 * c)
                             : make_uint4(0, 0, 0, 0);
            }
        } else {
#pragma unroll
            for (int u = 0; u < LOADS; u++) {
                const int i = tid + u * NT;
                const int r = i / CH, c = i % CH;
                pre[u] = (i < HT * CH)
                             ? load16<ALIGN>(a.img, a.ip, a.W, a.H, x0 + 16 * c, y0 + bt * HT + r)
                             : make_uint4(0, 0, 0, 0);
            }
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

    // batches of HT image rows: the first (PHASE 0), RS/HT - 1 full ones, and
    // one past the last output row's start (PHASE 2); a strip cut short by the
    // image bottom runs its last batches in PHASE 1 and discards what lands
    // past rowsOut
    const bool full = rowsOut == RS;
    const int nb = full ? RS / HT + 1 : (rowsOut + 2 * HT - 2) / HT;
    const int nmid = full ? nb - 1 : nb;  // batches before the PHASE 2 one
    const uint32_t *rowbase0 = &buf[0][0][lxa >> 2];
    uint32_t d[WT4 + 1];
    fetch(0);
    put(0);
    __syncthreads();
    // batch 0
    if (nb > 1) fetch(1);
#pragma unroll
    for (int k = 0; k <= WT4; k++) d[k] = rowbase0[k];
    // the first batch's one output (its last row) is the strip's row 0
    const uint32_t op = (uint32_t)a.op;
    stream_rows<ST, 0, 0, false>(st, rowbase0, PITCH, d, rowsOut, op);
    if (nb > 1) put(1);
    __syncthreads();
    // full batches
    for (int bt = 1; bt < nmid; bt++) {
        if (bt + 1 < nb) fetch(bt + 1);
        const uint32_t *rowbase = rowbase0 + (bt & 1) * HT * PITCH;
#pragma unroll
        for (int k = 0; k <= WT4; k++) d[k] = rowbase[k];
        stream_rows<ST, 0, 1, true>(st, rowbase, PITCH, d, rowsOut, op);
        if (bt + 1 < nb) put(bt + 1);
        __syncthreads();
    }
    // the batch past a full strip's last output row start
    if (full) {
        const uint32_t *rowbase = rowbase0 + ((nb - 1) & 1) * HT * PITCH;
#pragma unroll
        for (int k = 0; k <= WT4; k++) d[k] = rowbase[k];
        stream_rows<ST, 0, 2, true>(st, rowbase, PITCH, d, rowsOut, op);
    }
}

// --------------------------------------------------------------- generic --
constexpr int GT = 64;  // output tile edge

// The four-corner rule on a table view: S points at view position (0, 0),
// rows `pitch` elements apart; (tx, ty) is the view's origin in the table, so
// a corner left of or above the view is a table element unless it lies left
// of column 0 or above row 0 of the table, where it reads as zero.
__device__ __forceinline__ long long sat_box(const int64_t *S, size_t pitch, int tx, int ty, int x0,
                                             int y0, int x1, int y1) {
    // 0 <= x0 < x1, 0 <= y0 < y1 inside the view guaranteed by the caller
    const int64_t *rb = S + (ptrdiff_t)(y1 - 1) * (ptrdiff_t)pitch;
    long long D = rb[x1 - 1];
    long long C = tx + x0 > 0 ? rb[x0 - 1] : 0;
    long long B = 0, A = 0;
    if (ty + y0 > 0) {
        const int64_t *rt = S + (ptrdiff_t)(y0 - 1) * (ptrdiff_t)pitch;
        B = rt[x1 - 1];
        A = tx + x0 > 0 ? rt[x0 - 1] : 0;
    }
    return D - B - C + A;
}

__global__ __launch_bounds__(256) void corr_generic(CorrArgs a, int t, Tables tb, int pitch, int rowsT,
                                                    int jb, int kb) {
    extern __shared__ uint32_t tile[];  // rowsT x pitch bytes
    const int tid = threadIdx.x;
    const int ntx = (a.Wo + GT - 1) / GT;  // 1-D grid: any height
    const int x0 = ((int)blockIdx.x % ntx) * GT, y0 = ((int)blockIdx.x / ntx) * GT;
    const int wt4 = (a.wT + 3) / 4;
    const int pw = pitch / 4;
    const int tx = tid & 15, ty = tid >> 4;
    uint32_t acc[4][4];
#pragma unroll
    for (int dy = 0; dy < 4; dy++)
#pragma unroll
        for (int s = 0; s < 4; s++) acc[dy][s] = 0;
    const uint32_t *trow = a.rows + (size_t)t * a.hT * wt4;

    // the template in blocks of jb rows x kb dwords (one block when the whole
    // tile + halo fits in LDS); each block stages its part of the image
    for (int j0 = 0; j0 < a.hT; j0 += jb) {
        const int j1 = min(j0 + jb, a.hT);
        for (int k0 = 0; k0 < wt4; k0 += kb) {
            const int k1 = min(k0 + kb, wt4);
            const int rowsB = GT + (j1 - j0) + 2;  // staged rows of this block
            __syncthreads();  // the previous block's reads are done
            for (int i = tid; i < rowsB * pw; i += 256) {
                const int r = i / pw, c = i % pw;
                const int y = y0 + j0 + r, xb = x0 + 4 * (k0 + c);
                uint32_t v = 0;
                if (y < a.H) {
                    const uint8_t *row = a.img + (size_t)y * a.ip;
#pragma unroll
                    for (int bb = 0; bb < 4; bb++)
                        if (xb + bb < a.W) v |= (uint32_t)row[xb + bb] << (8 * bb);
                }
                tile[i] = v;
            }
            __syncthreads();
            // staged row r is image row y0 + j0 + r; output row 4ty + dy meets
            // template row j = j0 + r - 4ty - dy
            for (int r = 0; r < (j1 - j0) + 3; r++) {
                const uint32_t *rowp = tile + (4 * ty + r) * pw + tx;
                uint32_t lo = rowp[0];
                for (int k = k0; k < k1; k++) {
                    const uint32_t hi = rowp[k - k0 + 1];
                    const uint32_t v0 = lo, v1 = align_bytes(hi, lo, 1), v2 = align_bytes(hi, lo, 2),
                                   v3 = align_bytes(hi, lo, 3);
#pragma unroll
                    for (int dy = 0; dy < 4; dy++) {
                        const int j = j0 + r - dy;
                        if (j >= j0 && j < j1) {
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
        }
    }

    const TStat ts = a.stats[t];
    const long long K = (long long)a.wT * a.hT;
    const size_t plane = a.oplane;
#pragma unroll
    for (int dy = 0; dy < 4; dy++) {
        const int y = y0 + 4 * ty + dy;
        if (y >= a.Ho) break;
#pragma unroll
        for (int s = 0; s < 4; s++) {
            const int x = x0 + 4 * tx + s;
            if (x >= a.Wo) break;
            const long long sumI = sat_box(tb.S, tb.pitch, tb.tx, tb.ty, x, y, x + a.wT, y + a.hT);
            const long long sumISq = sat_box(tb.Q, tb.pitch, tb.tx, tb.ty, x, y, x + a.wT, y + a.hT);
            const long long sumIT = acc[dy][s];
            const long long num = K * sumIT - sumI * ts.sumT;
            const long long varI = K * sumISq - sumI * sumI;
            const float g = ncc_coef((float)num, (float)varI, ts.varTf);
            const size_t o = (size_t)y * a.op + x;
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

#ifndef NCC_STREAM_WAVES
#define NCC_STREAM_WAVES 4
#endif
#ifndef NCC_STREAM_POS
#define NCC_STREAM_POS 1
#endif
constexpr int STREAM_WAVES = NCC_STREAM_WAVES;  // wavefronts per workgroup
constexpr int STREAM_POS = NCC_STREAM_POS;      // output columns per lane
constexpr int STREAM_WG_PER_CU = 3;             // resident workgroups per CU (168 VGPRs)

template <int WT4, int HT, int RS, bool TALIGN, bool WSUM>
hipError_t launch_stream_rs(const CorrArgs &a, int t, hipStream_t st) {
    constexpr int NC = STREAM_WAVES * 64 * STREAM_POS;
    const int ntx = (a.Wo + NC - 1) / NC, nty = (a.Ho + RS - 1) / RS;
    dim3 grid(xcd_grid(ntx * nty)), block(STREAM_WAVES * 64);
    if (a.W % 16 == 0 && a.ip % 16 == 0 && ((uintptr_t)a.img & 15) == 0)
        hipLaunchKernelGGL((corr_stream<WT4, HT, STREAM_POS, STREAM_WAVES, RS, 16, TALIGN, WSUM>),
                           grid, block, 0, st, a, t, ntx, nty);
    else if (a.W % 4 == 0 && a.ip % 4 == 0 && ((uintptr_t)a.img & 3) == 0)
        hipLaunchKernelGGL((corr_stream<WT4, HT, STREAM_POS, STREAM_WAVES, RS, 4, TALIGN, WSUM>),
                           grid, block, 0, st, a, t, ntx, nty);
    else
        hipLaunchKernelGGL((corr_stream<WT4, HT, STREAM_POS, STREAM_WAVES, RS, 1, TALIGN, WSUM>),
                           grid, block, 0, st, a, t, ntx, nty);
    return hipGetLastError();
}

int device_cus() {
    static int cus[NCC_MAX_DEVICES] = {0};
    int dev = 0;
    if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= NCC_MAX_DEVICES) return 256;
    if (cus[dev] == 0) {
        int n = 0;
        if (hipDeviceGetAttribute(&n, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess ||
            n < 1)
            n = 256;
        cus[dev] = n;
    }
    return cus[dev];
}

// Strip height: a workgroup streams RS + HT - 1 image rows for RS output
// rows, one after another, so tall strips waste least on the halo and short
// ones give more workgroups.  Estimated time ~ (rows per strip) x (waves of
// workgroups), where fewer workgroups than resident slots still cost one
// wave; the tallest strip among the cheapest wins.  The option
// NCC_OPT_STREAM_ROWS = 16, 32 or 64 fixes it instead.
int stream_rs(int Ho, int ntx, int HT) {
    const int v = opt_get(NCC_OPT_STREAM_ROWS);
    if (v == 16 || v == 32 || v == 64) return v;
    const double slots = (double)device_cus() * STREAM_WG_PER_CU;
    int best = 64;
    double best_cost = 0;
    for (int rs : {64, 32, 16}) {
        const double wgs = (double)ntx * ((Ho + rs - 1) / rs);
        const double cost = (rs + HT - 1) * (wgs > slots ? wgs / slots : 1.0);
        if (rs == 64 || cost < best_cost) {
            best = rs;
            best_cost = cost;
        }
    }
    return best;
}

template <int WT4, int HT, bool TALIGN>
hipError_t launch_stream_t(const CorrArgs &a, int t, hipStream_t st) {
    static_assert(64 % HT == 0 && 32 % HT == 0 && 16 % HT == 0, "strips of whole batches");
    constexpr int NC = STREAM_WAVES * 64 * STREAM_POS;
    const int rs = stream_rs(a.Ho, (a.Wo + NC - 1) / NC, HT);
    if (a.sums) {
        switch (rs) {
            case 16: return launch_stream_rs<WT4, HT, 16, TALIGN, true>(a, t, st);
            case 32: return launch_stream_rs<WT4, HT, 32, TALIGN, true>(a, t, st);
            default: return launch_stream_rs<WT4, HT, 64, TALIGN, true>(a, t, st);
        }
    }
    switch (rs) {
        case 16: return launch_stream_rs<WT4, HT, 16, TALIGN, false>(a, t, st);
        case 32: return launch_stream_rs<WT4, HT, 32, TALIGN, false>(a, t, st);
        default: return launch_stream_rs<WT4, HT, 64, TALIGN, false>(a, t, st);
    }
}

template <int WT4, int HT>
hipError_t launch_stream(const CorrArgs &a, int t, hipStream_t st) {
    // whole-dword template rows at a 4-byte aligned address load as dwords
    if (a.wT == 4 * WT4 && ((uintptr_t)a.tpl & 3) == 0)
        return launch_stream_t<WT4, HT, true>(a, t, st);
    return launch_stream_t<WT4, HT, false>(a, t, st);
}

// Template blocking of the generic kernel: the whole template when its tile +
// halo fits the LDS budget, else blocks of GEN_JB rows x GEN_KB dwords.
constexpr size_t GEN_LDS = 160 * 1024;
constexpr int GEN_JB = 64, GEN_KB = 128;

void generic_geometry(int wT, int hT, int *pitch, int *rowsT, int *jb, int *kb) {
    const int wt4 = (wT + 3) / 4;
    *jb = hT;
    *kb = wt4;
    auto fits = [&]() {
        *pitch = ((GT + 4 * *kb + 4) + 15) / 16 * 16;
        *rowsT = GT + *jb + 2;
        return (size_t)*pitch * *rowsT <= GEN_LDS;
    };
    if (fits()) return;
    *jb = hT < GEN_JB ? hT : GEN_JB;
    *kb = wt4 < GEN_KB ? wt4 : GEN_KB;
    fits();  // at most 592 x 130 bytes (77 KB)
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
    return wT >= 1 && hT >= 1;  // any shape: large templates run in blocks
}

hipError_t corr_generic_launch(const CorrArgs &a, int t, const Tables &tb, hipStream_t st) {
    int pitch, rowsT, jb, kb;
    generic_geometry(a.wT, a.hT, &pitch, &rowsT, &jb, &kb);
    size_t lds = (size_t)pitch * rowsT;
    if (lds > GEN_LDS) return hipErrorNotSupported;
    static bool attr_set[NCC_MAX_DEVICES] = {};
    hipError_t e = set_once(attr_set, [] {
        return hipFuncSetAttribute((const void *)corr_generic,
                                   hipFuncAttributeMaxDynamicSharedMemorySize, GEN_LDS);
    });
    if (e != hipSuccess) return e;
    dim3 grid(((a.Wo + GT - 1) / GT) * ((a.Ho + GT - 1) / GT));
    hipLaunchKernelGGL(corr_generic, grid, dim3(256), lds, st, a, t, tb, pitch, rowsT, jb, kb);
    return hipGetLastError();
}

}  // namespace ncc
