// Summed-area tables S (of I) and Q (of I^2) of an 8-bit image, int64,
// inclusive: The CUDA Handbook ch. 15, section 15.8 "The Denominator: Summed
// Area Tables" -- table definition, width analysis (uint32 row running sums,
// int64 table) and the separable build (a row scan, then a column scan).
//
// MI355X design: reduce-then-scan over 128-column x 64-row tiles, with no
// waiting between workgroups.
//   1. sat_reduce: each tile reads its bytes once and writes per-column sums
//      of its band, per-row sums of its strip and its total (uint32/uint64,
//      a few MB at 4096^2).
//   2. sat_carry:  exclusive scans of those: for each band the column sums of
//      all rows above, for each row the sum of all columns to the left, and
//      the table value above-left of each tile.
//   3. sat_downsweep: each tile re-reads its bytes, forms the uint32 row
//      running sums with a wavefront DPP scan plus the left carry, and adds
//      them down each column into int64 running sums that start from the
//      tile's top carry; S and Q are written once.  Lane l owns columns 2l
//      and 2l+1, so one store instruction covers 1 KB of a table row.
// The row partials never go to HBM: the only full-size traffic is one read
// of the image per pass and one write of each table.
#include "ncc_internal.h"

namespace ncc {

namespace {

constexpr int WAVE_ROWS = SAT_BH / 4;  // rows per wavefront

// Pixels x, x+1 of row y as the low 16 bits of a dword; pixels outside the
// image read as 0.
template <bool VEC>
__device__ __forceinline__ uint32_t load2(const uint8_t *img, int W, int H, int x, int y) {
    if (y >= H) return 0u;
    const uint8_t *row = img + (size_t)y * W;
    if (VEC && x + 1 < W) return *(const uint16_t *)(row + x);
    uint32_t v = 0;
    if (x < W) v = row[x];
    if (x + 1 < W) v |= (uint32_t)row[x + 1] << 8;
    return v;
}

// Bytes x .. x+15 of row y (zero outside the image).
template <bool VEC>
__device__ __forceinline__ uint4 load16(const uint8_t *img, int W, int H, int x, int y) {
    uint4 v = make_uint4(0, 0, 0, 0);
    if (y >= H || x >= W) return v;
    const uint8_t *row = img + (size_t)y * W;
    if (VEC && x + 15 < W) return *(const uint4 *)(row + x);
    uint32_t w[4] = {0, 0, 0, 0};
#pragma unroll
    for (int b = 0; b < 16; b++)
        if (x + b < W) w[b >> 2] |= (uint32_t)row[x + b] << (8 * (b & 3));
    return make_uint4(w[0], w[1], w[2], w[3]);
}

// ----------------------------------------------------------------- reduce --
// Tile sums for the carries: per column of the band (colsum), per row of the
// strip (rowtot) and the tile total.  A wavefront reduces one 128 x 64 tile:
// lane l loads 16 columns (group l % 8) of the 8 rows 8*(l/8) .. +7.
template <bool VEC>
__global__ __launch_bounds__(256) void sat_reduce(const uint8_t *__restrict__ img, int W, int H,
                                                  SatWork wk) {
    const int tid = threadIdx.x, w = tid >> 6, l = tid & 63;
    const int s = blockIdx.x * 4 + w, b = blockIdx.y;
    const int c8 = l & 7, rg = l >> 3;
    const int x = s * SAT_SW + 16 * c8;
    const int y = b * SAT_BH + 8 * rg;
    const bool live = s < wk.nStrips;
    uint4 px[8];
#pragma unroll
    for (int r = 0; r < 8; r++)
        px[r] = live ? load16<VEC>(img, W, H, x, y + r) : make_uint4(0, 0, 0, 0);

    // row sums: 16 columns per lane, then over the 8 lanes of a row group
    // (DPP: swap pairs, swap pair-pairs, then lane 8g+7 adds lane 8g+3)
    uint32_t cI[16], cQ[16];
#pragma unroll
    for (int c = 0; c < 16; c++) cI[c] = cQ[c] = 0;
#pragma unroll
    for (int r = 0; r < 8; r++) {
        const uint32_t d[4] = {px[r].x, px[r].y, px[r].z, px[r].w};
        uint32_t a = 0, q = 0;
#pragma unroll
        for (int k = 0; k < 4; k++) {
            a = dot4u(d[k], 0x01010101u, a);
            q = dot4u(d[k], d[k], q);
#pragma unroll
            for (int e = 0; e < 4; e++) {
                const uint32_t v = (d[k] >> (8 * e)) & 0xffu;
                cI[4 * k + e] += v;
                cQ[4 * k + e] += v * v;
            }
        }
        a += (uint32_t)__builtin_amdgcn_update_dpp(0, (int)a, 0xB1, 0xf, 0xf, false);
        q += (uint32_t)__builtin_amdgcn_update_dpp(0, (int)q, 0xB1, 0xf, 0xf, false);
        a += (uint32_t)__builtin_amdgcn_update_dpp(0, (int)a, 0x4E, 0xf, 0xf, false);
        q += (uint32_t)__builtin_amdgcn_update_dpp(0, (int)q, 0x4E, 0xf, 0xf, false);
        a += (uint32_t)__builtin_amdgcn_update_dpp(0, (int)a, DPP_ROW_SHR4, 0xf, 0xf, false);
        q += (uint32_t)__builtin_amdgcn_update_dpp(0, (int)q, DPP_ROW_SHR4, 0xf, 0xf, false);
        if (c8 == 7 && live && y + r < H) {
            wk.rowtot[(size_t)(y + r) * wk.nStrips + s] = a;
            wk.rowtot[((size_t)H + y + r) * wk.nStrips + s] = q;
        }
    }

    // column sums: the 8 row groups of the wavefront meet in LDS
    __shared__ uint32_t part[4][2][8][SAT_SW];
#pragma unroll
    for (int c = 0; c < 16; c += 4) {
        *(uint4 *)&part[w][0][rg][16 * c8 + c] = make_uint4(cI[c], cI[c + 1], cI[c + 2], cI[c + 3]);
        *(uint4 *)&part[w][1][rg][16 * c8 + c] = make_uint4(cQ[c], cQ[c + 1], cQ[c + 2], cQ[c + 3]);
    }
    __syncthreads();
    uint32_t sI[2] = {0, 0}, sQ[2] = {0, 0};
#pragma unroll
    for (int r = 0; r < 8; r++) {
        const uint2 u = *(const uint2 *)&part[w][0][r][2 * l];
        const uint2 v = *(const uint2 *)&part[w][1][r][2 * l];
        sI[0] += u.x;
        sI[1] += u.y;
        sQ[0] += v.x;
        sQ[1] += v.y;
    }
    if (!live) return;  // wavefront-uniform; no barrier follows
    const int xc = s * SAT_SW + 2 * l;
    uint32_t *cs0 = wk.colsum + (size_t)b * W;
    uint32_t *cs1 = wk.colsum + ((size_t)wk.nBands + b) * W;
    if (xc < W) {
        cs0[xc] = sI[0];
        cs1[xc] = sQ[0];
    }
    if (xc + 1 < W) {
        cs0[xc + 1] = sI[1];
        cs1[xc + 1] = sQ[1];
    }
    // tile totals: 128 columns of at most 64*255^2 fit uint32
    const uint32_t tI = wave_sum_u32(sI[0] + sI[1]);
    const uint32_t tQ = wave_sum_u32(sQ[0] + sQ[1]);
    if (l == 0) {
        const size_t o = (size_t)b * wk.nStrips + s;
        wk.tiletot[o] = tI;
        wk.tiletot[(size_t)wk.nBands * wk.nStrips + o] = tQ;
    }
}

// ------------------------------------------------------------------ carry --
// Exclusive scans of the tile sums, in three roles by block index.
//  cp:     a block scans 64 columns of one table down all bands: thread
//          (column, quarter) loads its quarter of the bands at once, the four
//          quarters are combined in LDS, then written back.
//  lrow:   one thread per (table, row) scans the row's strip sums.
//  corner: one block per table forms the 2-D exclusive prefix of the tile
//          totals, in LDS when they fit.
constexpr int CP_COLS = 64;
constexpr int CP_MAXQ = 32;  // bands per quarter held in registers

__global__ __launch_bounds__(256) void sat_carry(int W, int H, SatWork wk, int nCpBlocks,
                                                 int nRowBlocks) {
    const int bid = blockIdx.x, tid = threadIdx.x;
    const int nB = wk.nBands, nS = wk.nStrips;
    if (bid < nCpBlocks) {
        const int colBlocks = (W + CP_COLS - 1) / CP_COLS;
        const int t = bid / colBlocks;
        const int x = (bid % colBlocks) * CP_COLS + (tid & (CP_COLS - 1));
        const int qtr = tid / CP_COLS;  // 0..3
        const uint32_t *__restrict__ cs = wk.colsum + (size_t)t * nB * W;
        uint64_t *__restrict__ cp = wk.cp + (size_t)t * nB * W;
        __shared__ uint64_t qsum[4][CP_COLS];
        const int per = (nB + 3) / 4;
        uint64_t run = 0;
        // quarters longer than CP_MAXQ bands are walked in pieces
        for (int p0 = 0; p0 < per; p0 += CP_MAXQ) {
            uint32_t v[CP_MAXQ];
#pragma unroll
            for (int k = 0; k < CP_MAXQ; k++) {
                const int bb = qtr * per + p0 + k;
                v[k] = (p0 + k < per && bb < nB && x < W) ? cs[(size_t)bb * W + x] : 0u;
            }
#pragma unroll
            for (int k = 0; k < CP_MAXQ; k++) run += v[k];
        }
        qsum[qtr][tid & (CP_COLS - 1)] = run;
        __syncthreads();
        uint64_t base = 0;
        for (int q = 0; q < qtr; q++) base += qsum[q][tid & (CP_COLS - 1)];
        if (x >= W) return;
        for (int p0 = 0; p0 < per; p0 += CP_MAXQ) {
            uint32_t v[CP_MAXQ];
#pragma unroll
            for (int k = 0; k < CP_MAXQ; k++) {
                const int bb = qtr * per + p0 + k;
                v[k] = (p0 + k < per && bb < nB) ? cs[(size_t)bb * W + x] : 0u;
            }
#pragma unroll
            for (int k = 0; k < CP_MAXQ; k++) {
                const int bb = qtr * per + p0 + k;
                if (p0 + k < per && bb < nB) cp[(size_t)bb * W + x] = base;
                base += v[k];
            }
        }
        return;
    }
    if (bid < nCpBlocks + nRowBlocks) {
        const int i = (bid - nCpBlocks) * 256 + tid;
        if (i >= 2 * H) return;
        const uint32_t *__restrict__ rt = wk.rowtot + (size_t)i * nS;
        uint32_t *__restrict__ lr = wk.lrow + (size_t)i * nS;
        uint32_t run = 0;
        for (int s0 = 0; s0 < nS; s0 += 32) {
            uint32_t v[32];
#pragma unroll
            for (int k = 0; k < 32; k++) v[k] = (s0 + k < nS) ? rt[s0 + k] : 0u;
#pragma unroll
            for (int k = 0; k < 32; k++) {
                if (s0 + k < nS) lr[s0 + k] = run;
                run += v[k];
            }
        }
        return;
    }
    // corner[b][s] = sum over b' < b, s' < s of tiletot[b'][s']
    const int t = bid - nCpBlocks - nRowBlocks;
    const uint64_t *tt = wk.tiletot + (size_t)t * nB * nS;
    int64_t *cn = wk.corner + (size_t)t * nB * nS;
    constexpr int LDS_MAX = 4096;
    __shared__ uint64_t g[LDS_MAX];
    if ((size_t)nB * nS <= LDS_MAX) {
        for (int i = tid; i < nB * nS; i += 256) g[i] = tt[i];
        __syncthreads();
        for (int s = tid; s < nS; s += 256) {  // down the bands
            uint64_t run = 0;
            for (int b = 0; b < nB; b++) {
                const uint64_t v = g[b * nS + s];
                g[b * nS + s] = run;
                run += v;
            }
        }
        __syncthreads();
        for (int b = tid; b < nB; b += 256) {  // across the strips
            uint64_t run = 0;
            for (int s = 0; s < nS; s++) {
                const uint64_t v = g[b * nS + s];
                g[b * nS + s] = run;
                run += v;
            }
        }
        __syncthreads();
        for (int i = tid; i < nB * nS; i += 256) cn[i] = (int64_t)g[i];
        return;
    }
    for (int s = tid; s < nS; s += 256) {
        uint64_t run = 0;
        for (int b = 0; b < nB; b++) {
            const uint64_t v = tt[(size_t)b * nS + s];
            cn[(size_t)b * nS + s] = (int64_t)run;
            run += v;
        }
    }
    __syncthreads();
    for (int b = tid; b < nB; b += 256) {
        int64_t run = 0;
        for (int s = 0; s < nS; s++) {
            const int64_t v = cn[(size_t)b * nS + s];
            cn[(size_t)b * nS + s] = run;
            run += v;
        }
    }
}

// ------------------------------------------------------------- downsweep --
// Lane l of every wavefront owns columns x = 128*s + 2l and x + 1, so each
// 16-byte store of a row lands next to its neighbours' (1 KB per wavefront).
template <bool VEC>
__global__ __launch_bounds__(256) void sat_downsweep(const uint8_t *__restrict__ img, int W, int H,
                                                     SatWork wk, int64_t *__restrict__ S,
                                                     int64_t *__restrict__ Q) {
    const int tix = xcd_tile((int)blockIdx.x, wk.nStrips * wk.nBands);
    if (tix < 0) return;
    const int s = tix % wk.nStrips, b = tix / wk.nStrips;
    const int tid = threadIdx.x, w = tid >> 6, l = tid & 63;
    const int x = s * SAT_SW + 2 * l;
    const int y0 = b * SAT_BH + w * WAVE_ROWS;

    uint32_t px[WAVE_ROWS];
#pragma unroll
    for (int r = 0; r < WAVE_ROWS; r++) px[r] = load2<VEC>(img, W, H, x, y0 + r);
    // left carries of the wavefront's rows: lane r holds row y0 + r
    uint32_t lc1 = 0, lc2 = 0;
    if (l < WAVE_ROWS && y0 + l < H) {
        lc1 = wk.lrow[(size_t)(y0 + l) * wk.nStrips + s];
        lc2 = wk.lrow[((size_t)H + y0 + l) * wk.nStrips + s];
    }

    // pass 1: uint32 row partials R(x,y) = sum over columns 0..x of row y
    // (left carry + wavefront exclusive scan + own pixels), kept in registers,
    // and their column totals over the wavefront's rows
    uint32_t R1a[WAVE_ROWS], R1b[WAVE_ROWS], R2a[WAVE_ROWS], R2b[WAVE_ROWS];
    uint64_t c1a = 0, c1b = 0, c2a = 0, c2b = 0;
#pragma unroll
    for (int r = 0; r < WAVE_ROWS; r++) {
        const uint32_t b0 = px[r] & 0xffu, b1 = (px[r] >> 8) & 0xffu;
        const uint32_t p1 = b0 + b1, p2 = b0 * b0 + b1 * b1;
        const uint32_t e1 = wave_incl_scan_u32(p1) - p1 +
                            (uint32_t)__builtin_amdgcn_readlane((int)lc1, r);
        const uint32_t e2 = wave_incl_scan_u32(p2) - p2 +
                            (uint32_t)__builtin_amdgcn_readlane((int)lc2, r);
        R1a[r] = e1 + b0;
        R1b[r] = e1 + p1;
        R2a[r] = e2 + b0 * b0;
        R2b[r] = e2 + p2;
        c1a += R1a[r];
        c1b += R1b[r];
        c2a += R2a[r];
        c2b += R2b[r];
    }
    __shared__ uint64_t part[4][4][64];  // [wave][value][lane]
    part[w][0][l] = c1a;
    part[w][1][l] = c1b;
    part[w][2][l] = c2a;
    part[w][3][l] = c2b;

    // top carry: S(x, top - 1) = corner + scan of the column sums above the band
    uint64_t s1a, s1b, s2a, s2b;
    {
        const uint64_t *cp1 = wk.cp + (size_t)b * W;
        const uint64_t *cp2 = wk.cp + ((size_t)wk.nBands + b) * W;
        const uint64_t u1a = x < W ? cp1[x] : 0, u1b = x + 1 < W ? cp1[x + 1] : 0;
        const uint64_t u2a = x < W ? cp2[x] : 0, u2b = x + 1 < W ? cp2[x + 1] : 0;
        const size_t co = (size_t)b * wk.nStrips + s;
        const uint64_t p1 = u1a + u1b, p2 = u2a + u2b;
        const uint64_t e1 = wave_incl_scan_u64(p1) - p1 + (uint64_t)wk.corner[co];
        const uint64_t e2 = wave_incl_scan_u64(p2) - p2 +
                            (uint64_t)wk.corner[(size_t)wk.nBands * wk.nStrips + co];
        s1a = e1 + u1a;
        s1b = e1 + p1;
        s2a = e2 + u2a;
        s2b = e2 + p2;
    }
    __syncthreads();
    for (int ww = 0; ww < w; ww++) {
        s1a += part[ww][0][l];
        s1b += part[ww][1][l];
        s2a += part[ww][2][l];
        s2b += part[ww][3][l];
    }

    // pass 2: running column sums, written row by row
    typedef long long v2l __attribute__((ext_vector_type(2)));
    const bool pair = VEC && x + 1 < W;
#pragma unroll
    for (int r = 0; r < WAVE_ROWS; r++) {
        const int y = y0 + r;
        if (y >= H) break;
        s1a += R1a[r];
        s1b += R1b[r];
        s2a += R2a[r];
        s2b += R2b[r];
        int64_t *srow = S + (size_t)y * W + x;
        int64_t *qrow = Q + (size_t)y * W + x;
        if (pair) {
            const v2l sv = {(long long)s1a, (long long)s1b};
            const v2l qv = {(long long)s2a, (long long)s2b};
            __builtin_nontemporal_store(sv, (v2l *)srow);
            __builtin_nontemporal_store(qv, (v2l *)qrow);
        } else {
            if (x < W) {
                __builtin_nontemporal_store((long long)s1a, (long long *)srow);
                __builtin_nontemporal_store((long long)s2a, (long long *)qrow);
            }
            if (x + 1 < W) {
                __builtin_nontemporal_store((long long)s1b, (long long *)srow + 1);
                __builtin_nontemporal_store((long long)s2b, (long long *)qrow + 1);
            }
        }
    }
}

}  // namespace

size_t sat_work_bytes(int W, int H) {
    size_t nS = (W + SAT_SW - 1) / SAT_SW, nB = (H + SAT_BH - 1) / SAT_BH;
    size_t bytes = 0;
    auto add = [&](size_t n) { bytes += (n + 255) & ~(size_t)255; };
    add(2 * nB * W * 4);   // colsum
    add(2 * (size_t)H * nS * 4);  // rowtot
    add(2 * nB * nS * 8);  // tiletot
    add(2 * nB * W * 8);   // cp
    add(2 * (size_t)H * nS * 4);  // lrow
    add(2 * nB * nS * 8);  // corner
    return bytes;
}

SatWork sat_work_carve(void *base, int W, int H) {
    SatWork wk;
    wk.nStrips = (W + SAT_SW - 1) / SAT_SW;
    wk.nBands = (H + SAT_BH - 1) / SAT_BH;
    size_t nS = wk.nStrips, nB = wk.nBands;
    char *p = (char *)base;
    auto take = [&](size_t n) { char *q = p; p += (n + 255) & ~(size_t)255; return (void *)q; };
    wk.colsum = (uint32_t *)take(2 * nB * W * 4);
    wk.rowtot = (uint32_t *)take(2 * (size_t)H * nS * 4);
    wk.tiletot = (uint64_t *)take(2 * nB * nS * 8);
    wk.cp = (uint64_t *)take(2 * nB * W * 8);
    wk.lrow = (uint32_t *)take(2 * (size_t)H * nS * 4);
    wk.corner = (int64_t *)take(2 * nB * nS * 8);
    return wk;
}

hipError_t sat_build_launch(const uint8_t *img, int W, int H, int64_t *S, int64_t *Q,
                            const SatWork &wk, hipStream_t st) {
    // 16-byte image rows for the reduce pass; even widths and 16-byte table
    // rows for the paired loads and stores of the downsweep
    const bool rvec = (W % 16 == 0) && (((uintptr_t)img & 15) == 0);
    const bool dvec = (W % 2 == 0) && (((uintptr_t)img & 1) == 0) &&
                      (((uintptr_t)S & 15) == 0) && (((uintptr_t)Q & 15) == 0);
    dim3 block(256);
    dim3 rgrid((wk.nStrips + 3) / 4, wk.nBands);
    if (rvec)
        hipLaunchKernelGGL(sat_reduce<true>, rgrid, block, 0, st, img, W, H, wk);
    else
        hipLaunchKernelGGL(sat_reduce<false>, rgrid, block, 0, st, img, W, H, wk);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
    const int nCpBlocks = 2 * ((W + CP_COLS - 1) / CP_COLS), nRowBlocks = (2 * H + 255) / 256;
    hipLaunchKernelGGL(sat_carry, dim3(nCpBlocks + nRowBlocks + 2), block, 0, st, W, H, wk,
                       nCpBlocks, nRowBlocks);
    e = hipGetLastError();
    if (e != hipSuccess) return e;
    dim3 grid(xcd_grid(wk.nStrips * wk.nBands));
    if (dvec)
        hipLaunchKernelGGL(sat_downsweep<true>, grid, block, 0, st, img, W, H, wk, S, Q);
    else
        hipLaunchKernelGGL(sat_downsweep<false>, grid, block, 0, st, img, W, H, wk, S, Q);
    return hipGetLastError();
}

// ------------------------------------------------------------- box query --
// The four-corner rule of the satBox listing: D - B - C + A, corners on the
// table's leading edges read as zero; empty boxes give 0, boxes outside the
// table INT64_MIN.
namespace {
__global__ __launch_bounds__(256) void box_kernel(const int64_t *__restrict__ S, int W, int H,
                                                  const int32_t *__restrict__ rects, int64_t n,
                                                  int64_t *__restrict__ out) {
    for (int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; i < n;
         i += (int64_t)gridDim.x * blockDim.x) {
        const int x0 = rects[4 * i + 0], y0 = rects[4 * i + 1];
        const int x1 = rects[4 * i + 2], y1 = rects[4 * i + 3];
        int64_t v;
        if (!(0 <= x0 && x0 <= x1 && x1 <= W && 0 <= y0 && y0 <= y1 && y1 <= H)) {
            v = INT64_MIN;
        } else if (x0 == x1 || y0 == y1) {
            v = 0;
        } else {
            const int64_t *rb = S + (size_t)(y1 - 1) * W;  // bottom row
            int64_t D = rb[x1 - 1];
            int64_t C = x0 > 0 ? rb[x0 - 1] : 0;
            int64_t B = 0, A = 0;
            if (y0 > 0) {
                const int64_t *rt = S + (size_t)(y0 - 1) * W;  // row above
                B = rt[x1 - 1];
                A = x0 > 0 ? rt[x0 - 1] : 0;
            }
            v = D - B - C + A;
        }
        __builtin_nontemporal_store((long long)v, (long long *)(out + i));
    }
}
}  // namespace

hipError_t box_launch(const int64_t *S, int W, int H, const int32_t *rects, int64_t n,
                      int64_t *out, hipStream_t st) {
    int64_t blocks = (n + 255) / 256;
    if (blocks > 65536) blocks = 65536;
    hipLaunchKernelGGL(box_kernel, dim3((unsigned)blocks), dim3(256), 0, st, S, W, H, rects, n, out);
    return hipGetLastError();
}

}  // namespace ncc
