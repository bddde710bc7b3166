// Summed-area tables S (of I) and Q (of I^2) of an 8-bit image, int64,
// inclusive: The CUDA Handbook ch. 15, section 15.8 "The Denominator: Summed
// Area Tables" -- table definition, width analysis (uint32 row running sums,
// int64 table) and the separable build (a row scan, then a column scan).
//
// MI355X design: reduce-then-scan over 256 x 64 tiles, with no waiting
// between workgroups.
//   1. sat_reduce: each tile reads its bytes once and writes per-column sums
//      of its band, per-row sums of its strip and its total (uint32/uint64,
//      a few MB at 4096^2).
//   2. sat_carry:  exclusive scans of those: for each band the column sums of
//      all rows above, for each row the sum of all columns to the left, and
//      the table value above-left of each tile.
//   3. sat_downsweep: each tile re-reads its bytes, forms the uint32 row
//      running sums with a wavefront DPP scan plus the left carry, and adds
//      them down each column into int64 running sums that start from the
//      tile's top carry; S and Q are written once, as 16-byte stores.
// The row partials never go to HBM: the only full-size traffic is one read
// of the image per pass and one write of each table.
#include "ncc_internal.h"

namespace ncc {

namespace {

constexpr int WAVE_ROWS = SAT_BH / 4;  // rows per wavefront

// Four pixels x..x+3 of row y as a little-endian dword; pixels outside the
// image read as 0.
template <bool VEC>
__device__ __forceinline__ uint32_t load4(const uint8_t *img, int W, int H,
                                          int x, int y) {
    if (y >= H) return 0u;
    const uint8_t *row = img + (size_t)y * W;
    if (VEC) {
        if (x + 3 < W) return *(const uint32_t *)(row + x);
    }
    uint32_t v = 0;
#pragma unroll
    for (int k = 0; k < 4; k++)
        if (x + k < W) v |= (uint32_t)row[x + k] << (8 * k);
    return v;
}

__device__ __forceinline__ void bytes_of(uint32_t p, uint32_t b[4], uint32_t q[4]) {
#pragma unroll
    for (int k = 0; k < 4; k++) {
        b[k] = (p >> (8 * k)) & 0xffu;
        q[k] = b[k] * b[k];
    }
}

// ----------------------------------------------------------------- reduce --
template <bool VEC>
__global__ __launch_bounds__(256) void sat_reduce(const uint8_t *__restrict__ img,
                                                  int W, int H, SatWork wk) {
    const int s = blockIdx.x, b = blockIdx.y;
    const int tid = threadIdx.x, w = tid >> 6, l = tid & 63;
    const int x = s * SAT_SW + 4 * l;
    const int y0 = b * SAT_BH + w * WAVE_ROWS;

    uint32_t c1[4] = {0, 0, 0, 0}, c2[4] = {0, 0, 0, 0};
    uint32_t px[WAVE_ROWS];
#pragma unroll
    for (int r = 0; r < WAVE_ROWS; r++) px[r] = load4<VEC>(img, W, H, x, y0 + r);
#pragma unroll
    for (int r = 0; r < WAVE_ROWS; r++) {
        uint32_t bb[4], qq[4];
        bytes_of(px[r], bb, qq);
        uint32_t s1 = 0, s2 = 0;
#pragma unroll
        for (int k = 0; k < 4; k++) {
            c1[k] += bb[k];
            c2[k] += qq[k];
            s1 += bb[k];
            s2 += qq[k];
        }
        uint32_t t1 = wave_sum_u32(s1), t2 = wave_sum_u32(s2);
        int y = y0 + r;
        if (l == 0 && y < H) {
            wk.rowtot[(size_t)y * wk.nStrips + s] = t1;
            wk.rowtot[((size_t)H + y) * wk.nStrips + s] = t2;
        }
    }

    __shared__ uint32_t part[2][4][SAT_SW];
#pragma unroll
    for (int k = 0; k < 4; k++) {
        part[0][w][4 * l + k] = c1[k];
        part[1][w][4 * l + k] = c2[k];
    }
    __syncthreads();
    // thread tid sums column tid of the tile over the four wavefronts
    uint32_t v1 = part[0][0][tid] + part[0][1][tid] + part[0][2][tid] + part[0][3][tid];
    uint32_t v2 = part[1][0][tid] + part[1][1][tid] + part[1][2][tid] + part[1][3][tid];
    const int xc = s * SAT_SW + tid;
    if (xc < W) {
        wk.colsum[(size_t)b * W + xc] = v1;
        wk.colsum[((size_t)wk.nBands + b) * W + xc] = v2;
    }
    // tile totals (uint64: 256 columns of up to 64*255^2)
    uint64_t t1 = wave_incl_scan_u64((uint64_t)v1);
    uint64_t t2 = wave_incl_scan_u64((uint64_t)v2);
    __shared__ uint64_t wtot[2][4];
    if (l == 63) {
        wtot[0][w] = t1;
        wtot[1][w] = t2;
    }
    __syncthreads();
    if (tid == 0) {
        size_t o = (size_t)b * wk.nStrips + s;
        wk.tiletot[o] = wtot[0][0] + wtot[0][1] + wtot[0][2] + wtot[0][3];
        wk.tiletot[(size_t)wk.nBands * wk.nStrips + o] =
            wtot[1][0] + wtot[1][1] + wtot[1][2] + wtot[1][3];
    }
}

// ------------------------------------------------------------------ carry --
// Blocks [0, nColBlocks): one thread per column, exclusive scan down the
// bands.  Blocks [nColBlocks, nColBlocks + nRowBlocks): one thread per row,
// exclusive scan across the strips.  Last block: 2-D exclusive prefix of the
// tile totals.
__global__ __launch_bounds__(256) void sat_carry(int W, int H, SatWork wk,
                                                 int nColBlocks, int nRowBlocks) {
    const int bid = blockIdx.x, tid = threadIdx.x;
    if (bid < nColBlocks) {
        const int x = bid * 256 + tid;
        if (x >= W) return;
#pragma unroll
        for (int t = 0; t < 2; t++) {
            const uint32_t *cs = wk.colsum + (size_t)t * wk.nBands * W;
            uint64_t *cp = wk.cp + (size_t)t * wk.nBands * W;
            uint64_t run = 0;
            for (int b = 0; b < wk.nBands; b++) {
                uint32_t v = cs[(size_t)b * W + x];
                cp[(size_t)b * W + x] = run;
                run += v;
            }
        }
        return;
    }
    if (bid < nColBlocks + nRowBlocks) {
        const int y = (bid - nColBlocks) * 256 + tid;
        if (y >= H) return;
#pragma unroll
        for (int t = 0; t < 2; t++) {
            const uint32_t *rt = wk.rowtot + ((size_t)t * H + y) * wk.nStrips;
            uint32_t *lr = wk.lrow + ((size_t)t * H + y) * wk.nStrips;
            uint32_t run = 0;
            for (int s = 0; s < wk.nStrips; s++) {
                uint32_t v = rt[s];
                lr[s] = run;
                run += v;
            }
        }
        return;
    }
    // corner[b][s] = sum over b' < b, s' < s of tiletot[b'][s']
    for (int t = 0; t < 2; t++) {
        const uint64_t *tt = wk.tiletot + (size_t)t * wk.nBands * wk.nStrips;
        int64_t *cn = wk.corner + (size_t)t * wk.nBands * wk.nStrips;
        for (int s = tid; s < wk.nStrips; s += 256) {
            uint64_t run = 0;
            for (int b = 0; b < wk.nBands; b++) {
                uint64_t v = tt[(size_t)b * wk.nStrips + s];
                cn[(size_t)b * wk.nStrips + s] = (int64_t)run;
                run += v;
            }
        }
        __syncthreads();
        for (int b = tid; b < wk.nBands; b += 256) {
            int64_t run = 0;
            for (int s = 0; s < wk.nStrips; s++) {
                int64_t v = cn[(size_t)b * wk.nStrips + s];
                cn[(size_t)b * wk.nStrips + s] = run;
                run += v;
            }
        }
        __syncthreads();
    }
}

// ------------------------------------------------------------- downsweep --
// Row partials R(x,y) = sum of row y over columns 0..x (uint32), for the
// lane's four columns: left carry + wavefront exclusive scan + local scan.
__device__ __forceinline__ void row_partials(uint32_t p, uint32_t left1, uint32_t left2,
                                             uint32_t r1[4], uint32_t r2[4]) {
    uint32_t bb[4], qq[4];
    bytes_of(p, bb, qq);
    r1[0] = bb[0];
    r2[0] = qq[0];
#pragma unroll
    for (int k = 1; k < 4; k++) {
        r1[k] = r1[k - 1] + bb[k];
        r2[k] = r2[k - 1] + qq[k];
    }
    uint32_t e1 = wave_incl_scan_u32(r1[3]) - r1[3] + left1;
    uint32_t e2 = wave_incl_scan_u32(r2[3]) - r2[3] + left2;
#pragma unroll
    for (int k = 0; k < 4; k++) {
        r1[k] += e1;
        r2[k] += e2;
    }
}

template <bool VEC>
__global__ __launch_bounds__(256) void sat_downsweep(const uint8_t *__restrict__ img,
                                                     int W, int H, SatWork wk,
                                                     int64_t *__restrict__ S,
                                                     int64_t *__restrict__ Q) {
    const int s = blockIdx.x, b = blockIdx.y;
    const int tid = threadIdx.x, w = tid >> 6, l = tid & 63;
    const int x = s * SAT_SW + 4 * l;
    const int y0 = b * SAT_BH + w * WAVE_ROWS;

    uint32_t px[WAVE_ROWS];
#pragma unroll
    for (int r = 0; r < WAVE_ROWS; r++) px[r] = load4<VEC>(img, W, H, x, y0 + r);
    // left carries of the wavefront's rows: lane r holds row y0 + r
    uint32_t lc1 = 0, lc2 = 0;
    if (l < WAVE_ROWS && y0 + l < H) {
        lc1 = wk.lrow[(size_t)(y0 + l) * wk.nStrips + s];
        lc2 = wk.lrow[((size_t)H + y0 + l) * wk.nStrips + s];
    }

    // pass 1: the wavefront's column totals of row partials
    uint64_t ct1[4] = {0, 0, 0, 0}, ct2[4] = {0, 0, 0, 0};
#pragma unroll
    for (int r = 0; r < WAVE_ROWS; r++) {
        uint32_t r1[4], r2[4];
        row_partials(px[r], (uint32_t)__builtin_amdgcn_readlane((int)lc1, r),
                     (uint32_t)__builtin_amdgcn_readlane((int)lc2, r), r1, r2);
#pragma unroll
        for (int k = 0; k < 4; k++) {
            ct1[k] += r1[k];
            ct2[k] += r2[k];
        }
    }
    __shared__ uint64_t part[2][4][SAT_SW];
#pragma unroll
    for (int k = 0; k < 4; k++) {
        part[0][w][4 * l + k] = ct1[k];
        part[1][w][4 * l + k] = ct2[k];
    }

    // top carry of the tile: corner + scan of the column sums above the band
    uint64_t a1[4], a2[4];
    {
        const uint64_t *cp1 = wk.cp + (size_t)b * W;
        const uint64_t *cp2 = wk.cp + ((size_t)wk.nBands + b) * W;
#pragma unroll
        for (int k = 0; k < 4; k++) {
            a1[k] = (x + k < W) ? cp1[x + k] : 0;
            a2[k] = (x + k < W) ? cp2[x + k] : 0;
        }
#pragma unroll
        for (int k = 1; k < 4; k++) {
            a1[k] += a1[k - 1];
            a2[k] += a2[k - 1];
        }
        size_t co = (size_t)b * wk.nStrips + s;
        uint64_t e1 = wave_incl_scan_u64(a1[3]) - a1[3] + (uint64_t)wk.corner[co];
        uint64_t e2 = wave_incl_scan_u64(a2[3]) - a2[3] +
                      (uint64_t)wk.corner[(size_t)wk.nBands * wk.nStrips + co];
#pragma unroll
        for (int k = 0; k < 4; k++) {
            a1[k] += e1;
            a2[k] += e2;
        }
    }
    __syncthreads();
    for (int ww = 0; ww < w; ww++) {
#pragma unroll
        for (int k = 0; k < 4; k++) {
            a1[k] += part[0][ww][4 * l + k];
            a2[k] += part[1][ww][4 * l + k];
        }
    }

    // pass 2: running column sums, written row by row
#pragma unroll
    for (int r = 0; r < WAVE_ROWS; r++) {
        const int y = y0 + r;
        if (y >= H) break;
        uint32_t r1[4], r2[4];
        row_partials(px[r], (uint32_t)__builtin_amdgcn_readlane((int)lc1, r),
                     (uint32_t)__builtin_amdgcn_readlane((int)lc2, r), r1, r2);
#pragma unroll
        for (int k = 0; k < 4; k++) {
            a1[k] += r1[k];
            a2[k] += r2[k];
        }
        int64_t *srow = S + (size_t)y * W;
        int64_t *qrow = Q + (size_t)y * W;
        if (VEC && x + 3 < W) {
            typedef long long v2l __attribute__((ext_vector_type(2)));
            v2l s01 = {(long long)a1[0], (long long)a1[1]};
            v2l s23 = {(long long)a1[2], (long long)a1[3]};
            v2l q01 = {(long long)a2[0], (long long)a2[1]};
            v2l q23 = {(long long)a2[2], (long long)a2[3]};
            __builtin_nontemporal_store(s01, (v2l *)(srow + x));
            __builtin_nontemporal_store(s23, (v2l *)(srow + x + 2));
            __builtin_nontemporal_store(q01, (v2l *)(qrow + x));
            __builtin_nontemporal_store(q23, (v2l *)(qrow + x + 2));
        } else {
#pragma unroll
            for (int k = 0; k < 4; k++) {
                if (x + k < W) {
                    __builtin_nontemporal_store((long long)a1[k], (long long *)(srow + x + k));
                    __builtin_nontemporal_store((long long)a2[k], (long long *)(qrow + x + k));
                }
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
    const bool vec = (W % 4 == 0) && (((uintptr_t)img & 3) == 0) &&
                     (((uintptr_t)S & 15) == 0) && (((uintptr_t)Q & 15) == 0);
    dim3 grid(wk.nStrips, wk.nBands), block(256);
    if (vec)
        hipLaunchKernelGGL(sat_reduce<true>, grid, block, 0, st, img, W, H, wk);
    else
        hipLaunchKernelGGL(sat_reduce<false>, grid, block, 0, st, img, W, H, wk);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
    int nColBlocks = (W + 255) / 256, nRowBlocks = (H + 255) / 256;
    hipLaunchKernelGGL(sat_carry, dim3(nColBlocks + nRowBlocks + 1), block, 0, st, W, H, wk,
                       nColBlocks, nRowBlocks);
    e = hipGetLastError();
    if (e != hipSuccess) return e;
    if (vec)
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
