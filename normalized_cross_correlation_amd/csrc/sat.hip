// Summed-area tables S (of I) and Q (of I^2) of an 8-bit image, int64,
// inclusive: The CUDA Handbook ch. 15, section 15.8 "The Denominator: Summed
// Area Tables" -- table definition, width analysis (uint32 row running sums,
// int64 table) and the separable build (a row scan, then a column scan).
//
// MI355X design: three passes with no waiting between workgroups.
//   1. sat_rows: a workgroup reads one band of SAT_BH rows across a segment of
//      SAT_QW columns once.  Per row it forms the strip sums and their running
//      sum along the segment (the row carries of the third pass); per column
//      it forms the band's column sums and their running sum along the
//      segment, i.e. the band's sum of the segment-local row running sums.
//   2. sat_top: for every column, the exclusive scan of those band values down
//      the bands (plus the segments to the left) is the table value on the
//      row just above each band: S(x, y0 - 1), Q(x, y0 - 1).  Beside these
//      column blocks, row blocks form each row's running sum of the segment
//      totals (the part of a row carry from the segments to the left).
//   3. sat_downsweep: a workgroup owns a tile of SAT_SW columns x SAT_SUB
//      bands and re-reads its bytes band by band (the next band's loads in
//      flight while the current one is stored); the uint32 row running sums
//      (left carry + wavefront DPP scan) stay in registers and are added down
//      each column into int64 running sums that start from the pass-2 value
//      above the tile.  S and Q are written once, lane l owning columns 2l
//      and 2l+1 so one store instruction covers 1 KB of a table row.
// The row running sums never go to HBM: the full-size traffic is two reads of
// the image and one write of each table; the carries are a few MB.
#include "ncc_internal.h"

namespace ncc {

namespace {

constexpr int WAVE_ROWS = SAT_BH / 4;      // downsweep rows per wavefront
constexpr int SAT_SPQ = SAT_QW / SAT_SW;   // strips per row-pass segment

// Image loads take a clamped, in-bounds address and zero what lies outside
// the image afterwards (a select, not a branch), so the loads of all rows
// issue back to back.

// Pixels x, x+1 of row y (at img + y * ip) as the low 16 bits of a dword,
// read from clamped in-bounds addresses (load2_raw) and then zeroed where
// they lie outside the image (mask2).  Keeping the two apart lets a caller
// issue a band's loads back to back and mask where it uses them.
// VEC: W, ip and x even and img 2-byte aligned, so x < W implies x + 1 < W.
template <bool VEC>
__device__ __forceinline__ uint32_t load2_raw(const uint8_t *img, size_t ip, int W, int H, int x, int y) {
    const uint8_t *row = img + (size_t)min(y, H - 1) * ip;
    if (VEC) return *(const uint16_t *)(row + min(x, W - 2));
    return (uint32_t)row[min(x, W - 1)] | ((uint32_t)row[min(x + 1, W - 1)] << 8);
}

__device__ __forceinline__ uint32_t mask2(uint32_t v, int W, int H, int x, int y) {
    const uint32_t m = y >= H ? 0u : (x + 1 < W ? 0xffffu : (x < W ? 0xffu : 0u));
    return v & m;
}

template <bool VEC>
__device__ __forceinline__ uint32_t load2(const uint8_t *img, size_t ip, int W, int H, int x, int y) {
    return mask2(load2_raw<VEC>(img, ip, W, H, x, y), W, H, x, y);
}

// -------------------------------------------------------------- row pass --
// Workgroup (segment q, band b): wavefront w takes rows 8w .. 8w+7 of the
// band and lane l the 16 columns q*SAT_QW + 16l .. +15 of each, so the 8
// lanes l/8 = k cover strip k of the segment.  Bounds that keep the sums in
// uint32: a segment row of 1024 squares and a band-segment of 32 x 1024
// squares stay below 2^31; 8-row column sums of bytes fit 16 bits.
constexpr int ROWS_PER_WAVE = SAT_BH / 4;

// Bytes x .. x+15 of row y.  VEC: W, ip and x multiples of 16, img 16-byte
// aligned.
// The zeroing is a mask, not a branch: a conditional assignment compiles to
// a branch that waits for its load, which serialises the band's loads.
template <bool VEC>
__device__ __forceinline__ uint4 load16(const uint8_t *img, size_t ip, int W, int H, int x, int y) {
    const uint8_t *row = img + (size_t)min(y, H - 1) * ip;
    uint4 v;
    if (VEC) {
        v = *(const uint4 *)(row + min(x, W - 16));
        const uint32_t m = (x < W && y < H) ? 0xffffffffu : 0u;
        v.x &= m;
        v.y &= m;
        v.z &= m;
        v.w &= m;
    } else {
        // five aligned dwords from addresses clamped to the dword holding the
        // row's last byte (every read touches an image byte), byte-aligned;
        // then bytes past W (and rows past H) are zeroed
        const uint8_t *first = row + min(x, W - 1), *lastb = row + W - 1;
        const uint32_t sh = (uint32_t)((uintptr_t)first & 3);
        const uint32_t *base = (const uint32_t *)(first - sh);
        const uint32_t *last = (const uint32_t *)(lastb - ((uintptr_t)lastb & 3));
        uint32_t d[5];
#pragma unroll
        for (int k = 0; k < 5; k++) d[k] = *(base + k <= last ? base + k : last);
        const int valid = y < H ? min(max(W - x, 0), 16) : 0;  // bytes of the chunk inside
        uint32_t o[4];
#pragma unroll
        for (int k = 0; k < 4; k++) {
            const int nb = min(max(valid - 4 * k, 0), 4);
            const uint32_t m = nb >= 4 ? 0xffffffffu : ((1u << (8 * nb)) - 1u);
            o[k] = align_bytes(d[k + 1], d[k], sh) & m;
        }
        v = make_uint4(o[0], o[1], o[2], o[3]);
    }
    return v;
}

// Sum over the 8 lanes 8g .. 8g+7, valid in lane 8g+7 (two quad butterflies,
// then lanes 4..7 of each 8 add lanes 0..3).
__device__ __forceinline__ uint32_t oct_sum_u32(uint32_t x) {
    x += (uint32_t)__builtin_amdgcn_update_dpp(0, (int)x, 0xB1, 0xf, 0xf, false);  // quad [1,0,3,2]
    x += (uint32_t)__builtin_amdgcn_update_dpp(0, (int)x, 0x4E, 0xf, 0xf, false);  // quad [2,3,0,1]
    x += (uint32_t)__builtin_amdgcn_update_dpp(0, (int)x, DPP_ROW_SHR4, 0xf, 0xf, false);
    return x;
}

template <bool VEC>
__global__ __launch_bounds__(256) void sat_rows(const uint8_t *__restrict__ img, int W, int H, size_t ip,
                                                SatWork wk) {
    const int q = (int)blockIdx.x % wk.nSeg, b = (int)blockIdx.x / wk.nSeg;  // 1-D grid: any height
    const int tid = threadIdx.x, w = tid >> 6, l = tid & 63;
    const int x = q * SAT_QW + 16 * l;
    const int y0 = b * SAT_BH + ROWS_PER_WAVE * w;
    uint4 px[ROWS_PER_WAVE];
#pragma unroll
    for (int r = 0; r < ROWS_PER_WAVE; r++) px[r] = load16<VEC>(img, ip, W, H, x, y0 + r);

    __shared__ uint32_t stot[2][SAT_BH][SAT_SPQ];   // strip sums of each row
    __shared__ uint32_t part[2][4][SAT_QW];         // [table][wave][column] 8-row sums
    __shared__ uint32_t wtot[2][4];                 // wavefront totals of the segment scan
    uint32_t cI[8];   // 16-bit column sums: cI[2k] columns 4k, 4k+2; cI[2k+1] 4k+1, 4k+3
    uint32_t cQ[16];
#pragma unroll
    for (int k = 0; k < 8; k++) cI[k] = 0;
#pragma unroll
    for (int k = 0; k < 16; k++) cQ[k] = 0;
#pragma unroll
    for (int r = 0; r < ROWS_PER_WAVE; r++) {
        const uint32_t d[4] = {px[r].x, px[r].y, px[r].z, px[r].w};
        uint32_t a = 0, qq = 0;
#pragma unroll
        for (int k = 0; k < 4; k++) {
            a = dot4u(d[k], 0x01010101u, a);
            qq = dot4u(d[k], d[k], qq);
            const uint32_t lo = d[k] & 0x00ff00ffu, hi = (d[k] >> 8) & 0x00ff00ffu;
            cI[2 * k] += lo;
            cI[2 * k + 1] += hi;
            const uint32_t v0 = lo & 0xffffu, v2 = lo >> 16, v1 = hi & 0xffffu, v3 = hi >> 16;
            cQ[4 * k + 0] = __umul24(v0, v0) + cQ[4 * k + 0];
            cQ[4 * k + 1] = __umul24(v1, v1) + cQ[4 * k + 1];
            cQ[4 * k + 2] = __umul24(v2, v2) + cQ[4 * k + 2];
            cQ[4 * k + 3] = __umul24(v3, v3) + cQ[4 * k + 3];
        }
        a = oct_sum_u32(a);
        qq = oct_sum_u32(qq);
        if ((l & 7) == 7) {
            stot[0][ROWS_PER_WAVE * w + r][l >> 3] = a;
            stot[1][ROWS_PER_WAVE * w + r][l >> 3] = qq;
        }
    }
    // this wavefront's 8-row column sums to LDS
#pragma unroll
    for (int k = 0; k < 4; k++) {
        *(uint4 *)&part[0][w][16 * l + 4 * k] =
            make_uint4(cI[2 * k] & 0xffffu, cI[2 * k + 1] & 0xffffu, cI[2 * k] >> 16, cI[2 * k + 1] >> 16);
        *(uint4 *)&part[1][w][16 * l + 4 * k] =
            make_uint4(cQ[4 * k], cQ[4 * k + 1], cQ[4 * k + 2], cQ[4 * k + 3]);
    }
    __syncthreads();

    // band column sums of columns 4*tid .. +3 of the segment -> running sums
    // along the segment (thread, then wavefront, then the wavefronts before)
    uint32_t c[2][4];
#pragma unroll
    for (int t = 0; t < 2; t++) {
        uint4 u = *(const uint4 *)&part[t][0][4 * tid];
#pragma unroll
        for (int ww = 1; ww < 4; ww++) {
            const uint4 v = *(const uint4 *)&part[t][ww][4 * tid];
            u.x += v.x;
            u.y += v.y;
            u.z += v.z;
            u.w += v.w;
        }
        c[t][0] = u.x;
        c[t][1] = c[t][0] + u.y;
        c[t][2] = c[t][1] + u.z;
        c[t][3] = c[t][2] + u.w;
    }
    uint32_t tot[2];
#pragma unroll
    for (int t = 0; t < 2; t++) {
        const uint32_t inc = wave_incl_scan_u32(c[t][3]);
        const uint32_t ex = inc - c[t][3];
#pragma unroll
        for (int k = 0; k < 4; k++) c[t][k] += ex;
        tot[t] = inc;
        if (l == 63) wtot[t][w] = inc;
    }
    __syncthreads();

    // band values: bandcol[t][b][x] = sum over the band's rows of the
    // segment-local row running sum at x
    const int xs = q * SAT_QW + 4 * tid;
#pragma unroll
    for (int t = 0; t < 2; t++) {
        uint32_t off = 0;
        for (int ww = 0; ww < w; ww++) off += wtot[t][ww];
        uint32_t *dst = wk.bandcol + ((size_t)t * wk.nBands + b) * W;
        const uint4 v = make_uint4(c[t][0] + off, c[t][1] + off, c[t][2] + off, c[t][3] + off);
        if (VEC && xs + 3 < W) {
            *(uint4 *)(dst + xs) = v;
        } else {
            if (xs < W) dst[xs] = v.x;
            if (xs + 1 < W) dst[xs + 1] = v.y;
            if (xs + 2 < W) dst[xs + 2] = v.z;
            if (xs + 3 < W) dst[xs + 3] = v.w;
        }
        if (tid == 255) wk.bandseg[((size_t)t * wk.nBands + b) * wk.nSeg + q] = tot[t] + off;
    }

    // row carries within the segment: for each row, the sum of the segment's
    // strips left of each strip, and the segment's row total
    if (tid < 2 * SAT_BH) {
        const int t = tid / SAT_BH, r = tid % SAT_BH, y = b * SAT_BH + r;
        if (y < H) {
            const size_t row = (size_t)t * H + y;
            uint32_t run = 0;
#pragma unroll
            for (int k = 0; k < SAT_SPQ; k++) {
                const int s = q * SAT_SPQ + k;
                if (s < wk.nStrips) wk.lrowl[row * wk.nStrips + s] = run;
                run += stot[t][r][k];
            }
            wk.segtot[row * wk.nSeg + q] = run;
        }
    }
}

// -------------------------------------------------------------- top pass --
// top[t][g][x] = sum over bands b' < b = g*SAT_SUB of (bandcol[t][b'][x] +
// the totals of band b' in the segments left of x's), i.e. the table value
// on row b*SAT_BH - 1 above downsweep tile row g.  A block takes 64 columns (inside one segment) of one table;
// its four wavefronts take a quarter of the bands each and meet in LDS.
// Lane k of a wavefront also carries the segment part of the k-th band of
// the current chunk, which is the same for every column of the block.
// Loads use clamped in-bounds indices so that a whole chunk issues at once.
constexpr int TOP_COLS = 64;
constexpr int TOP_CHUNK = 32;  // bands held in registers at a time

struct TopChunk {
    uint32_t v[TOP_CHUNK];  // bandcol of bands k0 .. k0+31 at this lane's column
    uint64_t sp;            // lane k: segment part of band k0 + k
};

__device__ __forceinline__ void top_load(TopChunk &ch, const uint32_t *__restrict__ bc,
                                         const uint32_t *__restrict__ bs, int W, int nB,
                                         int nSeg, int seg, int xc, int bfirst, int n, int lane) {
#pragma unroll
    for (int k = 0; k < TOP_CHUNK; k++) {
        const int bb = min(bfirst + k, nB - 1);
        const uint32_t u = bc[(size_t)bb * W + xc];
        ch.v[k] = k < n ? u : 0u;
    }
    const int bb = min(bfirst + lane, nB - 1);
    uint64_t sp = 0;
    for (int s0 = 0; s0 < seg; s0 += 4) {  // 4 loads in flight together
        uint32_t u4[4];
#pragma unroll
        for (int k = 0; k < 4; k++) u4[k] = bs[(size_t)bb * nSeg + min(s0 + k, seg - 1)];
#pragma unroll
        for (int k = 0; k < 4; k++) sp += s0 + k < seg ? u4[k] : 0u;
    }
    ch.sp = (lane < n && lane < TOP_CHUNK) ? sp : 0u;  // lanes past the chunk: next chunk's bands
}

// Row sums of the segments left of each segment, for one row rr of [2][H]
// (table, row): segpre[t][q][y] = sum of segtot[t][y][q'] over q' < q.
// Four segments at a time, every load of a batch issued before the first
// use; lanes take consecutive rows, so each store of a wavefront is 256
// contiguous bytes.
__device__ __forceinline__ void top_seg_prefix(const SatWork &wk, int H, int rr) {
    const int nSeg = wk.nSeg, t = rr >= H, y = rr - t * H;
    const uint32_t *__restrict__ st = wk.segtot + (size_t)rr * nSeg;
    uint32_t *__restrict__ sp = wk.segpre + (size_t)t * nSeg * H + y;
    uint32_t run = 0;
    for (int q0 = 0; q0 < nSeg; q0 += 4) {
        uint32_t v[4];
#pragma unroll
        for (int k = 0; k < 4; k++) v[k] = st[min(q0 + k, nSeg - 1)];
#pragma unroll
        for (int k = 0; k < 4; k++) {
            if (q0 + k < nSeg) sp[(size_t)(q0 + k) * H] = run;
            run += v[k];
        }
    }
}

__global__ __launch_bounds__(256) void sat_top(int W, int H, SatWork wk) {
    const int colBlocks = (W + TOP_COLS - 1) / TOP_COLS;
    if ((int)blockIdx.x >= 2 * colBlocks) {  // block-uniform: the row blocks
        const int rr = ((int)blockIdx.x - 2 * colBlocks) * 256 + (int)threadIdx.x;
        if (rr < 2 * H) top_seg_prefix(wk, H, rr);
        return;
    }
    const int t = blockIdx.x / colBlocks, cb = blockIdx.x % colBlocks;
    const int tid = threadIdx.x, c = tid & (TOP_COLS - 1), qtr = tid / TOP_COLS;
    const int x = cb * TOP_COLS + c, xc = min(x, W - 1);
    const int seg = cb * TOP_COLS / SAT_QW;
    const int nB = wk.nBands, nSeg = wk.nSeg;
    const uint32_t *__restrict__ bc = wk.bandcol + (size_t)t * nB * W;
    const uint32_t *__restrict__ bs = wk.bandseg + (size_t)t * nB * nSeg;
    uint64_t *__restrict__ top = wk.top + (size_t)t * ((nB + SAT_SUB - 1) / SAT_SUB) * W;
    const int per = (nB + 3) / 4, b0 = qtr * per;
    const int nb = min(per, max(nB - b0, 0));  // bands of this quarter

    __shared__ uint64_t qs[4][TOP_COLS];
    __shared__ uint64_t qseg[4];
    TopChunk ch;
    uint64_t colrun = 0, segrun = 0;
    for (int k0 = 0; k0 < per; k0 += TOP_CHUNK) {  // block-uniform trip count
        top_load(ch, bc, bs, W, nB, nSeg, seg, xc, b0 + k0, nb - k0, c);
#pragma unroll
        for (int k = 0; k < TOP_CHUNK; k++) colrun += ch.v[k];
        segrun += wave_incl_scan_u64(ch.sp);  // lane 63 ends with the chunk total
    }
    qs[qtr][c] = colrun;
    if (c == 63) qseg[qtr] = segrun;
    __syncthreads();
    uint64_t base = 0;
    for (int q2 = 0; q2 < qtr; q2++) base += qs[q2][c] + qseg[q2];
    for (int k0 = 0; k0 < per; k0 += TOP_CHUNK) {
        if (per > TOP_CHUNK)  // more than one chunk: reload (one chunk stays in registers)
            top_load(ch, bc, bs, W, nB, nSeg, seg, xc, b0 + k0, nb - k0, c);
        const uint64_t spi = wave_incl_scan_u64(ch.sp);
        const uint64_t spx = spi - ch.sp;  // lane k: segment part of the chunk's bands before k
#pragma unroll
        for (int k = 0; k < TOP_CHUNK; k++) {
            const uint64_t sk = ((uint64_t)(uint32_t)__builtin_amdgcn_readlane((int)(spx >> 32), k) << 32) |
                                (uint32_t)__builtin_amdgcn_readlane((int)(uint32_t)spx, k);
            const int bb = b0 + k0 + k;
            if (k < nb - k0 && x < W && bb % SAT_SUB == 0) top[(size_t)(bb / SAT_SUB) * W + x] = base + sk;
            base += ch.v[k];
        }
        base += (uint64_t)(((uint64_t)(uint32_t)__builtin_amdgcn_readlane((int)(spi >> 32), 63) << 32) |
                           (uint32_t)__builtin_amdgcn_readlane((int)(uint32_t)spi, 63));
    }
}

// ------------------------------------------------------------- downsweep --
// A workgroup owns a tile of SAT_SW columns x SAT_SUB bands and walks its
// bands in order; each band is written by the 4 wavefronts, WAVE_ROWS rows
// each, and the next band's bytes and row carries are loaded before the
// current band is stored.  Lane l of every wavefront owns columns
// x = 128*s + 2l and x + 1, so each 16-byte store of a row lands next to its
// neighbours' (1 KB per wavefront).

// Bytes of one band for one wavefront, read from clamped addresses and
// masked where they are used.
template <bool VEC>
struct BandIn {
    uint32_t px[WAVE_ROWS];
    __device__ __forceinline__ void load(const uint8_t *img, size_t ip, int W, int H, int x, int y0) {
#pragma unroll
        for (int r = 0; r < WAVE_ROWS; r++) px[r] = load2_raw<VEC>(img, ip, W, H, x, y0 + r);
    }
};

// Left carries of every row a wavefront writes in its tile, one per lane:
// lane 32t + 8k + r holds, for table t, the row sum of all columns left of
// the strip on row r of the wavefront's part of band k (the segment-local
// carry plus the segments to the left).  Loaded and added once, before the
// first band: within the band loop a use of a just-loaded value would wait
// for every load issued before it, the next band's bytes included.
static_assert(2 * SAT_SUB * WAVE_ROWS <= 64, "one left carry per lane");
__device__ __forceinline__ uint32_t tile_left_carries(const SatWork &wk, int H, int s, int ytile, int w,
                                                      int l) {
    const int t = l >> 5, k = (l / WAVE_ROWS) % SAT_SUB, r = l % WAVE_ROWS;
    const size_t y = (size_t)min(ytile + k * SAT_BH + w * WAVE_ROWS + r, H - 1);
    const size_t seg = s / SAT_SPQ;
    return wk.lrowl[((size_t)t * H + y) * wk.nStrips + s] + wk.segpre[((size_t)t * wk.nSeg + seg) * H + y];
}

template <bool VEC>
__global__ __launch_bounds__(256) void sat_downsweep(const uint8_t *__restrict__ img, int W, int H, size_t ip,
                                                     SatWork wk, int64_t *__restrict__ S,
                                                     int64_t *__restrict__ Q) {
    const int nTy = (wk.nBands + SAT_SUB - 1) / SAT_SUB;
    const int tix = xcd_tile((int)blockIdx.x, wk.nStrips * nTy);
    if (tix < 0) return;
    const int s = tix % wk.nStrips, g = tix / wk.nStrips;
    const int tid = threadIdx.x, w = tid >> 6, l = tid & 63;
    const int x = s * SAT_SW + 2 * l;
    const int ytile = g * SAT_SUB * SAT_BH;

    // column carries: the table values on the row above the tile
    uint64_t s1a, s1b, s2a, s2b;
    {
        const uint64_t *tp1 = wk.top + (size_t)g * W;
        const uint64_t *tp2 = wk.top + ((size_t)nTy + g) * W;
        const int xa = min(x, W - 1), xb = min(x + 1, W - 1);
        s1a = tp1[xa];
        s1b = tp1[xb];
        s2a = tp2[xa];
        s2b = tp2[xb];
    }
    const uint32_t lcar = tile_left_carries(wk, H, s, ytile, w, l);
    BandIn<VEC> cur, nxt;
    cur.load(img, ip, W, H, x, ytile + w * WAVE_ROWS);

    __shared__ uint64_t part[2][4][4][64];  // [band parity][wave][value][lane]
    typedef long long v2l __attribute__((ext_vector_type(2)));
    const bool pair = VEC && x + 1 < W;
    for (int k = 0; k < SAT_SUB; k++) {
        const int yb = ytile + k * SAT_BH;
        if (yb >= H) break;  // workgroup-uniform
        const int y0 = yb + w * WAVE_ROWS;

        // uint32 row running sums R(x,y) = sum over columns 0..x of row y
        // (left carry + wavefront exclusive scan + own pixels), and their
        // column totals over the wavefront's rows
        uint32_t R1a[WAVE_ROWS], R1b[WAVE_ROWS], R2a[WAVE_ROWS], R2b[WAVE_ROWS];
        uint32_t c1a = 0, c1b = 0;  // 8 rows of R1 < 8 * 66051 * 255 < 2^32
        uint64_t c2a = 0, c2b = 0;
#pragma unroll
        for (int r = 0; r < WAVE_ROWS; r++) {
            const uint32_t pv = mask2(cur.px[r], W, H, x, y0 + r);
            const uint32_t b0 = pv & 0xffu, b1 = pv >> 8;
            const uint32_t p1 = b0 + b1, p2 = b0 * b0 + b1 * b1;
            const uint32_t e1 = wave_incl_scan_u32(p1) - p1 +
                                (uint32_t)__builtin_amdgcn_readlane((int)lcar, WAVE_ROWS * k + r);
            const uint32_t e2 = wave_incl_scan_u32(p2) - p2 +
                                (uint32_t)__builtin_amdgcn_readlane((int)lcar, 32 + WAVE_ROWS * k + r);
            R1a[r] = e1 + b0;
            R1b[r] = e1 + p1;
            R2a[r] = e2 + b0 * b0;
            R2b[r] = e2 + p2;
            c1a += R1a[r];
            c1b += R1b[r];
            c2a += R2a[r];
            c2b += R2b[r];
        }
        // the next band's inputs are in flight while this band is stored
        if (k + 1 < SAT_SUB) nxt.load(img, ip, W, H, x, y0 + SAT_BH);

        const int pb = k & 1;
        part[pb][w][0][l] = c1a;
        part[pb][w][1][l] = c1b;
        part[pb][w][2][l] = c2a;
        part[pb][w][3][l] = c2b;
        __syncthreads();
        uint64_t t1a = s1a, t1b = s1b, t2a = s2a, t2b = s2b;
#pragma unroll
        for (int ww = 0; ww < 4; ww++) {
            const uint64_t u1a = part[pb][ww][0][l], u1b = part[pb][ww][1][l];
            const uint64_t u2a = part[pb][ww][2][l], u2b = part[pb][ww][3][l];
            if (ww < w) {
                t1a += u1a;
                t1b += u1b;
                t2a += u2a;
                t2b += u2b;
            }
            s1a += u1a;  // carries into the next band
            s1b += u1b;
            s2a += u2a;
            s2b += u2b;
        }

        // running column sums, written row by row
#pragma unroll
        for (int r = 0; r < WAVE_ROWS; r++) {
            const int y = y0 + r;
            if (y >= H) break;
            t1a += R1a[r];
            t1b += R1b[r];
            t2a += R2a[r];
            t2b += R2b[r];
            int64_t *srow = S + (size_t)y * W + x;
            int64_t *qrow = Q + (size_t)y * W + x;
            // ordinary (temporal) stores: on this part they sustain ~12% more
            // write bandwidth than nontemporal ones for this row-run pattern
            if (pair) {
                *(v2l *)srow = v2l{(long long)t1a, (long long)t1b};
                *(v2l *)qrow = v2l{(long long)t2a, (long long)t2b};
            } else {
                if (x < W) {
                    srow[0] = (int64_t)t1a;
                    qrow[0] = (int64_t)t2a;
                }
                if (x + 1 < W) {
                    srow[1] = (int64_t)t1b;
                    qrow[1] = (int64_t)t2b;
                }
            }
        }
        cur = nxt;
    }
}


// ----------------------------------------------------------- single pass --
// One kernel: a workgroup takes a ticket (tiles in band-major order), loads
// its 128 x 128 tile once, publishes its row sums and column sums, reads
// what it needs of earlier tiles' published words, and writes its part of S
// and Q.  Every published value is a 64-bit word value << 2 | state, stored
// and read with single-copy-atomic relaxed accesses, so no fence orders data
// against a flag.
//   row word (tile, table, row):   1 = the tile's row sum, 2 = that plus the
//                                  sum of the row left of the tile
//   column word (tile, table, x):  1 = V(x) = sum over the tile's rows of the
//                                  row running sum at x (from the image's
//                                  left edge), 2 = the table value on the
//                                  tile's last row
// A tile waits only for words of tiles with smaller tickets, whose
// workgroups are already running: the row words of state 1 are published
// right after a tile's loads, the column words of state 1 after its row
// look-back, which itself waits only for state-1 row words.  Each wait gives
// up after SAT_FSPIN polls and raises ctl[3].
constexpr int SAT_FSPIN = 1 << 22;
constexpr int SAT_FBATCH = 8;

__device__ __forceinline__ uint64_t word_load(const uint64_t *p) {
    return __hip_atomic_load(p, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
__device__ __forceinline__ void word_store(uint64_t *p, uint64_t v) {
    __hip_atomic_store(p, v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

// Sum of the values of the words at p - stride, p - 2*stride, ... (n of
// them), stopping after the first one of state 2; waits for words of state 0.
__device__ __forceinline__ uint64_t look_back(const uint64_t *p, size_t stride, int n,
                                              uint32_t *ctl) {
    uint64_t acc = 0;
    for (int i0 = 0; i0 < n; i0 += SAT_FBATCH) {
        uint64_t v[SAT_FBATCH];
#pragma unroll
        for (int k = 0; k < SAT_FBATCH; k++)
            v[k] = i0 + k < n ? word_load(p - (size_t)(i0 + k + 1) * stride) : 2ull;
        bool done = false;
#pragma unroll
        for (int k = 0; k < SAT_FBATCH; k++) {
            if (!done) {
                int spins = 0;
                while ((v[k] & 3) == 0) {
                    if (++spins > SAT_FSPIN) {
                        __hip_atomic_store(ctl + 3, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
                        break;
                    }
                    __builtin_amdgcn_s_sleep(1);
                    v[k] = word_load(p - (size_t)(i0 + k + 1) * stride);
                }
                acc += v[k] >> 2;
                done = (v[k] & 3) == 2;
            }
        }
        if (done) break;
    }
    return acc;
}

template <bool VEC>
__global__ __launch_bounds__(256) void sat_fused(const uint8_t *__restrict__ img, int W, int H, size_t ip,
                                                 SatState fs, int nS, int nTiles,
                                                 int64_t *__restrict__ S, int64_t *__restrict__ Q) {
    constexpr int TR = SAT_BH * SAT_FSUB;  // tile rows
    __shared__ int sh_tile;
    __shared__ uint32_t sh_epoch;
    __shared__ uint32_t colp[4][2][SAT_FW];  // per wavefront: pixel column sums of its rows
    __shared__ uint32_t rtS[2][TR];          // row sums inside the tile
    __shared__ uint32_t lrowS[2][TR];        // row sums left of the tile
    __shared__ uint32_t csS[2][SAT_FW];      // running sums along the tile of the column sums
    __shared__ uint64_t topS[2][SAT_FW];     // table values on the row above the tile
    __shared__ uint64_t llS[4];              // per wavefront: sum of its lanes' left carries
    __shared__ uint32_t wtS[4];              // per wavefront: column-sum scan totals
    __shared__ uint64_t part[2][4][4][64];
    const int tid = threadIdx.x, w = tid >> 6, l = tid & 63;
    if (tid == 0) {
        sh_tile = (int)__hip_atomic_fetch_add(fs.ctl, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        sh_epoch = __hip_atomic_load(fs.ctl + 2, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    }
    __syncthreads();
    const int tile = sh_tile;
    const uint32_t epoch = sh_epoch;
    if (tile >= nTiles) {  // counters not reset by the previous call: flag it, touch nothing
        if (tid == 0) __hip_atomic_store(fs.ctl + 3, 2u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        return;
    }
    const int gi = tile / nS, j = tile % nS;
    uint64_t *words = fs.words + (size_t)(epoch & 1) * fs.capTiles * SAT_FWORDS;
    {   // this workgroup's share of the next call's words
        uint64_t *nxt = fs.words + (size_t)((epoch & 1) ^ 1) * fs.capTiles * SAT_FWORDS;
        const size_t total = (size_t)fs.capTiles * SAT_FWORDS;
        const size_t per = (total + nTiles - 1) / nTiles;
        const size_t b = (size_t)tile * per, e = min(total, b + per);
        for (size_t i = b + tid; i < e; i += 256) nxt[i] = 0;
    }
    uint64_t *my = words + (size_t)tile * SAT_FWORDS;

    const int x = j * SAT_FW + 2 * l;
    const int ytile = gi * TR;

    // ---- the tile's own sums, band by band: row sums (published as soon as
    // a band is done) and column sums of the pixels
    const int tb = tid >> 7, ix = tid & 127;  // (table, row or column) of this thread's words
    uint32_t c1a = 0, c1b = 0, c2a = 0, c2b = 0;
#pragma unroll
    for (int k = 0; k < SAT_FSUB; k++) {
        uint32_t px[WAVE_ROWS];
#pragma unroll
        for (int r = 0; r < WAVE_ROWS; r++)
            px[r] = load2<VEC>(img, ip, W, H, x, ytile + SAT_BH * k + WAVE_ROWS * w + r);
#pragma unroll
        for (int r = 0; r < WAVE_ROWS; r++) {
            const uint32_t b0 = px[r] & 0xffu, b1 = (px[r] >> 8) & 0xffu;
            const uint32_t q0 = b0 * b0, q1 = b1 * b1;
            const uint32_t t1 = wave_sum_u32(b0 + b1), t2 = wave_sum_u32(q0 + q1);
            if (l == 0) {
                rtS[0][SAT_BH * k + WAVE_ROWS * w + r] = t1;
                rtS[1][SAT_BH * k + WAVE_ROWS * w + r] = t2;
            }
            c1a += b0;
            c1b += b1;
            c2a += q0;
            c2b += q1;
        }
    }
    *(uint2 *)&colp[w][0][2 * l] = make_uint2(c1a, c1b);
    *(uint2 *)&colp[w][1][2 * l] = make_uint2(c2a, c2b);
    __syncthreads();
    {
        word_store(my + tb * TR + ix, (uint64_t)rtS[tb][ix] << 2 | 1u);
        const uint32_t cs = colp[0][tb][ix] + colp[1][tb][ix] + colp[2][tb][ix] + colp[3][tb][ix];
        const uint32_t inc = wave_incl_scan_u32(cs);
        if (l == 63) wtS[w] = inc;
        __syncthreads();
        csS[tb][ix] = inc + ((w & 1) ? wtS[w - 1] : 0u);
    }

    // ---- row look-back: the sum of each row left of the tile
    {
        const uint32_t rt = rtS[tb][ix];
        const uint32_t lc = (uint32_t)look_back(my + tb * TR + ix, SAT_FWORDS, j, fs.ctl);
        word_store(my + tb * TR + ix, (uint64_t)(lc + rt) << 2 | 2u);
        lrowS[tb][ix] = lc;
        const uint64_t s = wave_incl_scan_u64((uint64_t)lc);
        if (l == 63) llS[w] = s;
    }
    __syncthreads();
    // ---- column look-back: the table value above the tile
    {
        const uint64_t LL = llS[2 * tb] + llS[2 * tb + 1];
        const uint64_t V = (uint64_t)csS[tb][ix] + LL;
        uint64_t *cw = my + 2 * TR + tb * SAT_FW + ix;
        word_store(cw, V << 2 | 1u);
        const uint64_t C = look_back(cw, (size_t)nS * SAT_FWORDS, gi, fs.ctl);
        word_store(cw, (C + V) << 2 | 2u);
        topS[tb][ix] = C;
    }
    __syncthreads();

    // ---- the tile's rows of S and Q, band by band (as the downsweep; the
    // bytes are read again, mostly from L2, the next band's in flight while
    // the current one is stored)
    uint64_t s1a = topS[0][2 * l], s1b = topS[0][2 * l + 1];
    uint64_t s2a = topS[1][2 * l], s2b = topS[1][2 * l + 1];
    typedef long long v2l __attribute__((ext_vector_type(2)));
    const bool pair = VEC && x + 1 < W;
    uint32_t pc[WAVE_ROWS], pn[WAVE_ROWS];
#pragma unroll
    for (int r = 0; r < WAVE_ROWS; r++) pc[r] = load2<VEC>(img, ip, W, H, x, ytile + WAVE_ROWS * w + r);
#pragma unroll
    for (int k = 0; k < SAT_FSUB; k++) {
        const int yb = ytile + SAT_BH * k;
        if (yb >= H) break;  // workgroup-uniform
        const int y0 = yb + WAVE_ROWS * w;
        const int rr = SAT_BH * k + WAVE_ROWS * w + (l & (WAVE_ROWS - 1));
        const uint32_t lc1 = lrowS[0][rr], lc2 = lrowS[1][rr];
        uint32_t R1a[WAVE_ROWS], R1b[WAVE_ROWS], R2a[WAVE_ROWS], R2b[WAVE_ROWS];
        uint64_t d1a = 0, d1b = 0, d2a = 0, d2b = 0;
#pragma unroll
        for (int r = 0; r < WAVE_ROWS; r++) {
            const uint32_t b0 = pc[r] & 0xffu, b1 = (pc[r] >> 8) & 0xffu;
            const uint32_t p1 = b0 + b1, p2 = b0 * b0 + b1 * b1;
            const uint32_t e1 = wave_incl_scan_u32(p1) - p1 +
                                (uint32_t)__builtin_amdgcn_readlane((int)lc1, r);
            const uint32_t e2 = wave_incl_scan_u32(p2) - p2 +
                                (uint32_t)__builtin_amdgcn_readlane((int)lc2, r);
            R1a[r] = e1 + b0;
            R1b[r] = e1 + p1;
            R2a[r] = e2 + b0 * b0;
            R2b[r] = e2 + p2;
            d1a += R1a[r];
            d1b += R1b[r];
            d2a += R2a[r];
            d2b += R2b[r];
        }
        if (k + 1 < SAT_FSUB) {
#pragma unroll
            for (int r = 0; r < WAVE_ROWS; r++) pn[r] = load2<VEC>(img, ip, W, H, x, y0 + SAT_BH + r);
        }
        const int pb = k & 1;
        part[pb][w][0][l] = d1a;
        part[pb][w][1][l] = d1b;
        part[pb][w][2][l] = d2a;
        part[pb][w][3][l] = d2b;
        __syncthreads();
        uint64_t t1a = s1a, t1b = s1b, t2a = s2a, t2b = s2b;
#pragma unroll
        for (int ww = 0; ww < 4; ww++) {
            const uint64_t u1a = part[pb][ww][0][l], u1b = part[pb][ww][1][l];
            const uint64_t u2a = part[pb][ww][2][l], u2b = part[pb][ww][3][l];
            if (ww < w) {
                t1a += u1a;
                t1b += u1b;
                t2a += u2a;
                t2b += u2b;
            }
            s1a += u1a;
            s1b += u1b;
            s2a += u2a;
            s2b += u2b;
        }
#pragma unroll
        for (int r = 0; r < WAVE_ROWS; r++) {
            const int y = y0 + r;
            if (y >= H) break;
            t1a += R1a[r];
            t1b += R1b[r];
            t2a += R2a[r];
            t2b += R2b[r];
            int64_t *srow = S + (size_t)y * W + x;
            int64_t *qrow = Q + (size_t)y * W + x;
            if (pair) {
                *(v2l *)srow = v2l{(long long)t1a, (long long)t1b};
                *(v2l *)qrow = v2l{(long long)t2a, (long long)t2b};
            } else {
                if (x < W) {
                    srow[0] = (int64_t)t1a;
                    qrow[0] = (int64_t)t2a;
                }
                if (x + 1 < W) {
                    srow[1] = (int64_t)t1b;
                    qrow[1] = (int64_t)t2b;
                }
            }
        }
#pragma unroll
        for (int r = 0; r < WAVE_ROWS; r++) pc[r] = pn[r];
    }

    // ---- the last tile to finish resets the counters for the next call
    if (tid == 0) {
        const uint32_t d = __hip_atomic_fetch_add(fs.ctl + 1, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        if (d == (uint32_t)nTiles - 1) {
            __hip_atomic_store(fs.ctl, 0u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
            __hip_atomic_store(fs.ctl + 1, 0u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
            __hip_atomic_store(fs.ctl + 2, epoch + 1, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        }
    }
}

}  // namespace

size_t sat_work_bytes(int W, int H) {
    const size_t nS = (W + SAT_SW - 1) / SAT_SW, nB = (H + SAT_BH - 1) / SAT_BH;
    const size_t nQ = (W + SAT_QW - 1) / SAT_QW;
    size_t bytes = 0;
    auto add = [&](size_t n) { bytes += (n + 255) & ~(size_t)255; };
    add(2 * (size_t)H * nS * 4);  // lrowl
    add(2 * (size_t)H * nQ * 4);  // segtot
    add(2 * (size_t)H * nQ * 4);  // segpre
    add(2 * nB * W * 4);          // bandcol
    add(2 * nB * nQ * 4);         // bandseg
    add(2 * ((nB + SAT_SUB - 1) / SAT_SUB) * W * 8);  // top
    return bytes;
}

SatWork sat_work_carve(void *base, int W, int H) {
    SatWork wk;
    wk.nStrips = (W + SAT_SW - 1) / SAT_SW;
    wk.nBands = (H + SAT_BH - 1) / SAT_BH;
    wk.nSeg = (W + SAT_QW - 1) / SAT_QW;
    const size_t nS = wk.nStrips, nB = wk.nBands, nQ = wk.nSeg;
    char *p = (char *)base;
    auto take = [&](size_t n) { char *q = p; p += (n + 255) & ~(size_t)255; return (void *)q; };
    wk.lrowl = (uint32_t *)take(2 * (size_t)H * nS * 4);
    wk.segtot = (uint32_t *)take(2 * (size_t)H * nQ * 4);
    wk.segpre = (uint32_t *)take(2 * (size_t)H * nQ * 4);
    wk.bandcol = (uint32_t *)take(2 * nB * W * 4);
    wk.bandseg = (uint32_t *)take(2 * nB * nQ * 4);
    wk.top = (uint64_t *)take(2 * ((nB + SAT_SUB - 1) / SAT_SUB) * W * 8);
    return wk;
}

size_t sat_state_bytes(int W, int H) {
    const size_t nS = (W + SAT_FW - 1) / SAT_FW;
    const size_t nG = (H + SAT_BH * SAT_FSUB - 1) / (SAT_BH * SAT_FSUB);
    return 256 + 2 * nS * nG * SAT_FWORDS * sizeof(uint64_t);
}

SatState sat_state_view(void *base, size_t bytes) {
    SatState fs;
    fs.ctl = (uint32_t *)base;
    fs.words = (uint64_t *)((char *)base + 256);
    fs.capTiles = (int)((bytes - 256) / (2 * SAT_FWORDS * sizeof(uint64_t)));
    return fs;
}

hipError_t sat_build_launch(const uint8_t *img, int W, int H, size_t ip, int64_t *S, int64_t *Q,
                            const SatWork &wk, const SatState &fs, hipStream_t st) {
    if (fs.ctl) {
        const int nS = (W + SAT_FW - 1) / SAT_FW;
        const int nG = (H + SAT_BH * SAT_FSUB - 1) / (SAT_BH * SAT_FSUB);
        const int nTiles = nS * nG;
        if (nTiles > fs.capTiles) return hipErrorInvalidValue;
        const bool vec = (W % 2 == 0) && (ip % 2 == 0) && (((uintptr_t)img & 1) == 0) &&
                         (((uintptr_t)S & 15) == 0) && (((uintptr_t)Q & 15) == 0);
        if (vec)
            hipLaunchKernelGGL(sat_fused<true>, dim3(nTiles), dim3(256), 0, st, img, W, H, ip, fs, nS,
                               nTiles, S, Q);
        else
            hipLaunchKernelGGL(sat_fused<false>, dim3(nTiles), dim3(256), 0, st, img, W, H, ip, fs, nS,
                               nTiles, S, Q);
        return hipGetLastError();
    }
    // aligned 16-byte image rows (and band rows) for the row pass; even
    // widths and 16-byte table rows for the paired loads and stores of the
    // downsweep
    const bool rvec = (W % 16 == 0) && (ip % 16 == 0) && (((uintptr_t)img & 15) == 0);
    const bool dvec = (W % 2 == 0) && (ip % 2 == 0) && (((uintptr_t)img & 1) == 0) &&
                      (((uintptr_t)S & 15) == 0) && (((uintptr_t)Q & 15) == 0);
    dim3 block(256);
    dim3 rgrid(wk.nSeg * wk.nBands);
    if (rvec)
        hipLaunchKernelGGL(sat_rows<true>, rgrid, block, 0, st, img, W, H, ip, wk);
    else
        hipLaunchKernelGGL(sat_rows<false>, rgrid, block, 0, st, img, W, H, ip, wk);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
    const int rowBlocks = (2 * H + 255) / 256;
    hipLaunchKernelGGL(sat_top, dim3(2 * ((W + TOP_COLS - 1) / TOP_COLS) + rowBlocks), block, 0, st, W,
                       H, wk);
    e = hipGetLastError();
    if (e != hipSuccess) return e;
    dim3 grid(xcd_grid(wk.nStrips * ((wk.nBands + SAT_SUB - 1) / SAT_SUB)));
    if (dvec)
        hipLaunchKernelGGL(sat_downsweep<true>, grid, block, 0, st, img, W, H, ip, wk, S, Q);
    else
        hipLaunchKernelGGL(sat_downsweep<false>, grid, block, 0, st, img, W, H, ip, wk, S, Q);
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
