// Summed-area tables S (of I) and Q (of I^2) of an 8-bit image, int64,
// inclusive: The CUDA Handbook ch. 15, section 15.8 "The Denominator: Summed
// Area Tables" -- table definition, width analysis (uint32 row running sums,
// int64 table) and the separable build (a row scan, then a column scan).
//
// MI355X design: two passes with no waiting between workgroups, over tiles
// of SAT_SW columns x SAT_TR rows (strip s, tile row g).
//   1. sat_tiles: tile workgroups read their tile once and write its column
//      sums (colsum) and total (btot); row workgroups read 4 whole rows and
//      write each row's exclusive running sum of strip sums (lcar: the row's
//      sum left of each strip).
//   2. sat_downsweep: a workgroup owns a tile.  Its prologue forms the table
//      value on the row above the tile: the column sums of the tiles above
//      (each wavefront a quarter of them, met in LDS), running along the
//      strip, plus the totals of the tiles above and to the left.  It then
//      re-reads its bytes band by band (the next band's loads in flight while
//      the current one is stored); the uint32 row running sums (left carry +
//      wavefront DPP scan) stay in registers and are added down each column
//      into int64 running sums.  S and Q are written once, lane l owning
//      columns 2l and 2l+1 so one store instruction covers 1 KB of a row.
// The row running sums never go to HBM: the full-size traffic is two reads of
// the image and one write of each table; the tile sums are about 1 MB.
#include "ncc_internal.h"

namespace ncc {

namespace {

constexpr int WAVE_ROWS = SAT_BH / 4;  // downsweep rows per wavefront
constexpr int PRO_BATCH = 8;           // downsweep prologue: tile rows per wavefront per batch
constexpr int PRO_BATCH_B = 2;         // ... block-total loads per thread per batch

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

// ------------------------------------------------------------- tile pass --
// Sum over the 8 lanes 8g .. 8g+7, valid in lane 8g+7 (two quad butterflies,
// then lanes 4..7 of each 8 add lanes 0..3).
__device__ __forceinline__ uint32_t oct_sum_u32(uint32_t x) {
    x += (uint32_t)__builtin_amdgcn_update_dpp(0, (int)x, 0xB1, 0xf, 0xf, false);  // quad [1,0,3,2]
    x += (uint32_t)__builtin_amdgcn_update_dpp(0, (int)x, 0x4E, 0xf, 0xf, false);  // quad [2,3,0,1]
    x += (uint32_t)__builtin_amdgcn_update_dpp(0, (int)x, DPP_ROW_SHR4, 0xf, 0xf, false);
    return x;
}

// Bytes x .. x+15 of row y, zero outside the image.  VEC: W, ip and x
// multiples of 16, img 16-byte aligned.  The zeroing is a mask, not a
// branch: a conditional assignment compiles to a branch that waits for its
// load, which would serialise the tile's loads.
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

// v_perm_b32: byte i of the result is byte sel_i of the 8 bytes hi:lo.
__device__ __forceinline__ uint32_t perm(uint32_t hi, uint32_t lo, uint32_t sel) {
    return __builtin_amdgcn_perm(hi, lo, sel);
}

// Two kinds of workgroup in one launch (tiles, and groups of 4 rows; when the
// tile rows divide evenly over the XCDs, each XCD gets the jobs of its tile
// rows, see sat_tiles):
//   tile (strip s, tile row g): thread (rg, cg) = (tid >> 3, tid & 7) holds
//     rows 4rg .. 4rg+3 and columns 16cg .. 16cg+15 of the tile.  Writes the
//     tile's column sums colsum[t][g][x] and its total btot[t][g][s].  Column
//     sums of 4 rows come from 4x4 byte transposes (v_perm) and dot4 of each
//     column's 4 bytes with ones and with itself; neighbouring row groups
//     add through DPP and the remaining 16 meet in LDS.
//   rows (rows 4b .. 4b+3, every column): thread tid holds columns
//     16tid .. 16tid+15 of a 4096-column chunk; per row, strip sums (8 lanes
//     each) and their exclusive running sum along the row: lcar[t][y][s], the
//     row's sum over the columns left of strip s.
// Every write covers whole 128-byte lines.  uint32 bounds: a tile column of
// 128 squares, a tile total <= 128 * 128 * 255^2 < 2^31, a row prefix
// <= W * 255^2 (the width bound).
constexpr int ROW_CHUNK = 4096;  // columns of a row workgroup per step

template <bool VEC>
__device__ __forceinline__ void tile_sums(const uint8_t *__restrict__ img, int W, int H, size_t ip,
                                          const SatWork &wk, int s, int g, uint32_t *lds) {
    const int tid = threadIdx.x, w = tid >> 6, l = tid & 63;
    const int cg = tid & 7, rg = tid >> 3;
    const int x = s * SAT_SW + 16 * cg, y0 = g * SAT_TR + 4 * rg;
    uint4 px[4];
#pragma unroll
    for (int r = 0; r < 4; r++) px[r] = load16<VEC>(img, ip, W, H, x, y0 + r);
    uint32_t(*red)[16][SAT_SW] = (uint32_t(*)[16][SAT_SW])lds;  // [table][row-group pair][column]
    uint32_t *btw = lds + 2 * 16 * SAT_SW;                        // [wave] half-tile totals
    // dword k of the 4 rows, transposed so that word c holds column 4k+c of
    // rows 0..3; then lanes l and l^8 (row groups 2j, 2j+1) add, and the
    // even row group writes the 4 columns (one dword group at a time, so few
    // sums are live at once)
#pragma unroll
    for (int k = 0; k < 4; k++) {
        const uint32_t d0 = ((const uint32_t *)&px[0])[k], d1 = ((const uint32_t *)&px[1])[k];
        const uint32_t d2 = ((const uint32_t *)&px[2])[k], d3 = ((const uint32_t *)&px[3])[k];
        const uint32_t e0 = perm(d1, d0, 0x06020400u), e1 = perm(d1, d0, 0x07030501u);
        const uint32_t e2 = perm(d3, d2, 0x06020400u), e3 = perm(d3, d2, 0x07030501u);
        const uint32_t tc[4] = {perm(e2, e0, 0x05040100u), perm(e3, e1, 0x05040100u), perm(e2, e0, 0x07060302u),
                                perm(e3, e1, 0x07060302u)};
        uint32_t ci[4], cq[4];
#pragma unroll
        for (int c = 0; c < 4; c++) {
            ci[c] = dot4u(tc[c], 0x01010101u, 0);
            cq[c] = dot4u(tc[c], tc[c], 0);
            ci[c] += (uint32_t)__builtin_amdgcn_update_dpp(0, (int)ci[c], DPP_ROW_ROR8, 0xf, 0xf, false);
            cq[c] += (uint32_t)__builtin_amdgcn_update_dpp(0, (int)cq[c], DPP_ROW_ROR8, 0xf, 0xf, false);
        }
        if ((rg & 1) == 0) {
            *(uint4 *)&red[0][rg >> 1][16 * cg + 4 * k] = make_uint4(ci[0], ci[1], ci[2], ci[3]);
            *(uint4 *)&red[1][rg >> 1][16 * cg + 4 * k] = make_uint4(cq[0], cq[1], cq[2], cq[3]);
        }
    }
    __syncthreads();
    // thread (table, column): the tile's column sum; the tile total per
    // wavefront (two per table)
    const int t = tid >> 7, c = tid & (SAT_SW - 1);
    uint32_t cs = 0;
#pragma unroll
    for (int r = 0; r < 16; r++) cs += red[t][r][c];
    wk.colsum[((size_t)t * wk.nG + g) * ((size_t)wk.nS * SAT_SW) + (size_t)s * SAT_SW + c] = cs;
    const uint32_t tot = wave_sum_u32(cs);
    if (l == 0) btw[w] = tot;
    __syncthreads();
    if (tid < 2) wk.btot[((size_t)tid * wk.nG + g) * wk.nS4 + s] = btw[2 * tid] + btw[2 * tid + 1];
}

template <bool VEC>
__device__ __forceinline__ void row_prefixes(const uint8_t *__restrict__ img, int W, int H, size_t ip,
                                             const SatWork &wk, int b, uint32_t *lds) {
    const int tid = threadIdx.x;
    const int y0 = 4 * b;
    uint32_t(*ss)[4][32] = (uint32_t(*)[4][32])lds;  // [table][row][strip of the chunk]
    uint32_t *carry = lds + 2 * 4 * 32;              // [table][row]
    // scan lane (t, r, j): table t, row r, strip j of the chunk
    const int st = tid >> 7, sr = (tid >> 5) & 3, sj = tid & 31;
    if (tid < 8) carry[tid] = 0;
    for (int q = 0; q * ROW_CHUNK < W; q++) {  // block-uniform
        const int x = q * ROW_CHUNK + 16 * tid;
        uint4 px[4];
#pragma unroll
        for (int r = 0; r < 4; r++) px[r] = load16<VEC>(img, ip, W, H, x, y0 + r);
#pragma unroll
        for (int r = 0; r < 4; r++) {
            const uint32_t d[4] = {px[r].x, px[r].y, px[r].z, px[r].w};
            uint32_t a = 0, qq = 0;
#pragma unroll
            for (int k = 0; k < 4; k++) {
                a = dot4u(d[k], 0x01010101u, a);
                qq = dot4u(d[k], d[k], qq);
            }
            a = oct_sum_u32(a);
            qq = oct_sum_u32(qq);
            if ((tid & 7) == 7) {
                ss[0][r][tid >> 3] = a;
                ss[1][r][tid >> 3] = qq;
            }
        }
        __syncthreads();
        const uint32_t v = ss[st][sr][sj];
        uint32_t inc = wave_incl_scan_u32(v);
        inc -= (tid & 32) ? (uint32_t)__builtin_amdgcn_readlane((int)inc, 31) : 0u;  // two 32-lane scans
        const uint32_t base = carry[st * 4 + sr];
        const int strip = q * (ROW_CHUNK / SAT_SW) + sj, y = y0 + sr;
        if (strip < wk.nS && y < H) wk.lcar[((size_t)st * H + y) * wk.nS + strip] = base + inc - v;
        __syncthreads();
        if (sj == 31) carry[st * 4 + sr] = base + inc;
        __syncthreads();
    }
}

template <bool VEC>
__global__ __launch_bounds__(256) void sat_tiles(const uint8_t *__restrict__ img, int W, int H, size_t ip,
                                                 SatWork wk) {
    __shared__ uint32_t lds[2 * 16 * SAT_SW + 4];
    if (wk.nG % NUM_XCD == 0) {  // uniform
        // The jobs of tile row g go to XCD g % NUM_XCD (blockIdx % NUM_XCD),
        // the XCD whose downsweep workgroups take that tile row: per XCD
        // first the tiles of its tile rows, then their 4-row groups (4096^2:
        // 50.3 against 50.6 us per build with tiles and row groups spread
        // over the XCDs).
        const int x8 = (int)blockIdx.x % NUM_XCD, i8 = (int)blockIdx.x / NUM_XCD;
        const int rows8 = wk.nG / NUM_XCD;  // tile rows per XCD
        if (i8 < rows8 * wk.nS) {  // block-uniform
            tile_sums<VEC>(img, W, H, ip, wk, i8 % wk.nS, x8 + NUM_XCD * (i8 / wk.nS), lds);
        } else {
            const int j = i8 - rows8 * wk.nS;
            const int g = x8 + NUM_XCD * (j / (SAT_TR / 4));
            const int b = g * (SAT_TR / 4) + j % (SAT_TR / 4);  // rows 4b .. 4b+3
            if (b < (H + 3) / 4) row_prefixes<VEC>(img, W, H, ip, wk, b, lds);
        }
    } else {  // blocks [0, nS*nG) are tiles, the rest 4-row groups
        const int ntiles = wk.nS * wk.nG;
        if ((int)blockIdx.x < ntiles)
            tile_sums<VEC>(img, W, H, ip, wk, (int)blockIdx.x % wk.nS, (int)blockIdx.x / wk.nS, lds);
        else
            row_prefixes<VEC>(img, W, H, ip, wk, (int)blockIdx.x - ntiles, lds);
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
// the strip on row r of the wavefront's part of band k (rows past the image
// read the last row; their values are not used).  Loaded once, before the
// first band: within the band loop a use of a just-loaded value would wait
// for every load issued before it, the next band's bytes included.
static_assert(2 * SAT_SUB * WAVE_ROWS <= 64, "one left carry per lane");
__device__ __forceinline__ uint32_t tile_left_carries(const SatWork &wk, int H, int s, int ytile, int w, int l) {
    const int t = l >> 5, k = (l / WAVE_ROWS) % SAT_SUB, r = l % WAVE_ROWS;
    const size_t y = (size_t)min(ytile + k * SAT_BH + w * WAVE_ROWS + r, H - 1);
    return wk.lcar[((size_t)t * H + y) * wk.nS + s];
}

template <bool VEC>
__global__ __launch_bounds__(256) void sat_downsweep(const uint8_t *__restrict__ img, int W, int H, size_t ip,
                                                     SatWork wk, int64_t *__restrict__ S,
                                                     int64_t *__restrict__ Q) {
    const int nS = wk.nS, nG = wk.nG;
    // When the tile rows divide evenly over the XCDs, they are interleaved:
    // the workgroups that go to XCD x (blockIdx % NUM_XCD) take tile rows x,
    // x + NUM_XCD, ..., each with all its strips.  On this part that drains
    // the tables' rows faster than each XCD taking a contiguous band of tile
    // rows (4096^2: 50.5 against 50.8 us per build; strips per XCD instead of
    // rows: 59.8 us).  Otherwise each XCD takes a contiguous range of tiles,
    // which keeps the XCDs' shares equal for any shape.
    int s, g;
    if (nG % NUM_XCD == 0) {  // uniform
        const int x8 = (int)blockIdx.x % NUM_XCD, i8 = (int)blockIdx.x / NUM_XCD;
        s = i8 % nS;
        g = x8 + NUM_XCD * (i8 / nS);
    } else {
        const int tix = xcd_tile((int)blockIdx.x, nS * nG);
        if (tix < 0) return;
        s = tix % nS;
        g = tix / nS;
    }
    const int tid = threadIdx.x, w = tid >> 6, l = tid & 63;
    const int x = s * SAT_SW + 2 * l;
    const int ytile = g * SAT_TR;

    // Table values on the row above the tile, for this lane's columns x and
    // x + 1 (column c = x - s*SAT_SW):
    //   sum over tile rows g' < g of colsum[g'] at columns s*SAT_SW .. x
    //   + sum over g' < g, s' < s of btot[g'][s'].
    // Wavefront w adds the column sums of tile rows w, w+4, ...; the block
    // totals are spread over all 256 threads (four per 16-byte load).
    // Every load of a batch is issued before the first use (clamped
    // indices, masked sums): a use waits for all loads issued before it.
    const size_t pcs = (size_t)nS * SAT_SW;
    const int wu = __builtin_amdgcn_readfirstlane(w);
    uint64_t a0 = 0, a1 = 0, q0 = 0, q1 = 0;  // [table][column parity]
    for (int i0 = wu; i0 < g; i0 += 4 * PRO_BATCH) {  // wavefront-uniform
        uint2 u[PRO_BATCH], v[PRO_BATCH];
#pragma unroll
        for (int k = 0; k < PRO_BATCH; k++) {
            const size_t gg = (size_t)min(i0 + 4 * k, g - 1);
            u[k] = *(const uint2 *)(wk.colsum + gg * pcs + x);
            v[k] = *(const uint2 *)(wk.colsum + ((size_t)nG + gg) * pcs + x);
        }
#pragma unroll
        for (int k = 0; k < PRO_BATCH; k++) {
            const bool in = i0 + 4 * k < g;
            a0 += in ? u[k].x : 0u;
            a1 += in ? u[k].y : 0u;
            q0 += in ? v[k].x : 0u;
            q1 += in ? v[k].y : 0u;
        }
    }
    uint64_t bl = 0;  // block totals above-left, table tid >> 7
    {
        const int sq = (s + 3) >> 2, n = g * sq, bt = tid >> 7;
        for (int i0 = 0; i0 < n; i0 += 128 * PRO_BATCH_B) {  // workgroup-uniform
            uint4 u[PRO_BATCH_B];
            int qk[PRO_BATCH_B];
#pragma unroll
            for (int k = 0; k < PRO_BATCH_B; k++) {
                const int i = min(i0 + (tid & 127) + 128 * k, n - 1), gg = i / sq;
                qk[k] = i - gg * sq;
                u[k] = *(const uint4 *)(wk.btot + ((size_t)bt * nG + gg) * wk.nS4 + 4 * qk[k]);
            }
#pragma unroll
            for (int k = 0; k < PRO_BATCH_B; k++) {
                const bool in = i0 + (tid & 127) + 128 * k < n;
                const int c0 = 4 * qk[k];
                bl += (in && c0 + 0 < s ? u[k].x : 0u) + (uint64_t)(in && c0 + 1 < s ? u[k].y : 0u) +
                      (uint64_t)(in && c0 + 2 < s ? u[k].z : 0u) + (uint64_t)(in && c0 + 3 < s ? u[k].w : 0u);
            }
        }
    }
    const uint32_t lcar = tile_left_carries(wk, H, s, ytile, w, l);
    BandIn<VEC> cur, nxt;
    cur.load(img, ip, W, H, x, ytile + w * WAVE_ROWS);
    __shared__ uint64_t pro[4][4][64];  // [wave][table*2 + parity][lane] partial column sums
    __shared__ uint64_t blw[4];           // [wave] partial block totals
    pro[w][0][l] = a0;
    pro[w][1][l] = a1;
    pro[w][2][l] = q0;
    pro[w][3][l] = q1;
    {
        const uint64_t sc = wave_incl_scan_u64(bl);
        if (l == 63) blw[w] = sc;
    }
    __syncthreads();
    uint64_t s1a, s1b, s2a, s2b;
    {
        uint64_t c[4];
#pragma unroll
        for (int j = 0; j < 4; j++) c[j] = pro[0][j][l] + pro[1][j][l] + pro[2][j][l] + pro[3][j][l];
        const uint64_t i1 = wave_incl_scan_u64(c[0] + c[1]), i2 = wave_incl_scan_u64(c[2] + c[3]);
        const uint64_t L1 = blw[0] + blw[1], L2 = blw[2] + blw[3];
        s1b = i1 + L1;
        s1a = s1b - c[1];
        s2b = i2 + L2;
        s2a = s2b - c[3];
    }
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
            // S with ordinary stores, Q with nontemporal ones: on this part a
            // mix of the two kinds sustains more write bandwidth than either
            // kind alone for this row-run pattern (4096^2 build: 52.3 us all
            // ordinary, 59.7 us all nontemporal, 50.7 us mixed)
            if (pair) {
                *(v2l *)srow = v2l{(long long)t1a, (long long)t1b};
                __builtin_nontemporal_store(v2l{(long long)t2a, (long long)t2b}, (v2l *)qrow);
            } else {
                if (x < W) {
                    srow[0] = (int64_t)t1a;
                    __builtin_nontemporal_store((long long)t2a, (long long *)qrow);
                }
                if (x + 1 < W) {
                    srow[1] = (int64_t)t1b;
                    __builtin_nontemporal_store((long long)t2b, (long long *)(qrow + 1));
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
//   state 3 (either kind):         the value rests on a wait that gave up;
//                                  every tile that reads it fails as well
// A tile waits only for words of tiles with smaller tickets, whose
// workgroups are already running: the row words of state 1 are published
// right after a tile's loads, the column words of state 1 after its row
// look-back, which itself waits only for state-1 row words.  Each wait gives
// up after fs.spin polls; a workgroup that gave up writes INT64_MIN for its
// tile and reports the failure (ctl[3] and the pinned host word).
constexpr int SAT_FBATCH = 8;

// A failure of this call: kind 1 = a wait gave up, 2 = a ticket past the
// last tile (counters left by a call that never finished).
__device__ __forceinline__ void report_failure(const SatState &fs, uint32_t kind) {
    __hip_atomic_store(fs.ctl + 3, kind, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    __hip_atomic_store(fs.hostflag, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_SYSTEM);
}

__device__ __forceinline__ uint64_t word_load(const uint64_t *p) {
    return __hip_atomic_load(p, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
__device__ __forceinline__ void word_store(uint64_t *p, uint64_t v) {
    __hip_atomic_store(p, v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

// Sum of the values of the words at p - stride, p - 2*stride, ... (n of
// them), stopping after the first one of state 2; waits for words of state 0
// (at most fs.spin polls each).  `failed` is set when a wait gives up or a
// word of state 3 (published by a tile that failed) is met: the sum is then
// not valid.
__device__ __forceinline__ uint64_t look_back(const uint64_t *p, size_t stride, int n,
                                              const SatState &fs, bool &failed) {
    uint64_t acc = 0;
    failed = false;
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
                    if (++spins > fs.spin) {
                        report_failure(fs, 1u);
                        failed = true;
                        break;
                    }
                    __builtin_amdgcn_s_sleep(1);
                    v[k] = word_load(p - (size_t)(i0 + k + 1) * stride);
                }
                if ((v[k] & 3) == 3) failed = true;
                acc += v[k] >> 2;
                done = failed || (v[k] & 3) == 2;
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
    __shared__ int sh_fail;  // a wait of this workgroup gave up
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
        sh_fail = 0;
    }
    __syncthreads();
    const int tile = sh_tile;
    const uint32_t epoch = sh_epoch;
    if (tile >= nTiles) {  // counters not reset by the previous call: flag it, touch nothing
        if (tid == 0) report_failure(fs, 2u);
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
        bool rf;
        const uint32_t lc = (uint32_t)look_back(my + tb * TR + ix, SAT_FWORDS, j, fs, rf);
        if (rf) sh_fail = 1;
        word_store(my + tb * TR + ix, (uint64_t)(lc + rt) << 2 | (rf ? 3u : 2u));
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
        const bool tf = sh_fail != 0;  // V rests on row sums left of the tile that failed
        word_store(cw, V << 2 | (tf ? 3u : 1u));
        bool cf;
        const uint64_t C = look_back(cw, (size_t)nS * SAT_FWORDS, gi, fs, cf);
        if (cf) sh_fail = 1;
        word_store(cw, (C + V) << 2 | (tf || cf ? 3u : 2u));
        topS[tb][ix] = C;
    }
    __syncthreads();

    // ---- the tile's rows of S and Q, band by band (as the downsweep; the
    // bytes are read again, mostly from L2, the next band's in flight while
    // the current one is stored)
    const bool failed = sh_fail != 0;  // this tile's carries are not valid: INT64_MIN
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
            const long long o1a = failed ? INT64_MIN : (long long)t1a, o1b = failed ? INT64_MIN : (long long)t1b;
            const long long o2a = failed ? INT64_MIN : (long long)t2a, o2b = failed ? INT64_MIN : (long long)t2b;
            if (pair) {
                *(v2l *)srow = v2l{o1a, o1b};
                *(v2l *)qrow = v2l{o2a, o2b};
            } else {
                if (x < W) {
                    srow[0] = o1a;
                    qrow[0] = o2a;
                }
                if (x + 1 < W) {
                    srow[1] = o1b;
                    qrow[1] = o2b;
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

// Build scratch of the two-pass build for an H x W image: colsum
// [2][nG][nS*SAT_SW], btot [2][nG][nS4] (nS4 = nS rounded up to 4) and lcar
// [2][H][nS], all uint32 (about 0.07 bytes per pixel).
size_t sat_work_bytes(int W, int H) {
    const size_t nS = (W + SAT_SW - 1) / SAT_SW, nG = (H + SAT_TR - 1) / SAT_TR, nS4 = (nS + 3) & ~(size_t)3;
    size_t bytes = 0;
    auto add = [&](size_t n) { bytes += (n + 255) & ~(size_t)255; };
    add(2 * nG * nS * SAT_SW * 4);  // colsum
    add(2 * nG * nS4 * 4);          // btot
    add(2 * (size_t)H * nS * 4);    // lcar
    return bytes;
}

SatWork sat_work_carve(void *base, int W, int H) {
    SatWork wk;
    wk.nS = (W + SAT_SW - 1) / SAT_SW;
    wk.nG = (H + SAT_TR - 1) / SAT_TR;
    wk.nS4 = (wk.nS + 3) & ~3;
    const size_t nS = wk.nS, nG = wk.nG;
    char *p = (char *)base;
    auto take = [&](size_t n) { char *q = p; p += (n + 255) & ~(size_t)255; return (void *)q; };
    wk.colsum = (uint32_t *)take(2 * nG * nS * SAT_SW * 4);
    wk.btot = (uint32_t *)take(2 * nG * (size_t)wk.nS4 * 4);
    wk.lcar = (uint32_t *)take(2 * (size_t)H * nS * 4);
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
    fs.hostflag = nullptr;
    fs.spin = 0;
    return fs;
}

namespace {
__global__ void sat_state_poison(uint32_t *ctl) {
    if (threadIdx.x == 0) __hip_atomic_store(ctl, 1u << 30, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
}  // namespace

hipError_t sat_state_poison_launch(const SatState &fs, hipStream_t st) {
    hipLaunchKernelGGL(sat_state_poison, dim3(1), dim3(64), 0, st, fs.ctl);
    return hipGetLastError();
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
    // aligned 16-byte image rows for the tile pass; even widths and 16-byte
    // table rows for the paired loads and stores of the downsweep
    const bool rvec = (W % 16 == 0) && (ip % 16 == 0) && (((uintptr_t)img & 15) == 0);
    const bool dvec = (W % 2 == 0) && (ip % 2 == 0) && (((uintptr_t)img & 1) == 0) &&
                      (((uintptr_t)S & 15) == 0) && (((uintptr_t)Q & 15) == 0);
    dim3 block(256);
    // per XCD its tile rows' tiles and 4-row groups when the tile rows divide
    // evenly over the XCDs, else every tile and then every 4-row group
    const unsigned blocks = wk.nG % NUM_XCD == 0
                                ? (unsigned)wk.nG * (unsigned)(wk.nS + SAT_TR / 4)
                                : (unsigned)wk.nS * (unsigned)wk.nG + (unsigned)((H + 3) / 4);
    if (rvec)
        hipLaunchKernelGGL(sat_tiles<true>, dim3(blocks), block, 0, st, img, W, H, ip, wk);
    else
        hipLaunchKernelGGL(sat_tiles<false>, dim3(blocks), block, 0, st, img, W, H, ip, wk);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
    dim3 grid(xcd_grid(wk.nS * wk.nG));  // nS * nG when nG % NUM_XCD == 0
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
