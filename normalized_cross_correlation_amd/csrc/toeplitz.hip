// Single-template correlation on the int8 matrix cores, as a banded
// Toeplitz product.
//
// What is computed is the per-window accumulation of The CUDA Handbook
// ch. 15 "Image in shared memory" (SumI, SumISq, SumIT over a wT x hT
// template, then the coefficient).  SumIT and SumI are accumulated per
// window, as that section does, on the matrix cores; the sum of squares is
// read off running column sums of the strip's row window sums of squares
// (the four-corner rule of section 15.8 on the strip's own summed-area table,
// the horizontal difference taken first).  Every sum is an exact integer, so
// the route does not change a single output bit.
//
// SumIT as a matrix product.  For template row j and the 16 positions
// x0 + 16n + m (m = 0..15) of one 16-column block n, row j contributes
//   sum_{u=0}^{31} T[j][u - m] * I[y + j][x0 + 16n + u]
// (T[j][c] = 0 outside 0 <= c < wT): a 16 x 32 band matrix of the template
// row times 32 image bytes.  With the 16 template rows stacked along k,
//   C[m][n] = SumIT(x0 + 16n + m, y) = sum_k A[m][k] B[k][n],
//   A[m][(j,u)] = T[j][u - m],  B[(j,u)][n] = I[y + j][x0 + 16n + u],
// K = 16 rows x 32 = 512 k-slots, 8 steps of v_mfma_i32_16x16x64_i8 per 256
// positions of one output row; half of A is structural zeros.  The
// instruction multiplies signed bytes, so both sides move by 128 (T' = T - 128
// inside the band, 0 outside it; I' = I - 128, the byte I^0x80 read as signed)
// and C = sum over the window of I'T'.  Numerator and variance do not change
// when every pixel or every template byte moves by the same amount, so with
// D = sum of I' over the window, sT = sum of T' and V = sum of I'^2
//   num  = K*SumIT - SumI*SumT = K*C - D*sT,
//   varI = K*SumISq - SumI^2  = K*V - D^2
// exactly (24-bit multiplies modulo 2^32; |num|, varI < 2^31).
//
// Operand layout (16x16x64, as the bank kernel uses it): lane 16g + m of A
// holds 16 k-slots of row m, lane 16g + n of B the same 16 k-slots of column
// n, lane 16g + n of the result rows 4g .. 4g+3 of column n.  Step s, lane
// group g covers template row j = s + 8(g >> 1), bytes u = 16(g & 1) .. +15.
// So lane (g, n) holds, at output row y, image row y + s + 8(g >> 1) at
// bytes 16(n + (g & 1)) .. +15 of its wavefront's columns: a ring of 8 image
// rows per lane, one new 16-byte read per output row.  Its results are the
// four adjacent positions x0 + 16n + 4g .. +3.
//
// Window sums.  D is the same product with an all-ones template, whose band
// matrix does not depend on the template row: one constant A operand.  The
// strip's first row takes the 8-step chain; each next row slides it,
// D(y + 1) = D(y) + rs(y + 16) - rs(y) (rs = row window sums of I'), in two
// steps whose A operand is the band negated on lane groups 0 and 1: a ring
// slot holds rows r and r + 8 on the two halves, so one step adds
// rs(r + 8) - rs(r).  V: the lane's row sums of I'^2 at its 4 positions
// (signed dot4 for the first, then the squares that enter and leave as the
// window slides 1 byte), added down a ring of the last 16 rows; the running
// value is -K*V, so that -varI = D^2 - K*V is one multiply-add.  The plain
// sums, when asked for, follow from these: SumI = D + 128K,
// SumISq = V + 256D + 16384K, SumIT = C + 128(D + sT) + 16384K.
//
// A workgroup (4 wavefronts, 256 columns each) owns 1024 output columns and
// RS output rows (32; 16 for small launches and for calls that write the
// sums planes).  The strip's RS + 16 image rows (rows + halo) are read once
// with one round of 16-byte loads and staged in LDS as I^0x80: the rows the
// first RS/4 output rows read before the loop, the rest (whose loads arrive
// meanwhile) at output row RS/4.  Software pipeline: iteration y reads row y + 1's LDS
// data and issues its chains, while finishing row y.  Coefficient rows go
// out through an LDS buffer of 4 rows: after every 4th row (a barrier) each
// wavefront stores one whole 1024-column row of the group, 4 KB in four
// 1 KB instructions, and a second barrier frees the buffer.  With the sums
// planes the results instead go through a lane permutation, and each
// wavefront stores 1 KB of every row and plane.
#include "ncc_internal.h"


namespace ncc {

namespace {

typedef int v4i __attribute__((ext_vector_type(4)));
typedef float f4u __attribute__((ext_vector_type(4), aligned(4)));
typedef int i4u __attribute__((ext_vector_type(4), aligned(4)));

constexpr int TZ_HT = 16;              // template rows
constexpr int TZ_WAVES = 4;
constexpr int TZ_NT = TZ_WAVES * 64;   // lanes per workgroup
constexpr int TZ_NC = TZ_WAVES * 256;  // output columns per workgroup
constexpr int TZ_CH = TZ_NC / 16 + 1;  // 16-byte chunks staged per row (tile + halo)
constexpr int TZ_PITCH = TZ_CH * 4 + 4;  // dwords per LDS row
// Strip of RS output rows: RS + 16 staged image rows (the strip and its
// halo), read with LOADS 16-byte loads per lane; BUFROWS also holds the tail
// of the last round of loads (never read), so that every load is stored
// without a branch (a guarded store lets the compiler sink its load into the
// branch and wait for it there).
template <int RS>
struct TzStrip {
    static constexpr int ROWS = RS + 16;
    static constexpr int LOADS = (ROWS * TZ_CH + TZ_NT - 1) / TZ_NT;
    static constexpr int BUFROWS = (LOADS * TZ_NT + TZ_CH - 1) / TZ_CH;
};

// Byte q (0..19) of the 5-dword little-endian sequence d, as a signed byte.
template <int Q>
__device__ __forceinline__ int sbyte_at(const uint32_t (&d)[5]) {
    return (int)(int8_t)(uint8_t)(d[Q >> 2] >> (8 * (Q & 3)));
}

// Row window sums of I'^2 (signed bytes) at the four columns c0 .. c0+3
// whose bytes start at d[0] (byte 0 = column c0): the first window by signed
// dot4, then each next one by adding the square that enters and removing the
// one that leaves (b'^2 - b^2 = (b' - b)(b' + b)).  Each is at most
// 16 * 128^2.
template <int WT>
__device__ __forceinline__ void row_sq4(const uint32_t (&d)[5], int (&q)[4]) {
    constexpr int WT4 = (WT + 3) / 4;
    int s2 = 0;
#pragma unroll
    for (int k = 0; k < WT4; k++) {
        const uint32_t v = (k == WT4 - 1) ? (d[k] & byte_mask(WT - 4 * k)) : d[k];
        s2 = __builtin_amdgcn_sdot4((int)v, (int)v, s2, false);
    }
    q[0] = s2;
#pragma unroll
    for (int t = 0; t < 3; t++) {
        int bo, bn;
        // byte t leaves, byte t + WT enters
        switch (t) {
            case 0: bo = sbyte_at<0>(d); bn = sbyte_at<WT>(d); break;
            case 1: bo = sbyte_at<1>(d); bn = sbyte_at<WT + 1>(d); break;
            default: bo = sbyte_at<2>(d); bn = sbyte_at<WT + 2>(d); break;
        }
        q[t + 1] = q[t] + __mul24(bn - bo, bn + bo);
    }
}

// v[i] = the value v[i] of the lane whose byte address (lane * 4) is pidx.
template <class V>
__device__ __forceinline__ void to_lane_order(V (&v)[4], int pidx) {
#pragma unroll
    for (int i = 0; i < 4; i++) {
        int x;
        __builtin_memcpy(&x, &v[i], 4);
        x = __builtin_amdgcn_ds_bpermute(pidx, x);
        __builtin_memcpy(&v[i], &x, 4);
    }
}

// Two workgroups (8 wavefronts) per CU: up to 256 registers per lane.
template <int WT, int RS, int ALIGN, bool WSUM>
__global__ __launch_bounds__(TZ_NT, 2) void corr_toeplitz(CorrArgs a, int t, int ntx, int nty) {
    static_assert(RS % 16 == 0, "strips of whole 16-row groups");
    constexpr int NG = RS / 16;           // output-row groups of 16
    constexpr int TZ_LOADS = TzStrip<RS>::LOADS;
    constexpr int TZ_BUFROWS = TzStrip<RS>::BUFROWS;
    // The loads are staged in two parts: the first UA (every row that rows
    // 0 .. YB-1 read) before the loop, the rest at row YB, so that the later
    // rows' loads arrive while the first rows are computed.  Row y reads
    // image rows up to y + 17 (its successor's window and B operands).
    constexpr int YB = RS / 4;
    constexpr int UA = ((YB + 17) * TZ_CH + TZ_NT - 1) / TZ_NT;
    static_assert(UA <= TZ_LOADS && UA * TZ_NT / TZ_CH >= YB + 17, "first part holds rows 0 .. YB+16");
    constexpr int K = WT * TZ_HT;
    __shared__ uint32_t buf[TZ_BUFROWS][TZ_PITCH];  // image rows y0 .. y0 + TZ_ROWS - 1 (+ tail)
    __shared__ uint32_t tE[TZ_HT][16];      // template row j at bytes 16 .. 16+wT-1 of 64, as T^0x80
    __shared__ int tsum[TZ_WAVES][2];       // per wavefront: sums of T' and T'^2
    // Coefficient rows on their way out (no sums planes): slot [r][c][18g + n]
    // holds, for row r of a group of 4, wavefront c's lane (g, n) results
    // (positions 16n + 4g .. +3 of its 256 columns).  18, not 16, slots per
    // lane group keep both the writes and the transposed reads free of bank
    // conflicts.
    __shared__ float4 obuf[WSUM ? 1 : 4][TZ_WAVES][72];

    const int tix = xcd_tile((int)blockIdx.x, ntx * nty);
    if (tix < 0) return;
    const int tid = threadIdx.x, w = tid >> 6, l = tid & 63;
    const int g = l >> 4, n = l & 15;
    const int X0 = (tix % ntx) * TZ_NC, y0 = (tix / ntx) * RS;
    const int rowsOut = min(RS, a.Ho - y0);

    // template bytes, loaded first from clamped indices (no branch)
    const uint8_t *T = a.tpl + (size_t)t * TZ_HT * WT;
    uint32_t tb[4];
#pragma unroll
    for (int b = 0; b < 4; b++) {
        const int c = 4 * (tid % 16) + b - 16;
        tb[b] = T[(tid / 16) * WT + min(max(c, 0), WT - 1)];
    }
    // ---- the strip's image rows, loaded all at once (one round of loads)
    // and then staged in LDS; chunk i of the staged block is row i / TZ_CH,
    // bytes 16 * (i % TZ_CH)
    uint4 pre[TZ_LOADS];
#pragma unroll
    for (int u = 0; u < TZ_LOADS; u++) {
        const int i = tid + u * TZ_NT;
        const int r = i / TZ_CH, c = i % TZ_CH;
        const int y = y0 + r, x = X0 + 16 * c;
        if (ALIGN == 16) {
            // W, ip % 16 == 0: clamped in-bounds addresses, no branch.  Bytes
            // of rows past H or columns past W feed only positions past Ho
            // or Wo, which are not stored, so what they hold is immaterial.
            pre[u] = *(const uint4 *)(a.img + (size_t)min(y, a.H - 1) * a.ip + min(x, a.W - 16));
        } else {
            pre[u] = load16_any(a.img, a.ip, a.W, a.H, x, y);
        }
    }
    // template rows with a 16-byte zero margin on both sides, as signed
    // bytes: lane (j, dw) builds dword dw of row j from its four bytes
    {
        const int j = tid / 16, dw = tid % 16;
        uint32_t v = 0;
#pragma unroll
        for (int b = 0; b < 4; b++) {
            const int c = 4 * dw + b - 16;
            v |= (c >= 0 && c < WT) ? (tb[b] ^ 0x80u) << (8 * b) : 0u;
        }
        tE[j][dw] = v;
        const uint32_t p1 = wave_incl_scan_u32((uint32_t)__builtin_amdgcn_sdot4((int)v, 0x01010101, 0, false));
        const uint32_t p2 = wave_incl_scan_u32((uint32_t)__builtin_amdgcn_sdot4((int)v, (int)v, 0, false));
        if (l == 63) {
            tsum[w][0] = (int)p1;
            tsum[w][1] = (int)p2;
        }
    }
    auto stage = [&](int u) {  // load u into LDS, as I^0x80
        const int i = tid + u * TZ_NT;
        const int r = i / TZ_CH, c = i % TZ_CH;
        const uint4 v = pre[u];
        *(uint4 *)&buf[r][4 * c] = make_uint4(v.x ^ 0x80808080u, v.y ^ 0x80808080u,
                                              v.z ^ 0x80808080u, v.w ^ 0x80808080u);
    };
#pragma unroll
    for (int u = 0; u < UA; u++) stage(u);
    __syncthreads();

    // ---- A operands: step s, lane (g, m = n): template row s + 8(g >> 1),
    // bytes 16(g & 1) - m .. +15 of the row (zero outside it)
    v4i atp[8];
    {
        const int st = 16 + 16 * (g & 1) - n;  // 1 .. 32
        const int dw0 = st >> 2;
        const uint32_t sh = (uint32_t)(st & 3);
#pragma unroll
        for (int s = 0; s < 8; s++) {
            const uint32_t *p = &tE[s + 8 * (g >> 1)][dw0];
            const uint32_t e0 = p[0], e1 = p[1], e2 = p[2], e3 = p[3];
            const uint32_t e4 = p[4];
            atp[s] = (v4i){(int)align_bytes(e1, e0, sh), (int)align_bytes(e2, e1, sh),
                           (int)align_bytes(e3, e2, sh), (int)align_bytes(e4, e3, sh)};
        }
    }
    // template sums: each lane's tE dword (T' = T - 128, zeros around it),
    // summed over the wavefront and then over the 4 wavefronts
    const int sT1 = tsum[0][0] + tsum[1][0] + tsum[2][0] + tsum[3][0];
    const int sT2 = tsum[0][1] + tsum[1][1] + tsum[2][1] + tsum[3][1];
    // varT = K * sum T'^2 - (sum T')^2 (shift-invariant; <= K^2 * 127.5^2 < 2^31).
    // The epilogue forms -varI (one multiply-add) and multiplies it by -varT:
    // the same float product, since negation is exact (both are integers
    // >= 1 unless num = 0, where the coefficient is 0 either way).
    const float nvarTf = -(float)((unsigned)K * (unsigned)sT2 - (unsigned)(sT1 * sT1));
    const int nsT = -sT1;

    // ---- lane geometry
    const int wcol = 256 * w;                      // wavefront's first column (rel. X0)
    const int bch = wcol / 4 + 4 * (n + (g & 1));  // dword of the lane's B chunk
    const int roff = 8 * (g >> 1);                 // B rows: y + s + roff
    const int hdw = wcol / 4 + 4 * n + g;          // dword of the lane's window bytes
    // The lane's results are positions x0 + 16n + 4g .. +3 (x0 = X0 + wcol):
    // consecutive lanes 64 bytes apart.  Before the stores, lane 4n + g takes
    // lane 16g + n's four values through the LDS crossbar, so lane l holds
    // positions x0 + 4l .. +3 and each store instruction writes 1 KB in lane
    // order.
    const int pidx = 4 * (16 * (l & 3) + (l >> 2));  // ds_bpermute byte address of the source lane
    const int c0 = X0 + wcol + 4 * l;              // the lane's first position after that
    const bool wfull = X0 + wcol >= a.xs && X0 + wcol + 256 <= a.Wo;  // wave-uniform

    auto bload = [&](int r) -> v4i {  // image row r (rel. y0) of the lane's B chunk (I^0x80)
        const uint4 v = *(const uint4 *)&buf[r][bch];
        return (v4i){(int)v.x, (int)v.y, (int)v.z, (int)v.w};
    };
    auto hload = [&](int r, uint32_t (&d)[5]) {  // window bytes of image row r
        const uint32_t *p = &buf[r][hdw];
#pragma unroll
        for (int k = 0; k < 5; k++) d[k] = p[k];
    };
    auto hsq = [&](int r, int (&q)[4]) {  // row sums of I'^2 of image row r
        uint32_t d[5];
        hload(r, d);
        row_sq4<WT>(d, q);
    };

    // B ring: slot r & 7 holds image row r + roff
    v4i bring[8];
#pragma unroll
    for (int s = 0; s < 8; s++) bring[s] = bload(s + roff);
    // D (the window sum of I') on the matrix cores too: the band matrix of
    // an all-ones template is the same for every template row, so one A
    // operand serves all 8 steps (lane (g, m): byte i is 1 iff
    // 0 <= 16(g & 1) + i - m < wT)
    v4i aone;
#pragma unroll
    for (int k = 0; k < 4; k++) {
        uint32_t v = 0;
#pragma unroll
        for (int b = 0; b < 4; b++) {
            const int c = 16 * (g & 1) + 4 * k + b - n;
            v |= (c >= 0 && c < WT) ? (1u << (8 * b)) : 0u;
        }
        aone[k] = (int)v;
    }
    // The same band, negated on lane groups 0 and 1 (bytes 0xff = -1), for
    // the window sum's slide from row to row: with B from one ring slot
    // (image row r on groups 0, 1 and row r + 8 on groups 2, 3) one step adds
    // rs(r + 8) - rs(r), rs = the row window sums of I'.
    v4i adiff;
#pragma unroll
    for (int k = 0; k < 4; k++) adiff[k] = g < 2 ? (int)((uint32_t)aone[k] * 0xffu) : aone[k];
    // ring of row sums of I'^2: slot r & 15 holds image row r.  The running
    // value is NV = -K * V (V the window's sum of I'^2), so that -varI =
    // D^2 + NV is one multiply-add; output row 0 starts from image rows
    // 0 .. 14 (|NV| <= K^2 * 128^2 <= 2^30).
    int ring[4][16], NV[4] = {0, 0, 0, 0};
#pragma unroll
    for (int r = 0; r < 15; r++) {
        int q[4];
        hsq(r, q);
#pragma unroll
        for (int i = 0; i < 4; i++) {
            ring[i][r] = q[i];
            NV[i] -= K * q[i];
        }
    }
#pragma unroll
    for (int i = 0; i < 4; i++) ring[i][15] = 0;

    const size_t plane = a.oplane;
    float *outp = a.coef + (size_t)t * plane + (size_t)y0 * a.op;
    int32_t *sp0 = WSUM ? a.sums + (size_t)y0 * a.op : nullptr;
    int32_t *sp1 = WSUM ? sp0 + plane : nullptr;
    int32_t *sp2 = WSUM ? a.sums + (size_t)(2 + t) * plane + (size_t)y0 * a.op : nullptr;
    // The lane's pointers to its output of column c0 in the next row (xs is
    // the column of a view's first output), advanced by op each row: one
    // 64-bit add per row and plane.
    const size_t op = a.op;
    float *orp = outp + (c0 - a.xs);
    int32_t *s0p = WSUM ? sp0 + (c0 - a.xs) : nullptr;
    int32_t *s1p = WSUM ? sp1 + (c0 - a.xs) : nullptr;
    int32_t *s2p = WSUM ? sp2 + (c0 - a.xs) : nullptr;
    // Without the sums planes a group of 4 rows is written through obuf:
    // wavefront w stores row 4k + w of the group, all 1024 columns (4 KB in
    // four 1 KB instructions), which the memory system drains faster than
    // four wavefronts writing 1 KB of the same row each.  rrow: this lane's
    // first output of that row (columns X0 + 4l + 256c, c = chunk).
    float *rrow = outp + (size_t)w * op + (X0 + 4 * l - a.xs);
    bool cfull[TZ_WAVES];
#pragma unroll
    for (int c = 0; c < TZ_WAVES; c++)
        cfull[c] = X0 + 256 * c >= a.xs && X0 + 256 * c + 256 <= a.Wo;  // wave-uniform

    // Software pipeline: iteration y reads from LDS what row y + 1 needs,
    // issues the matrix-core chain of row y + 1 and finishes row y (window
    // sums, epilogue, stores) while that chain runs.  Step s of row y reads B
    // slot (y + s) & 7; step 7 of row y + 1 reads image row y + 8 + roff,
    // read in iteration y - 1 and put into the slot row y's step 0 has read.
    v4i accC = (v4i){0, 0, 0, 0}, acoC = (v4i){0, 0, 0, 0};
#pragma unroll
    for (int s = 0; s < 8; s++) {
        accC = __builtin_amdgcn_mfma_i32_16x16x64_i8(atp[s], bring[s], accC, 0, 0, 0);
        acoC = __builtin_amdgcn_mfma_i32_16x16x64_i8(aone, bring[s], acoC, 0, 0, 0);
    }
    uint32_t hd[5];  // window bytes of image row y + 15 (for row y)
    hload(15, hd);
    v4i nb = bload(8 + roff);  // step 7 of row 1

#pragma unroll
    for (int q = 0; q < NG; q++) {
#pragma unroll
        for (int yy = 0; yy < 16; yy++) {
            const int y = 16 * q + yy;
            if (y == YB) {  // the rest of the strip (wave-uniform, all lanes)
#pragma unroll
                for (int u = UA; u < TZ_LOADS; u++) stage(u);
                __syncthreads();
            }
            // reads for row y + 1
            uint32_t hdN[5];
            v4i nbN = nb;
            if (y + 1 < RS) hload(y + 16, hdN);
            if (y + 2 < RS) nbN = bload(y + 9 + roff);
            v4i accN = (v4i){0, 0, 0, 0}, acoN = acoC;
            if (y + 1 < RS) {
#pragma unroll
                for (int s = 0; s < 8; s++) {
                    const v4i b = s < 7 ? bring[(yy + 1 + s) & 7] : nb;
                    accN = __builtin_amdgcn_mfma_i32_16x16x64_i8(atp[s], b, accN, 0, 0, 0);
                }
                // D(y + 1) = D(y) + rs(y + 16) - rs(y): slot y & 7 holds rows
                // y, y + 8 (groups 0, 1 / 2, 3), nb rows y + 8, y + 16
                acoN = __builtin_amdgcn_mfma_i32_16x16x64_i8(adiff, bring[yy & 7], acoN, 0, 0, 0);
                acoN = __builtin_amdgcn_mfma_i32_16x16x64_i8(adiff, nb, acoN, 0, 0, 0);
                bring[yy & 7] = nb;
            }
            nb = nbN;
            // V of row y: row y + 15 enters, row y - 1 leaves
            int qq[4];
            row_sq4<WT>(hd, qq);
#pragma unroll
            for (int k = 0; k < 5; k++) hd[k] = hdN[k];
#pragma unroll
            for (int i = 0; i < 4; i++) {
                NV[i] += __mul24(ring[i][(yy + 15) & 15] - qq[i], K);
                ring[i][(yy + 15) & 15] = qq[i];
                // keep NV itself as the loop's running value (the compiler
                // would otherwise carry the sum of the differences and form
                // K times it anew for every use: one more instruction)
                asm volatile("" : "+v"(NV[i]));
            }
            const v4i acc = accC, aco = acoC;
            accC = accN;
            acoC = acoN;

            // the coefficients are formed unconditionally (one basic block
            // with the matrix-core chain, so the two interleave); only the
            // stores depend on the row being an output row
            float gv[4];
            int sI[4], sQ[4], sIT[4];
#pragma unroll
            for (int i = 0; i < 4; i++) {
                const int D = aco[i], C = acc[i];  // sums of I' and of I'T' over the window
                const int num = (int)((unsigned)__mul24(D, nsT) + (unsigned)__mul24(K, C));
                const int nvarI = __mul24(D, D) + NV[i];
                gv[i] = ncc_coef((float)num, (float)nvarI, nvarTf);
                if (WSUM) {
                    sI[i] = D + 128 * K;
                    sQ[i] = -NV[i] / K + 256 * D + 16384 * K;
                    sIT[i] = C + 128 * (D + sT1) + 16384 * K;
                }
            }
            if constexpr (!WSUM) {
                obuf[yy & 3][w][18 * g + n] = make_float4(gv[0], gv[1], gv[2], gv[3]);
                if ((yy & 3) == 3) {  // the group's 4 rows are in obuf
                    __syncthreads();
                    const int R = y - 3 + w;  // the row this wavefront stores
                    float4 v[TZ_WAVES];
#pragma unroll
                    for (int c = 0; c < TZ_WAVES; c++) v[c] = obuf[w][c][18 * (l & 3) + (l >> 2)];
                    if (R < rowsOut) {  // wave-uniform
#pragma unroll
                        for (int c = 0; c < TZ_WAVES; c++) {
                            float *dst = rrow + 256 * c;
                            if (cfull[c]) {
                                __builtin_nontemporal_store((f4u){v[c].x, v[c].y, v[c].z, v[c].w}, (f4u *)dst);
                            } else {
                                const float vv[4] = {v[c].x, v[c].y, v[c].z, v[c].w};
#pragma unroll
                                for (int i = 0; i < 4; i++) {
                                    const int x = X0 + 256 * c + 4 * l + i;
                                    if (x >= a.xs && x < a.Wo) dst[i] = vv[i];
                                }
                            }
                        }
                    }
                    rrow += 4 * op;
                    // reads done before the slots take the next group
                    __syncthreads();
                }
            } else {
                to_lane_order(gv, pidx);
                if (WSUM) {
                    to_lane_order(sI, pidx);
                    to_lane_order(sQ, pidx);
                    to_lane_order(sIT, pidx);
                }
                if (y < rowsOut) {  // wave-uniform
                    if (wfull) {
                        // coefficients and SumI nontemporal, SumISq and SumIT
                        // ordinary: with four planes to write, a mix of the
                        // two store kinds drains faster than either kind alone
                        // (4096^2: 74.0 us all nontemporal, 54.2 all ordinary,
                        // 50.4 mixed)
                        __builtin_nontemporal_store((f4u){gv[0], gv[1], gv[2], gv[3]}, (f4u *)orp);
                        if (WSUM) {
                            if (t == 0) {
                                __builtin_nontemporal_store((i4u){sI[0], sI[1], sI[2], sI[3]},
                                                            (i4u *)s0p);
                                *(i4u *)s1p = (i4u){sQ[0], sQ[1], sQ[2], sQ[3]};
                            }
                            *(i4u *)s2p = (i4u){sIT[0], sIT[1], sIT[2], sIT[3]};
                        }
                    } else {
    #pragma unroll
                        for (int i = 0; i < 4; i++) {
                            const int x = c0 + i;
                            if (x >= a.xs && x < a.Wo) {
                                orp[i] = gv[i];
                                if (WSUM) {
                                    if (t == 0) {
                                        s0p[i] = sI[i];
                                        s1p[i] = sQ[i];
                                    }
                                    s2p[i] = sIT[i];
                                }
                            }
                        }
                    }
                }
                orp += op;
                if (WSUM) {
                    s0p += op;
                    s1p += op;
                    s2p += op;
                }
            }
            // keep each iteration's loads and arithmetic inside it
            __builtin_amdgcn_sched_barrier(0);
        }
    }
}

template <int WT, int RS, bool WSUM>
hipError_t launch_tz(const CorrArgs &a, int t, hipStream_t st) {
    const int ntx = (a.Wo + TZ_NC - 1) / TZ_NC, nty = (a.Ho + RS - 1) / RS;
    dim3 grid(xcd_grid(ntx * nty));
    const uintptr_t al = (uintptr_t)a.img | (uintptr_t)a.ip;
    if ((al & 15) == 0 && a.W % 16 == 0)
        hipLaunchKernelGGL((corr_toeplitz<WT, RS, 16, WSUM>), grid, dim3(TZ_NT), 0, st, a, t, ntx, nty);
    else
        hipLaunchKernelGGL((corr_toeplitz<WT, RS, 1, WSUM>), grid, dim3(TZ_NT), 0, st, a, t, ntx, nty);
    return hipGetLastError();
}

// Strip height: 32 rows halve the halo of 16-row strips, but a launch of
// fewer than two 32-row workgroups per CU leaves CUs idle; then 16 rows
// (measured: 28.7 vs 30.5 us at 4096 x 4096, 19.3 vs 16.5 us for a 2048 x
// 2048 search rectangle).  With the sums planes (four output planes instead
// of one) the call is bound by its stores, which 16-row strips drain faster:
// 74.6 against 82.6 us at 4096 x 4096, so those calls always take 16.  The
// option NCC_OPT_TZ_STRIP = 16 or 32 fixes it instead.
int tz_strip(const CorrArgs &a) {
    const int v = opt_get(NCC_OPT_TZ_STRIP);
    if (v == 16 || v == 32) return v;
    if (a.sums) return 16;
    static int cus[NCC_MAX_DEVICES];
    int dev = 0, n = 256;
    if (hipGetDevice(&dev) == hipSuccess && dev >= 0 && dev < NCC_MAX_DEVICES) {
        if (cus[dev] == 0) {
            int v = 0;
            cus[dev] = hipDeviceGetAttribute(&v, hipDeviceAttributeMultiprocessorCount, dev) ==
                                   hipSuccess && v > 0
                           ? v
                           : 256;
        }
        n = cus[dev];
    }
    const long long wgs32 = (long long)((a.Wo + TZ_NC - 1) / TZ_NC) * ((a.Ho + 31) / 32);
    return wgs32 >= 2LL * n ? 32 : 16;
}

template <int WT>
hipError_t launch_tz_w(const CorrArgs &a, int t, hipStream_t st) {
    const bool rs32 = tz_strip(a) == 32;
    if (a.sums) return rs32 ? launch_tz<WT, 32, true>(a, t, st) : launch_tz<WT, 16, true>(a, t, st);
    return rs32 ? launch_tz<WT, 32, false>(a, t, st) : launch_tz<WT, 16, false>(a, t, st);
}

}  // namespace

bool corr_toeplitz_supported(int wT, int hT) { return hT == 16 && wT >= 13 && wT <= 16; }

// A launch of fewer than 128 workgroups (1024 columns x 16 rows each) is
// latency-bound, and there the matrix-core tile kernel's 64 x 32 workgroups
// are faster (search rectangles on a 4096 x 4096 image, 16 x 16 template:
// 1024 x 1024 positions 8.0 against 10.9 us; 1536 x 1536 14.4 against
// 11.3 us).
bool corr_toeplitz_preferred(int Wo, int Ho) {
    return (long long)((Wo + TZ_NC - 1) / TZ_NC) * ((Ho + 15) / 16) >= 128;
}

hipError_t corr_toeplitz_launch(const CorrArgs &a, int t, hipStream_t st) {
    if (a.hT != 16) return hipErrorNotSupported;
    switch (a.wT) {
        case 13: return launch_tz_w<13>(a, t, st);
        case 14: return launch_tz_w<14>(a, t, st);
        case 15: return launch_tz_w<15>(a, t, st);
        case 16: return launch_tz_w<16>(a, t, st);
        default: return hipErrorNotSupported;
    }
}

}  // namespace ncc
