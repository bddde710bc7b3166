// Single-template correlation on the int8 matrix cores for templates up to
// 32 x 32, in 16 x 16 output tiles.
//
// What is computed is the per-window accumulation of The CUDA Handbook
// ch. 15 "Image in shared memory" (SumI, SumISq, SumIT over a wT x hT window
// of an image tile staged on chip, then the coefficient); every sum is an
// exact integer, so the route does not change an output bit.
//
// SumIT as a matrix product.  For template row j, the 16 positions
// x0 + m (m = 0..15) of an output row y and the 16 output rows y0 + n
// (n = 0..15) of a tile,
//   C[m][n] += sum_{u=0}^{63} T[j][u - m] * I[y0 + n + j][x0 + u]
// (T[j][c] = 0 outside 0 <= c < wT <= 32, so u - m < 32 and u < 48 <= 64):
// one v_mfma_i32_16x16x64_i8 per template row, A the 16 x 64 band matrix of
// template row j (in registers for the whole kernel), B 64 image bytes of 16
// image rows (read from LDS).  Both operands move to signed bytes by XOR
// 0x80 (T' = T - 128 inside the band, 0 outside it; I' = I - 128), so
// C = sum of I'T' over the window, and with D and V the window sums of I'
// and I'^2 and sT the sum of T',
//   num = K*SumIT - SumI*SumT = K*C - D*sT,  varI = K*V - D^2
// (both exact in double: |K*C|, D*sT, K*V, D^2 < 2^35 for K <= 1024).
//
// Operand layout (16x16x64): lane 16g + m of A holds k-slots 16g .. 16g+15
// of row m, lane 16g + n of B the same k-slots of column n, lane 16g + n of
// the result rows 4g .. 4g+3 of column n: positions x0 + 4g .. +3 of output
// row y0 + n, which the lane stores as one 16-byte write.
//
// Window sums D and V on the vector units.  Lane (g, n) forms the row sums
// of I' and I'^2 over the windows of its 4 positions for image row
// 16 rho + n of round rho (signed dot4 for the first window, then the byte
// that enters and the one that leaves), scans them down the 16 lanes of its
// row group (DPP shifts) with a carry from the earlier rounds (DPP
// row_share of lane 15), and writes the running column sums to LDS; each
// window sum is then the difference of two of them (the four-corner rule of
// section 15.8 on the tile's own summed-area table, the horizontal
// difference taken first).
//
// A workgroup (4 wavefronts) owns 64 positions x 32 output rows: wavefront
// w the 16 positions x0 = X0 + 16w, as two tiles (output rows Y0 .. Y0+15
// and Y0+16 .. Y0+31).  It stages the template (16-byte zero margins) and
// the 63 image rows x 128 bytes its windows cover in LDS once.
#include "ncc_internal.h"

namespace ncc {

namespace {

typedef int v4i __attribute__((ext_vector_type(4)));
typedef float f4u __attribute__((ext_vector_type(4), aligned(4)));
typedef int i4u __attribute__((ext_vector_type(4), aligned(4)));

constexpr int MT_HMAX = 32;            // template rows (A operands in registers)
constexpr int MT_WMAX = 32;            // template bytes per row
constexpr int MT_WAVES = 4;
constexpr int MT_NT = MT_WAVES * 64;
constexpr int MT_NC = MT_WAVES * 16;   // output columns per workgroup
constexpr int MT_NR = 32;              // output rows per workgroup (two 16-row tiles)
constexpr int MT_ROWS = 64;            // staged image rows (MT_NR + MT_HMAX - 1, + 1)
constexpr int MT_CH = 8;               // staged 16-byte chunks per row (128 bytes)
constexpr int MT_PITCH = MT_CH * 4 + 4;  // dwords per staged row (+16 bytes against bank conflicts)
constexpr int MT_TPITCH = 24;          // dwords per template row: 16 zero bytes, the row, zeros
constexpr int MT_CSP = 36;             // dwords per row of running sums: [g][8] + 16 bytes (banks)
constexpr int DPP_ROW_SHARE15 = 0x15f;  // every lane of a 16-lane row reads its lane 15

// Row window sums of I' (r) and I'^2 (q), signed bytes, at the four columns
// whose bytes start at d[0]: the first window by signed dot4 over the masked
// dwords, then the bytes that leave (byte t) and enter (be[t], byte wT + t).
__device__ __forceinline__ void mt_row_sums(const uint32_t (&d)[8], const uint32_t (&mk)[8],
                                            const int (&be)[3], int (&r)[4], int (&q)[4]) {
    int s1 = 0, s2 = 0;
#pragma unroll
    for (int k = 0; k < 8; k++) {
        const int v = (int)(d[k] & mk[k]);
        s1 = __builtin_amdgcn_sdot4(v, 0x01010101, s1, false);
        s2 = __builtin_amdgcn_sdot4(v, v, s2, false);
    }
    r[0] = s1;
    q[0] = s2;
#pragma unroll
    for (int t = 0; t < 3; t++) {
        const int bo = (int)(int8_t)(uint8_t)(d[0] >> (8 * t)), bn = be[t];
        r[t + 1] = r[t] + (bn - bo);
        q[t + 1] = q[t] + __mul24(bn - bo, bn + bo);
    }
}

// Inclusive sum down the 16 lanes of each row group.
__device__ __forceinline__ int row16_scan(int x) {
    x += __builtin_amdgcn_update_dpp(0, x, DPP_ROW_SHR1, 0xf, 0xf, false);
    x += __builtin_amdgcn_update_dpp(0, x, DPP_ROW_SHR2, 0xf, 0xf, false);
    x += __builtin_amdgcn_update_dpp(0, x, DPP_ROW_SHR4, 0xf, 0xf, false);
    x += __builtin_amdgcn_update_dpp(0, x, DPP_ROW_SHR8, 0xf, 0xf, false);
    return x;
}

// NJ: matrix-core steps, hT rounded up to a multiple of 8 (rows hT .. NJ-1
// of the template are zero); RR: rounds of 16 image rows of window sums.
template <int NJ, int ALIGN, bool WSUM>
__global__ __launch_bounds__(MT_NT, 2) void corr_mtile(CorrArgs a, int t, int ntx, int nty) {
    static_assert(NJ % 8 == 0 && NJ <= MT_HMAX, "steps in whole groups of 8");
    constexpr int RR = (MT_NR + NJ - 1 + 15) / 16;
    __shared__ uint32_t img_s[MT_ROWS][MT_PITCH];      // image rows Y0 .. Y0+63 as I^0x80
    __shared__ uint32_t tpl_s[NJ][MT_TPITCH];          // template row j at bytes 16 .. 16+wT-1, as T^0x80
    __shared__ int cs_s[MT_WAVES][MT_ROWS][MT_CSP];     // running column sums (per wavefront)
    __shared__ int tsum[MT_WAVES][2];

    const int tix = xcd_tile((int)blockIdx.x, ntx * nty);
    if (tix < 0) return;
    const int tid = threadIdx.x, w = tid >> 6, l = tid & 63;
    const int g = l >> 4, n = l & 15;
    const int X0 = (tix % ntx) * MT_NC, Y0 = (tix / ntx) * MT_NR;
    const int wT = a.wT, hT = a.hT, K = wT * hT;

    // ---- image rows Y0 .. Y0+63, bytes X0 .. X0+127 (two 16-byte loads per
    // lane; clamped addresses: what lies past the image feeds only positions
    // past Wo or Ho, which are not stored)
    uint4 pre[2];
#pragma unroll
    for (int u = 0; u < 2; u++) {
        const int i = tid + u * MT_NT, r = i / MT_CH, c = i % MT_CH;
        const int y = Y0 + r, x = X0 + 16 * c;
        if (ALIGN == 16)
            pre[u] = *(const uint4 *)(a.img + (size_t)min(y, a.H - 1) * a.ip + min(x, a.W - 16));
        else
            pre[u] = load16_any(a.img, a.ip, a.W, a.H, x, y);
    }
    // ---- template rows with 16-byte zero margins, as signed bytes (rows
    // past hT are zero, so their matrix-core steps add nothing), and the
    // sums of T' and T'^2.  Every byte is read from a clamped in-bounds index
    // and masked afterwards (no branch), so all of a lane's loads issue
    // together.
    const uint8_t *T = a.tpl + (size_t)t * hT * wT;
    constexpr int TE = NJ * MT_TPITCH;              // staged template dwords
    constexpr int TIT = (TE + MT_NT - 1) / MT_NT;   // per lane
    uint32_t tbyte[TIT][4];
#pragma unroll
    for (int it = 0; it < TIT; it++) {
        const int e = tid + it * MT_NT, j = e / MT_TPITCH, dw = e % MT_TPITCH;
#pragma unroll
        for (int b = 0; b < 4; b++) {
            const int c = 4 * dw + b - 16;
            const bool ok = e < TE && j < hT && c >= 0 && c < wT;
            tbyte[it][b] = T[ok ? j * wT + c : 0];
        }
    }
    int st1 = 0, st2 = 0;
#pragma unroll
    for (int it = 0; it < TIT; it++) {
        const int e = tid + it * MT_NT, j = e / MT_TPITCH, dw = e % MT_TPITCH;
        uint32_t v = 0;
#pragma unroll
        for (int b = 0; b < 4; b++) {
            const int c = 4 * dw + b - 16;
            const bool ok = e < TE && j < hT && c >= 0 && c < wT;
            v |= ok ? (tbyte[it][b] ^ 0x80u) << (8 * b) : 0u;
        }
        if (e < TE) tpl_s[j][dw] = v;
        st1 = __builtin_amdgcn_sdot4((int)v, 0x01010101, st1, false);
        st2 = __builtin_amdgcn_sdot4((int)v, (int)v, st2, false);
    }
    {
        const int p1 = (int)wave_sum_u32((uint32_t)st1), p2 = (int)wave_sum_u32((uint32_t)st2);
        if (l == 0) {
            tsum[w][0] = p1;
            tsum[w][1] = p2;
        }
    }
#pragma unroll
    for (int u = 0; u < 2; u++) {
        const int i = tid + u * MT_NT, r = i / MT_CH, c = i % MT_CH;
        const uint4 v = pre[u];
        *(uint4 *)&img_s[r][4 * c] = make_uint4(v.x ^ 0x80808080u, v.y ^ 0x80808080u,
                                                v.z ^ 0x80808080u, v.w ^ 0x80808080u);
    }
    __syncthreads();

    // ---- A operands: template row j, lane (g, m = n): bytes 16g - m .. +15
    // of the row (zero outside it), i.e. bytes st .. st+15 of tpl_s[j]
    v4i A[NJ];
    {
        const int st = 16 + 16 * g - n;  // 1 .. 64
        const int dw0 = st >> 2;
        const uint32_t sh = (uint32_t)(st & 3);
#pragma unroll
        for (int j = 0; j < NJ; j++) {
            const uint32_t *p = &tpl_s[j][dw0];
            const uint32_t e0 = p[0], e1 = p[1], e2 = p[2], e3 = p[3], e4 = p[4];
            A[j] = (v4i){(int)align_bytes(e1, e0, sh), (int)align_bytes(e2, e1, sh),
                         (int)align_bytes(e3, e2, sh), (int)align_bytes(e4, e3, sh)};
        }
    }
    const int sT1 = tsum[0][0] + tsum[1][0] + tsum[2][0] + tsum[3][0];
    const int sT2 = tsum[0][1] + tsum[1][1] + tsum[2][1] + tsum[3][1];
    // varT = K * sum T'^2 - (sum T')^2 (shift-invariant, < 2^35)
    const float varTf = (float)((long long)K * sT2 - (long long)sT1 * sT1);

    // ---- SumIT: two 16 x 16 tiles (output rows Y0 + n and Y0 + 16 + n),
    // one step per template row.  Lane (g, n) reads image row n + s (bytes
    // 16w + 16g .. +15) once for both tiles: template row s of the first,
    // row s - 16 of the second.
    v4i acc0 = (v4i){0, 0, 0, 0}, acc1 = (v4i){0, 0, 0, 0};
    const int bcol = 4 * w + 4 * g;
#pragma unroll
    for (int s = 0; s < NJ + 16; s++) {
        const v4i b = *(const v4i *)&img_s[n + s][bcol];
        if (s < NJ) acc0 = __builtin_amdgcn_mfma_i32_16x16x64_i8(A[s], b, acc0, 0, 0, 0);
        if (s >= 16) acc1 = __builtin_amdgcn_mfma_i32_16x16x64_i8(A[s - 16], b, acc1, 0, 0, 0);
    }

    // ---- window sums: row sums of image rows 16 rho + n over the windows of
    // positions 16w + 4g .. +3, running sums down the rows (with the carry of
    // the earlier rounds), into cs_s[w][row][8g .. 8g+7] = r0..r3, q0..q3
    uint32_t mk[8];
#pragma unroll
    for (int k = 0; k < 8; k++) mk[k] = byte_mask(min(max(wT - 4 * k, 0), 4));
    const int hw = 4 * w + g;                           // dword of the lane's window bytes
    const int8_t *rowb = (const int8_t *)&img_s[0][0];  // bytes
    int carry[8] = {0, 0, 0, 0, 0, 0, 0, 0};
#pragma unroll
    for (int rho = 0; rho < RR; rho++) {
        const int r = 16 * rho + n;
        uint32_t d[8];
#pragma unroll
        for (int k = 0; k < 8; k++) d[k] = img_s[r][hw + k];
        int be[3];
#pragma unroll
        for (int tt = 0; tt < 3; tt++) be[tt] = rowb[r * (MT_PITCH * 4) + 4 * hw + wT + tt];
        int rs[4], qs[4];
        mt_row_sums(d, mk, be, rs, qs);
        int v[8] = {rs[0], rs[1], rs[2], rs[3], qs[0], qs[1], qs[2], qs[3]};
#pragma unroll
        for (int k = 0; k < 8; k++) {
            v[k] = row16_scan(v[k]) + carry[k];
            carry[k] = __builtin_amdgcn_update_dpp(0, v[k], DPP_ROW_SHARE15, 0xf, 0xf, false);
        }
        *(int4 *)&cs_s[w][r][8 * g] = make_int4(v[0], v[1], v[2], v[3]);
        *(int4 *)&cs_s[w][r][8 * g + 4] = make_int4(v[4], v[5], v[6], v[7]);
    }
    // (cs_s rows are written and then read by the same wavefront: LDS keeps
    // a wavefront's accesses in order)

    // ---- epilogue: tile tau, lane (g, n): output row Y0 + 16 tau + n,
    // positions X0 + 16w + 4g .. +3
    const double Kd = (double)K, sTd = (double)sT1;
    const size_t plane = a.oplane;
    const int xo = X0 + 16 * w + 4 * g;     // the lane's first position
    const bool full4 = xo + 4 <= a.Wo;
#pragma unroll
    for (int tau = 0; tau < 2; tau++) {
        const v4i acc = tau ? acc1 : acc0;
        const int o = 16 * tau + n;             // output row within the workgroup
        const int y = Y0 + o;
        int lo[8], hi[8];
        {
            const int rl = max(o - 1, 0), rh = o + hT - 1;
            const int4 l0 = *(const int4 *)&cs_s[w][rl][8 * g], l1 = *(const int4 *)&cs_s[w][rl][8 * g + 4];
            const int4 h0 = *(const int4 *)&cs_s[w][rh][8 * g], h1 = *(const int4 *)&cs_s[w][rh][8 * g + 4];
            const int z = o > 0 ? 1 : 0;  // the running sum above row 0 is 0
            lo[0] = z * l0.x; lo[1] = z * l0.y; lo[2] = z * l0.z; lo[3] = z * l0.w;
            lo[4] = z * l1.x; lo[5] = z * l1.y; lo[6] = z * l1.z; lo[7] = z * l1.w;
            hi[0] = h0.x; hi[1] = h0.y; hi[2] = h0.z; hi[3] = h0.w;
            hi[4] = h1.x; hi[5] = h1.y; hi[6] = h1.z; hi[7] = h1.w;
        }
        float gv[4];
        int sI[4], sQ[4], sIT[4];
#pragma unroll
        for (int i = 0; i < 4; i++) {
            const int D = hi[i] - lo[i], V = hi[4 + i] - lo[4 + i], C = acc[i];
            const double Dd = (double)D;
            const double num = __builtin_fma(Kd, (double)C, -(Dd * sTd));
            const double varI = __builtin_fma(Kd, (double)V, -(Dd * Dd));
            gv[i] = ncc_coef((float)num, (float)varI, varTf);
            if (WSUM) {
                sI[i] = D + 128 * K;
                sQ[i] = V + 256 * D + 16384 * K;
                sIT[i] = C + 128 * (D + sT1) + 16384 * K;
            }
        }
        if (y < a.Ho && xo < a.Wo) {
            const size_t ob = (size_t)y * a.op + (size_t)(xo - a.xs);
            float *cp = a.coef + (size_t)t * plane + ob;
            if (full4) {
                __builtin_nontemporal_store((f4u){gv[0], gv[1], gv[2], gv[3]}, (f4u *)cp);
                if (WSUM) {
                    if (t == 0) {
                        __builtin_nontemporal_store((i4u){sI[0], sI[1], sI[2], sI[3]}, (i4u *)(a.sums + ob));
                        __builtin_nontemporal_store((i4u){sQ[0], sQ[1], sQ[2], sQ[3]},
                                                    (i4u *)(a.sums + plane + ob));
                    }
                    __builtin_nontemporal_store((i4u){sIT[0], sIT[1], sIT[2], sIT[3]},
                                                (i4u *)(a.sums + (size_t)(2 + t) * plane + ob));
                }
            } else {
#pragma unroll
                for (int i = 0; i < 4; i++) {
                    if (xo + i < a.Wo) {
                        cp[i] = gv[i];
                        if (WSUM) {
                            if (t == 0) {
                                a.sums[ob + i] = sI[i];
                                a.sums[plane + ob + i] = sQ[i];
                            }
                            a.sums[(size_t)(2 + t) * plane + ob + i] = sIT[i];
                        }
                    }
                }
            }
        }
    }
}

template <int NJ, bool WSUM>
hipError_t launch_mtile(const CorrArgs &a, int t, hipStream_t st) {
    const int ntx = (a.Wo + MT_NC - 1) / MT_NC, nty = (a.Ho + MT_NR - 1) / MT_NR;
    dim3 grid(xcd_grid(ntx * nty));
    const uintptr_t al = (uintptr_t)a.img | (uintptr_t)a.ip;
    if ((al & 15) == 0 && a.W % 16 == 0)
        hipLaunchKernelGGL((corr_mtile<NJ, 16, WSUM>), grid, dim3(MT_NT), 0, st, a, t, ntx, nty);
    else
        hipLaunchKernelGGL((corr_mtile<NJ, 1, WSUM>), grid, dim3(MT_NT), 0, st, a, t, ntx, nty);
    return hipGetLastError();
}

template <bool WSUM>
hipError_t launch_mtile_nj(const CorrArgs &a, int t, hipStream_t st) {
    switch ((a.hT + 7) / 8) {
        case 1: return launch_mtile<8, WSUM>(a, t, st);
        case 2: return launch_mtile<16, WSUM>(a, t, st);
        case 3: return launch_mtile<24, WSUM>(a, t, st);
        default: return launch_mtile<32, WSUM>(a, t, st);
    }
}

}  // namespace

bool corr_mtile_supported(int wT, int hT) {
    return wT >= 1 && wT <= MT_WMAX && hT >= 1 && hT <= MT_HMAX;
}

hipError_t corr_mtile_launch(const CorrArgs &a, int t, hipStream_t st) {
    if (!corr_mtile_supported(a.wT, a.hT)) return hipErrorNotSupported;
    return a.sums ? launch_mtile_nj<true>(a, t, st) : launch_mtile_nj<false>(a, t, st);
}

}  // namespace ncc
