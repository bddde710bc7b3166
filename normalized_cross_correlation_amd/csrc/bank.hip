// Template bank on the int8 matrix cores (v_mfma_i32_16x16x64_i8).
//
// The correlation of a bank of templates with one image (The CUDA Handbook
// ch. 15 section 15.8 notes that one summed-area table serves every template
// in a bank) has SumIT as a dense contraction: windows x K times K x
// templates, K = wT*hT.  Bytes are moved to int8 by T' = T - 128 and
// I' = I - 128 (an XOR with 0x80), the matrix cores accumulate
// SIT' = sum I'T' in int32, and the exact sums come back by
//   SumIT = SIT' + 128*SumI + 128*SumT - 16384*K.
// The coefficient's numerator is then
//   num = K*SIT' + SumI*(128K - SumT) + (128K*SumT - 16384K^2),
// evaluated with 24-bit multiplies modulo 2^32: exact, since every factor
// fits 24 signed bits and |num| <= K^2 * 127.5^2 < 2^31 for the K <= 256
// this kernel takes.
//
// Operand layout (16x16x64, checked on the device): lane 16*g + m of the A
// operand holds 16 bytes of row m, lane 16*g + n of B the same 16 k-slots of
// column n, and lane 16*g + n of the result holds rows 4g..4g+3 of column n.
// The k order inside the 64 is the same for A and B, so chunk c = 4*kstep + g
// is a 16-byte piece of one template row (row c / NB16, bytes 16*(c % NB16)).
//
// A workgroup (4 wavefronts) owns 64 x 16 output positions and NB (1 or 2) blocks of
// 16 templates.  It stages the image tile + halo in LDS as int8 (all of its
// 16-byte loads in flight at once), then
//   1. window statistics: SumI and 1/sqrt(varI) of its 1024 positions (row
//      window sums per image row, each 4-column item by one dot4 window and
//      three 1-byte slides, then the hT-row sums), kept in LDS; every step
//      issues its LDS loads together, so the phase costs a few LDS round
//      trips rather than one per dword;
//   2. per row of 64 positions (4 groups of 16 A rows): byte-aligns the
//      chunks, runs KSTEPS x 4 MFMAs per block of 16 templates, turns each
//      result into a coefficient with the statistics of its position and
//      template, and writes them through a per-wavefront LDS transpose so
//      that each store instruction covers 256 contiguous bytes of each of 4
//      template maps (the MFMA result layout spreads one instruction over 16
//      maps, 64 bytes each, which the memory system serves poorly).
#include <algorithm>

#include "ncc_internal.h"

namespace ncc {

namespace {

typedef int v4i __attribute__((ext_vector_type(4)));
typedef float f4u __attribute__((ext_vector_type(4), aligned(4)));
typedef int i4u __attribute__((ext_vector_type(4), aligned(4)));

constexpr int BX = 64;  // positions per workgroup row
constexpr int BY = 16;  // rows per workgroup
constexpr int MAXR = BY + 15;  // tile rows for hT <= 16
constexpr int OBP = BX + 4;    // row pitch (floats) of the output transpose buffer
// 16-byte staging loads per thread: at most (BY + hT - 1) x (BX + 16 * nb16 +
// 4 rounded to 16) / 16 chunks over hT * nb16 <= 16 (the largest: hT = 1,
// wT = 256: 16 rows x 21 chunks)
constexpr int STAGE_LOADS = 2;
// row window sum items (4 columns each) per thread: at most MAXR x BX / 4
constexpr int ROW_ITEMS = (MAXR * (BX / 4) + 255) / 256;
// one LDS array for the row window sums of I' and I'^2 (MAXR x BX each) and,
// later, the per-wavefront transpose buffers (4 x 16 templates x OBP)
constexpr int UBUF = 2 * MAXR * BX > 4 * 16 * OBP ? 2 * MAXR * BX : 4 * 16 * OBP;
// LDS of one workgroup, static part (UBUF, SumI and 1/sqrt(varI) per position)
constexpr int STATIC_LDS = 4 * UBUF + 2 * 4 * BY * BX;
// Two workgroups per CU at most (the LDS request of each is raised to more
// than a third of the CU's 160 KB): more in flight spread the output writes
// over more DRAM pages at once and slow the whole bank down (64 templates at
// 4096^2: 1.50 against 1.06 ms with three per CU).
constexpr int LDS_TWO_PER_CU = 56 * 1024;

__device__ __forceinline__ int sdot4(uint32_t a, uint32_t b, int c) {
    return __builtin_amdgcn_sdot4((int)a, (int)b, c, false);
}

template <int KSTEPS, int NB, bool FULLT>
__global__ __launch_bounds__(256) void corr_bank(CorrArgs a, int nb16, int pitch, int rowsT,
                                                 int g0, int ntx, int nty, int nz) {
    extern __shared__ __align__(16) uint32_t tile[];  // rowsT x pitch bytes of I' = I ^ 0x80
    // The row window sums (step 1) and the output transpose buffers (step 2)
    // are never live together: one array holds both.
    __shared__ __align__(16) int ubuf[UBUF];
    int(*const hsI)[BX] = (int(*)[BX])ubuf;               // row window sums of I'
    int(*const hsQ)[BX] = (int(*)[BX])(ubuf + MAXR * BX);  // row window sums of I'^2
    __shared__ int sIs[BY][BX];         // SumI per position
    __shared__ float rIs[BY][BX];       // 1/sqrt(varI) per position, 0 if varI == 0
    // Launch order: template blocks slowest, so that at any time the whole
    // chip writes the maps of one block (fewer maps in flight: 1.22 against
    // 1.39 ms for 64 maps at 4096^2); inside a block, XCD-contiguous tile
    // order (several times the write bandwidth of tiles interleaved across
    // the XCDs' L2s for these output maps).
    const int per = (ntx * nty + NUM_XCD - 1) / NUM_XCD * NUM_XCD;
    const int bz = (int)blockIdx.x / per;
    const int bxy = xcd_tile((int)blockIdx.x % per, ntx * nty);
    if (bxy < 0) return;
    const int tid = threadIdx.x, w = tid >> 6, l = tid & 63;
    const int g = l >> 4, m = l & 15;
    const int x0 = (bxy % ntx) * BX, y0 = (bxy / ntx) * BY;
    const int pw = pitch / 4;
    const bool a16 = ((((uintptr_t)a.img) | a.ip | (size_t)a.W) & 15) == 0;
    const int K = a.wT * a.hT;
    const int wt4 = (a.wT + 3) / 4;

    // ---- stage the tile + halo as int8, 16 bytes per load, every load issued
    // before the first is used.  A 16-byte aligned image (address and row
    // pitch) takes clamped in-bounds addresses; bytes of columns past W or
    // rows past H then repeat image bytes, and those feed only positions
    // past Wo or Ho or meet zero template bytes (the padding of the B
    // operands), so what they hold is immaterial.
    const int pc = pitch / 16, nch = rowsT * pc;  // 16-byte chunks
    // each chunk with the 4 bytes after it, for the byte-shifted copies
    uint4 pre[STAGE_LOADS];
    uint32_t nxt[STAGE_LOADS];
#pragma unroll
    for (int u = 0; u < STAGE_LOADS; u++) {
        const int i = min(tid + 256 * u, nch - 1);
        const int y = y0 + i / pc, x = x0 + 16 * (i % pc);
        if (a16) {
            const uint8_t *row = a.img + (size_t)min(y, a.H - 1) * a.ip;
            pre[u] = *(const uint4 *)(row + min(x, a.W - 16));
            nxt[u] = *(const uint32_t *)(row + min(x + 16, a.W - 4));
        } else {
            pre[u] = load16_any(a.img, a.ip, a.W, a.H, x, y);
            nxt[u] = load16_any(a.img, a.ip, a.W, a.H, x + 16, y).x;
        }
    }
    // ---- B operands and per-template constants of the NB blocks
    v4i bop[NB][KSTEPS];
    int ca[NB], cb[NB];
    float rT[NB];
#pragma unroll
    for (int nb = 0; nb < NB; nb++) {
        const int gg = g0 + bz * NB + nb;
#pragma unroll
        for (int ks = 0; ks < KSTEPS; ks++)
            bop[nb][ks] = *(const v4i *)(a.mfma + (((size_t)gg * KSTEPS + ks) * 64 + l) * 16);
        const int tt = gg * 16 + m;  // this lane's template in block nb
        if (FULLT || tt < a.nTpl) {
            const TStat ts = a.stats[tt];
            const int sT = (int)ts.sumT;
            ca[nb] = 128 * K - sT;
            cb[nb] = (int)((unsigned)(128 * K) * (unsigned)sT - (unsigned)(16384 * K) * (unsigned)K);
            rT[nb] = ts.rT;
        } else {
            ca[nb] = cb[nb] = 0;
            rT[nb] = 0.0f;
        }
    }
    // copy s (0..3) of the tile holds each row shifted left by s bytes, so
    // that a 16-byte piece at any byte offset is 4 dword-aligned words of one
    // copy
    const int csz = rowsT * pw;  // dwords per copy
#pragma unroll
    for (int u = 0; u < STAGE_LOADS; u++) {
        const int i = tid + 256 * u;
        if (i < nch) {
            const uint4 v = pre[u];
            const uint32_t d[5] = {v.x ^ 0x80808080u, v.y ^ 0x80808080u, v.z ^ 0x80808080u,
                                   v.w ^ 0x80808080u, nxt[u] ^ 0x80808080u};
            uint32_t *dst = &tile[(i / pc) * pw + 4 * (i % pc)];
            *(uint4 *)dst = make_uint4(d[0], d[1], d[2], d[3]);
#pragma unroll
            for (int sh = 1; sh < 4; sh++)
                *(uint4 *)(dst + sh * csz) =
                    make_uint4(align_bytes(d[1], d[0], sh), align_bytes(d[2], d[1], sh),
                               align_bytes(d[3], d[2], sh), align_bytes(d[4], d[3], sh));
        }
    }
    __syncthreads();

    // ---- 1. window statistics of the tile's positions
    // row window sums: item (image row r, columns c0 .. c0+3).  The window at
    // c0 by dot4 over its dwords (the bytes past wT masked off), then each
    // next one by the byte that enters and the one that leaves:
    // s1 += b' - b, s2 += b'^2 - b^2 = (b' - b)(b' + b).
    const int rowsHs = BY + a.hT - 1;
    const uint32_t mlast = byte_mask(a.wT - 4 * (wt4 - 1));
    const int8_t *tb = (const int8_t *)tile;
    const int nit = rowsHs * (BX / 4);
    // masks of a window's first four dwords: whole, the last one's wT bytes, none
    uint32_t mk[4];
#pragma unroll
    for (int k = 0; k < 4; k++) mk[k] = k < wt4 - 1 ? 0xffffffffu : k == wt4 - 1 ? mlast : 0u;
#pragma unroll
    for (int it = 0; it < ROW_ITEMS; it++) {
        // an index past the last item repeats it (loads in bounds, no store)
        const int i = min(tid + 256 * it, nit - 1);
        const int r = i / (BX / 4), c0 = 4 * (i % (BX / 4));
        const uint32_t *p = tile + r * pw + (c0 >> 2);
        const int8_t *pn = tb + r * pitch + c0 + a.wT;  // bytes entering
        uint32_t d[4];
        int bn[3];
#pragma unroll
        for (int k = 0; k < 4; k++) d[k] = p[k];
#pragma unroll
        for (int t = 0; t < 3; t++) bn[t] = pn[t];
        int s1 = 0, s2 = 0;
#pragma unroll
        for (int k = 0; k < 4; k++) {
            const uint32_t v = d[k] & mk[k];
            s1 = sdot4(v, 0x01010101u, s1);
            s2 = sdot4(v, v, s2);
        }
        for (int k = 4; k < wt4; k++) {  // templates wider than 16
            uint32_t v = p[k];
            if (k == wt4 - 1) v &= mlast;
            s1 = sdot4(v, 0x01010101u, s1);
            s2 = sdot4(v, v, s2);
        }
        int o1[4], o2[4];
        o1[0] = s1;
        o2[0] = s2;
#pragma unroll
        for (int t = 0; t < 3; t++) {
            const int bo = (int)(int8_t)(uint8_t)(d[0] >> (8 * t));
            s1 += bn[t] - bo;
            s2 += __mul24(bn[t] - bo, bn[t] + bo);
            o1[t + 1] = s1;
            o2[t + 1] = s2;
        }
        if (tid + 256 * it < nit) {
            *(int4 *)&hsI[r][c0] = make_int4(o1[0], o1[1], o1[2], o1[3]);
            *(int4 *)&hsQ[r][c0] = make_int4(o2[0], o2[1], o2[2], o2[3]);
        }
    }
    __syncthreads();
    {
        // thread (c, q): output rows r0 = RPT * q .. r0 + RPT - 1 of column c
        constexpr int RPT = BY / 4;
        const int c = tid & 63, r0 = RPT * (tid >> 6);
        // rows r0 .. r0 + 15 (those past hT - 1 masked off) and the rows
        // entering for outputs r0 + 1 .. r0 + RPT - 1, loaded together
        int vI[16], vQ[16], eI[RPT], eQ[RPT];
#pragma unroll
        for (int j = 0; j < 16; j++) {
            vI[j] = hsI[r0 + j][c];
            vQ[j] = hsQ[r0 + j][c];
        }
#pragma unroll
        for (int o = 1; o < RPT; o++) {
            eI[o] = hsI[r0 + o + a.hT - 1][c];
            eQ[o] = hsQ[r0 + o + a.hT - 1][c];
        }
        int s1 = 0, s2 = 0;
#pragma unroll
        for (int j = 0; j < 16; j++) {
            s1 += j < a.hT ? vI[j] : 0;
            s2 += j < a.hT ? vQ[j] : 0;
        }
#pragma unroll
        for (int o = 0; o < RPT; o++) {
            if (o > 0) {
                s1 += eI[o] - vI[o - 1];
                s2 += eQ[o] - vQ[o - 1];
            }
            // SumI = sum I' + 128K;  SumISq = sum I'^2 + 256 sum I' + 16384K
            const int sumI = s1 + 128 * K;
            const int sumISq = s2 + 256 * s1 + 16384 * K;
            const unsigned varI = (unsigned)K * (unsigned)sumISq - (unsigned)sumI * (unsigned)sumI;
            sIs[r0 + o][c] = sumI;
            rIs[r0 + o][c] = varI ? __builtin_amdgcn_rsqf((float)varI) : 0.0f;
            if (a.sums && bz == 0 && g0 == 0) {
                const int y = y0 + r0 + o, x = x0 + c;
                if (y < a.Ho && x < a.Wo) {
                    const size_t plane = a.oplane, oo = (size_t)y * a.op + x;
                    __builtin_nontemporal_store(sumI, a.sums + oo);
                    __builtin_nontemporal_store(sumISq, a.sums + plane + oo);
                }
            }
        }
    }
    __syncthreads();

    // ---- 2. the contraction: each wavefront takes whole rows of 64 positions
    // (4 groups of 16, the A rows) and, per block of 16 templates, turns the
    // MFMA results into coefficients, transposes them through its LDS buffer
    // and writes 256 contiguous bytes per template row.
    float *ob = (float *)ubuf + w * 16 * OBP;
    const size_t plane = a.oplane;
    const bool whole = x0 + BX <= a.Wo;  // every column of the tile is an output
    for (int yy = w; yy < BY; yy += 4) {
        const int y = y0 + yy;
        if (y >= a.Ho) break;
        // A operands: group mg, row m = position 16*mg + m, chunk c = 4*ks + g;
        // the piece starts at byte offset off, off % 4 = m % 4 (pitch is a
        // multiple of 16), read from the copy shifted by m % 4
        v4i A[4][KSTEPS];
#pragma unroll
        for (int mg = 0; mg < 4; mg++)
#pragma unroll
            for (int ks = 0; ks < KSTEPS; ks++) {
                const int c = 4 * ks + g, j = c / nb16, ib = c % nb16;
                const int jj = j < a.hT ? j : 0;  // padding chunks meet zero template bytes
                const int off = (yy + jj) * pitch + 16 * mg + m + 16 * ib;
                const uint32_t *p = tile + (m & 3) * csz + (off >> 2);
                A[mg][ks] = (v4i){(int)p[0], (int)p[1], (int)p[2], (int)p[3]};
            }
        // statistics of this lane's result rows: positions 16*mg + 4g .. +3
        int4 sI4[4];
        float4 rI4[4];
#pragma unroll
        for (int mg = 0; mg < 4; mg++) {
            sI4[mg] = *(const int4 *)&sIs[yy][16 * mg + 4 * g];
            rI4[mg] = *(const float4 *)&rIs[yy][16 * mg + 4 * g];
        }
        const size_t orow = (size_t)y * a.op + x0;
#pragma unroll
        for (int nb = 0; nb < NB; nb++) {
            v4i acc[4];
#pragma unroll
            for (int mg = 0; mg < 4; mg++) acc[mg] = (v4i){0, 0, 0, 0};
#pragma unroll
            for (int ks = 0; ks < KSTEPS; ks++)
#pragma unroll
                for (int mg = 0; mg < 4; mg++)
                    acc[mg] = __builtin_amdgcn_mfma_i32_16x16x64_i8(A[mg][ks], bop[nb][ks], acc[mg],
                                                                    0, 0, 0);
            // coefficients into ob[template m][position]
#pragma unroll
            for (int mg = 0; mg < 4; mg++) {
                const int sIi[4] = {sI4[mg].x, sI4[mg].y, sI4[mg].z, sI4[mg].w};
                const float rIi[4] = {rI4[mg].x, rI4[mg].y, rI4[mg].z, rI4[mg].w};
                float gv[4];
#pragma unroll
                for (int i = 0; i < 4; i++) {
                    const int num = __mul24(K, acc[mg][i]) + __mul24(sIi[i], ca[nb]) + cb[nb];
                    gv[i] = __builtin_amdgcn_fmed3f((float)num * (rIi[i] * rT[nb]), -1.0f, 1.0f);
                }
                *(float4 *)&ob[m * OBP + 16 * mg + 4 * g] = make_float4(gv[0], gv[1], gv[2], gv[3]);
                if (a.sums) {
                    const int tt = (g0 + bz * NB + nb) * 16 + m;
                    const int xb = x0 + 16 * mg + 4 * g;
                    if (FULLT || tt < a.nTpl) {
                        const int sT = 128 * K - ca[nb];
                        int32_t *sd = a.sums + (size_t)(2 + tt) * plane + (size_t)y * a.op + xb;
#pragma unroll
                        for (int i = 0; i < 4; i++)
                            if (xb + i < a.Wo)
                                sd[i] = acc[mg][i] + 128 * (sIi[i] + sT) - 16384 * K;
                    }
                }
            }
            // the lanes' writes are visible to the whole wavefront past here
            __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
            __builtin_amdgcn_wave_barrier();
            __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
            // lane l writes template 4s + l/16, positions 4*(l%16) .. +3
#pragma unroll
            for (int s = 0; s < 4; s++) {
                const int tl = 4 * s + (l >> 4), xq = 4 * (l & 15);
                const float4 v = *(const float4 *)&ob[tl * OBP + xq];
                const int tt = (g0 + bz * NB + nb) * 16 + tl;
                if (!FULLT && tt >= a.nTpl) continue;
                float *dst = a.coef + (size_t)tt * plane + orow + xq;
                if (whole) {
                    *(f4u *)dst = (f4u){v.x, v.y, v.z, v.w};
                } else {
                    const float vv[4] = {v.x, v.y, v.z, v.w};
#pragma unroll
                    for (int i = 0; i < 4; i++)
                        if (x0 + xq + i < a.Wo) dst[i] = vv[i];
                }
            }
            // reads done before the buffer is written again
            __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
            __builtin_amdgcn_wave_barrier();
            __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
        }
    }
}

void bank_geometry(int wT, int hT, int *pitch, int *rowsT) {
    const int nb16 = (wT + 15) / 16;
    *pitch = ((BX + 16 * nb16 + 4) + 15) / 16 * 16;
    *rowsT = BY + hT - 1;
}

template <int KS, int NB>
hipError_t launch_bank_nb(const CorrArgs &a, int g0, int nz, bool fullt, int nb16, int pitch,
                          int rowsT, size_t lds, hipStream_t st) {
    const int ntx = (a.Wo + BX - 1) / BX, nty = (a.Ho + BY - 1) / BY;
    dim3 grid(xcd_grid(ntx * nty) * nz);
    if (fullt)
        hipLaunchKernelGGL((corr_bank<KS, NB, true>), grid, dim3(256), lds, st, a, nb16, pitch,
                           rowsT, g0, ntx, nty, nz);
    else
        hipLaunchKernelGGL((corr_bank<KS, NB, false>), grid, dim3(256), lds, st, a, nb16, pitch,
                           rowsT, g0, ntx, nty, nz);
    return hipGetLastError();
}

template <int KS>
hipError_t launch_bank_ks(const CorrArgs &a, int nb16, int pitch, int rowsT, size_t lds,
                          hipStream_t st) {
    // groups of 16 templates: blocks of 2 groups (32 templates) per workgroup,
    // then a last single group.  Measured at 4096^2 with 64 templates (an
    // earlier form of the kernel): 2 groups per workgroup 1.22 ms, 4 groups
    // 1.39 ms, 1 group 1.34 ms (each workgroup stages its tile and window
    // statistics once per block).
    const int ng = (a.nTpl + 15) / 16;
    const bool tail16 = (a.nTpl % 16) != 0;
    const int n2 = ng / 2, rest = ng % 2;
    hipError_t e = hipSuccess;
    if (n2 > 0) {
        // the last group of the last full block may be partial
        const bool fullt = !(tail16 && rest == 0);
        e = launch_bank_nb<KS, 2>(a, 0, n2, fullt, nb16, pitch, rowsT, lds, st);
        if (e != hipSuccess) return e;
    }
    if (rest == 1) e = launch_bank_nb<KS, 1>(a, 2 * n2, 1, !tail16, nb16, pitch, rowsT, lds, st);
    return e;
}

}  // namespace

bool corr_bank_supported(int wT, int hT, int nTpl) {
    const int chunks = hT * ((wT + 15) / 16);
    return nTpl > 1 && hT <= 16 && chunks <= 16 && wT * hT <= 256;
}

hipError_t corr_bank_launch(const CorrArgs &a, hipStream_t st) {
    const int nb16 = (a.wT + 15) / 16;
    const int ks = (a.hT * nb16 + 3) / 4;
    int pitch, rowsT;
    bank_geometry(a.wT, a.hT, &pitch, &rowsT);
    // the tile's four copies, or more so that at most two workgroups share a CU
    const size_t lds = std::max((size_t)4 * pitch * rowsT, (size_t)(LDS_TWO_PER_CU - STATIC_LDS));
    // the kernel's staging covers at most 256 * STAGE_LOADS chunks of 16 bytes
    if (rowsT * (pitch / 16) > 256 * STAGE_LOADS) return hipErrorNotSupported;
    switch (ks) {
        case 1: return launch_bank_ks<1>(a, nb16, pitch, rowsT, lds, st);
        case 2: return launch_bank_ks<2>(a, nb16, pitch, rowsT, lds, st);
        case 3: return launch_bank_ks<3>(a, nb16, pitch, rowsT, lds, st);
        case 4: return launch_bank_ks<4>(a, nb16, pitch, rowsT, lds, st);
        default: return hipErrorNotSupported;
    }
}

}  // namespace ncc
