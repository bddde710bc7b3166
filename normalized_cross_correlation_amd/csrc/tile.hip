// Single-template normalized cross-correlation on the vector units for
// templates up to 32 bytes wide and 64 rows high.
//
// What is computed follows The CUDA Handbook ch. 15 "Image in shared
// memory" (corrShared_kernel: an image tile plus a (wT-1) x (hT-1) halo
// staged in on-chip memory; for each window SumI, SumISq and SumIT, then the
// coefficient).  As in that kernel, the window sums come from the staged
// tile, not from global tables.
//
// corr_tile<WT4, A4>: a workgroup of 512 lanes (two wavefronts per SIMD)
// owns 64 x 64 output positions.  It stages
//   - the template as zero-padded dwords and its sums SumT, SumTSq (every
//     workgroup forms them again: at most 2 KB of template);
//   - the image tile + halo (64 + hT - 1 rows of 16 + WT4 dwords);
// and then
//   1. row window sums of I and I^2 for every staged row and position
//      (v_dot4_u32_u8 against ones / against itself), then their sums down
//      hT rows: SumI and SumISq of the 64 x 64 windows, kept in LDS;
//   2. SumIT: lane (tx, ty) owns positions 4tx .. 4tx+3 of output rows
//      2ty and 2ty+1 and walks the image rows 2ty .. 2ty+hT; per image row
//      it reads WT4+1 dwords, byte-aligns them to its 4 windows
//      (v_alignbyte_b32) and adds their products with the template rows that
//      meet this image row in each of its 2 output rows (the template words
//      are read from LDS, the same address for every lane);
//   3. the coefficient from the exact integers, as every other route forms
//      it, so all routes agree bit for bit.
// Integer widths: K = wT*hT <= 2048, so SumIT and SumISq <= 2048 * 255^2 <
// 2^28 in uint32 and num, varI exact in int64.
#include "ncc_internal.h"

namespace ncc {

namespace {

constexpr int TL_TX = 16, TL_TY = 32;  // lanes across and down a workgroup
constexpr int TL_PX = 4, TL_R = 2;      // positions and output rows per lane
constexpr int TL_BX = TL_TX * TL_PX;    // 64 output columns per workgroup
constexpr int TL_BY = TL_TY * TL_R;     // 64 output rows per workgroup
constexpr int TL_NT = TL_TX * TL_TY;    // 512 lanes: two wavefronts per SIMD
constexpr int TL_MAXW4 = 8;             // template dwords per row (wT <= 32)
constexpr int TL_MAXH = 64;             // template rows
// LDS row pitch of the tile in dwords: at least 16 + WT4 + 1 and
// TL_R * pitch = 16 (mod 64), so the 4 row groups of a wavefront (lanes
// 16 apart) read disjoint banks.
constexpr int TL_P = 40;
static_assert((TL_R * TL_P) % 64 == 16, "bank-disjoint row groups");

typedef float f4u __attribute__((ext_vector_type(4), aligned(4)));

// Dword c of the tile row at image row y: bytes x .. x+3 (x = x0 + 4c),
// zero outside the image.  A4: img and ip are multiples of 4, so the dword
// holding the row's last byte lies in the same (mapped) page as that byte;
// the read is clamped to it and the bytes past W masked.  Otherwise four
// clamped byte reads.  No branch, so a lane's staging loads issue together.
template <bool A4>
__device__ __forceinline__ uint32_t tl_load4(const uint8_t *img, size_t ip, int W, int H, int x,
                                             int y) {
    const uint8_t *row = img + (size_t)min(y, H - 1) * ip;
    const int nvalid = y < H ? min(max(W - x, 0), 4) : 0;
    const uint32_t m = nvalid >= 4 ? 0xffffffffu : ((1u << (8 * nvalid)) - 1u);
    if (A4) {
        const uint32_t *p = (const uint32_t *)row + min(x, W - 1) / 4;
        return *p & m;
    }
    uint32_t v = 0;
#pragma unroll
    for (int b = 0; b < 4; b++) v |= (uint32_t)row[min(x + b, W - 1)] << (8 * b);
    return v & m;
}

template <int WT4, bool A4>
__global__ __launch_bounds__(TL_NT) void corr_tile(CorrArgs a, int t, int ntx, int nty) {
    constexpr int TW = (WT4 + 3) / 4 * 4;  // template dwords per LDS row (whole uint4s)
    constexpr int NDW = 16 + WT4;          // staged dwords per tile row
    static_assert(NDW + 1 <= TL_P, "tile row fits its pitch");
    extern __shared__ uint32_t lds[];
    const int hT = a.hT, wT = a.wT;
    const int RT = TL_BY + hT - 1;          // staged rows
    uint32_t *tile = lds;                   // [RT + 3][TL_P] (the last 3 rows never staged)
    uint32_t *H1 = tile + (RT + 3) * TL_P;  // [RT][64] row window sums of I, then SumI
    uint32_t *H2 = H1 + RT * TL_BX;         // [RT][64] ... of I^2, then SumISq
    uint32_t *tw = H2 + RT * TL_BX;         // [hT + 6][TW] template dwords, rows >= hT zero
    __shared__ uint32_t red[2][TL_NT / 64];

    const int tix = xcd_tile((int)blockIdx.x, ntx * nty);
    if (tix < 0) return;
    const int x0 = (tix % ntx) * TL_BX, y0 = (tix / ntx) * TL_BY;
    const int tid = threadIdx.x, l = tid & 63, w = tid >> 6;

    // ---- image tile + halo and template: every load of the lane issued in
    // one round before the first use (a use of a just-loaded value waits for
    // every load issued before it).  Lanes past the end redo the last item
    // (clamped indices) and store the same value again, so no store sits in
    // a branch (the compiler would sink its load into the branch).
    constexpr int SB = ((TL_BY + TL_MAXH - 1) * NDW + TL_NT - 1) / TL_NT;  // image dwords per lane
    constexpr int TB = ((TL_MAXH + 6) * TW + TL_NT - 1) / TL_NT;           // template dwords per lane
    const int nst = RT * NDW, ntw = (hT + 6) * TW;
    uint32_t sv[SB];
#pragma unroll
    for (int n = 0; n < SB; n++) {
        const int i = min(tid + n * TL_NT, nst - 1);
        const int r = i / NDW, c = i - r * NDW;
        sv[n] = tl_load4<A4>(a.img, a.ip, a.W, a.H, x0 + 4 * c, y0 + r);
    }
    const uint8_t *T = a.tpl + (size_t)t * hT * wT;
    uint32_t tb[TB][4];
#pragma unroll
    for (int n = 0; n < TB; n++) {
        const int i = min(tid + n * TL_NT, ntw - 1);
        const int j = min(i / TW, hT - 1), k = i % TW;
#pragma unroll
        for (int b = 0; b < 4; b++) tb[n][b] = T[(size_t)j * wT + min(4 * k + b, wT - 1)];
    }
    uint32_t s1 = 0, s2 = 0;
#pragma unroll
    for (int n = 0; n < TB; n++) {
        const int i0 = tid + n * TL_NT, i = min(i0, ntw - 1);
        const int j = i / TW, k = i % TW;
        uint32_t v = 0;
#pragma unroll
        for (int b = 0; b < 4; b++) v |= (4 * k + b < wT && j < hT ? tb[n][b] : 0u) << (8 * b);
        tw[i] = v;
        if (i0 < ntw) {  // each dword counted once
            s1 = dot4u(v, 0x01010101u, s1);
            s2 = dot4u(v, v, s2);
        }
    }
    s1 = wave_incl_scan_u32(s1);
    s2 = wave_incl_scan_u32(s2);
    if (l == 63) {
        red[0][w] = s1;
        red[1][w] = s2;
    }
#pragma unroll
    for (int n = 0; n < SB; n++) {
        const int i = min(tid + n * TL_NT, nst - 1);
        const int r = i / NDW, c = i - r * NDW;
        tile[r * TL_P + c] = sv[n];
    }
    __syncthreads();
    long long sumT = 0, sumTSq = 0;
#pragma unroll
    for (int ww = 0; ww < TL_NT / 64; ww++) {
        sumT += red[0][ww];
        sumTSq += red[1][ww];
    }
    const long long K = (long long)wT * hT;
    const float varTf = (float)(K * sumTSq - sumT * sumT);

    // ---- 1. window sums: row sums over wT, then sums down hT rows
    const uint32_t mlast = (wT & 3) ? (1u << (8 * (wT & 3))) - 1u : 0xffffffffu;
    // four items per lane at a time, every LDS read of the four issued before
    // the first store (reads and stores share the LDS array, so the compiler
    // cannot move a later item's reads above an earlier item's stores);
    // items past the end redo the last one and store the same values
    const int nh = RT * TL_BX;
    for (int i0 = tid; i0 < nh; i0 += 4 * TL_NT) {
        uint32_t wv[4][WT4 + 1];
#pragma unroll
        for (int u = 0; u < 4; u++) {
            const int i = min(i0 + u * TL_NT, nh - 1);
            const uint32_t *rp = tile + (i / TL_BX) * TL_P + ((i % TL_BX) >> 2);
#pragma unroll
            for (int k = 0; k <= WT4; k++) wv[u][k] = rp[k];
        }
#pragma unroll
        for (int u = 0; u < 4; u++) {
            const int i = min(i0 + u * TL_NT, nh - 1);
            const uint32_t sh = (uint32_t)(i & 3);  // pos & 3
            uint32_t h1 = 0, h2 = 0;
#pragma unroll
            for (int k = 0; k < WT4; k++) {
                uint32_t v = align_bytes(wv[u][k + 1], wv[u][k], sh);
                if (k == WT4 - 1) v &= mlast;
                h1 = dot4u(v, 0x01010101u, h1);
                h2 = dot4u(v, v, h2);
            }
            H1[i] = h1;
            H2[i] = h2;
        }
    }
    __syncthreads();
    {
        // lane: column pos, output rows RW*w .. RW*w + RW-1
        constexpr int RW = TL_BY / (TL_NT / 64);
        const int pos = l, oy0 = RW * w;
        uint32_t c1 = 0, c2 = 0;
#pragma unroll 8
        for (int j = 0; j < hT; j++) {
            c1 += H1[(oy0 + j) * TL_BX + pos];
            c2 += H2[(oy0 + j) * TL_BX + pos];
        }
        uint32_t v1[RW], v2[RW];
#pragma unroll
        for (int i = 0; i < RW; i++) {
            v1[i] = c1;
            v2[i] = c2;
            if (i < RW - 1) {
                c1 += H1[(oy0 + i + hT) * TL_BX + pos] - H1[(oy0 + i) * TL_BX + pos];
                c2 += H2[(oy0 + i + hT) * TL_BX + pos] - H2[(oy0 + i) * TL_BX + pos];
            }
        }
        __syncthreads();  // every read of the row sums is done
#pragma unroll
        for (int i = 0; i < RW; i++) {
            H1[(oy0 + i) * TL_BX + pos] = v1[i];
            H2[(oy0 + i) * TL_BX + pos] = v2[i];
        }
    }

    // ---- 2. SumIT
    const int tx = tid % TL_TX, ty = tid / TL_TX;
    uint32_t acc[TL_R][TL_PX];
#pragma unroll
    for (int dy = 0; dy < TL_R; dy++)
#pragma unroll
        for (int p = 0; p < TL_PX; p++) acc[dy][p] = 0;
    // Template rows in a ring of TL_R register slots: image row q meets
    // template row q - dy in output row dy, so row j sits in slot j % TL_R
    // and, with q stepping by TL_R in an unrolled body, every slot index is
    // static.  Template rows outside 0 .. hT-1 are zero (the ring starts
    // zeroed, the LDS template has 6 zero rows past hT), so the body has no
    // branch: the products with them add exactly 0 (the steps past
    // hT + TL_R - 2 read the spare tile rows, whatever they hold, against
    // zero rows).
    static_assert(TL_R - 1 <= 3 && 2 * (TL_R - 1) <= 6, "spare tile rows and zero template rows");
    uint32_t tr[TL_R][TW];
#pragma unroll
    for (int s = 0; s < TL_R; s++)
#pragma unroll
        for (int k = 0; k < TW; k++) tr[s][k] = 0;
    const int nq4 = (hT + TL_R - 1 + TL_R - 1) / TL_R * TL_R;
    for (int q0 = 0; q0 < nq4; q0 += TL_R) {
#pragma unroll
        for (int s = 0; s < TL_R; s++) {
            const int q = q0 + s;
#pragma unroll
            for (int k4 = 0; k4 < TW / 4; k4++) {
                const uint4 u = *(const uint4 *)&tw[q * TW + 4 * k4];
                tr[s][4 * k4] = u.x;
                tr[s][4 * k4 + 1] = u.y;
                tr[s][4 * k4 + 2] = u.z;
                tr[s][4 * k4 + 3] = u.w;
            }
            const uint32_t *rp = tile + (TL_R * ty + q) * TL_P + tx;
            uint32_t d[WT4 + 1];
#pragma unroll
            for (int k = 0; k <= WT4; k++) d[k] = rp[k];
            uint32_t v[TL_PX][WT4];
#pragma unroll
            for (int k = 0; k < WT4; k++) {
                v[0][k] = d[k];
                v[1][k] = align_bytes(d[k + 1], d[k], 1);
                v[2][k] = align_bytes(d[k + 1], d[k], 2);
                v[3][k] = align_bytes(d[k + 1], d[k], 3);
            }
#pragma unroll
            for (int dy = 0; dy < TL_R; dy++) {
                const int slot = (s - dy + TL_R) % TL_R;  // template row q - dy
#pragma unroll
                for (int k = 0; k < WT4; k++)
#pragma unroll
                    for (int p = 0; p < TL_PX; p++)
                        acc[dy][p] = dot4u(v[p][k], tr[slot][k], acc[dy][p]);
            }
        }
    }
    __syncthreads();  // SumI, SumISq in LDS

    // ---- 3. coefficients
    const size_t plane = a.oplane;
    const int xb = x0 + TL_PX * tx;
#pragma unroll
    for (int dy = 0; dy < TL_R; dy++) {
        const int oy = TL_R * ty + dy, y = y0 + oy;
        if (y >= a.Ho) break;
        const uint4 sI4 = *(const uint4 *)&H1[oy * TL_BX + TL_PX * tx];
        const uint4 sQ4 = *(const uint4 *)&H2[oy * TL_BX + TL_PX * tx];
        const uint32_t sI[4] = {sI4.x, sI4.y, sI4.z, sI4.w};
        const uint32_t sQ[4] = {sQ4.x, sQ4.y, sQ4.z, sQ4.w};
        float g[TL_PX];
#pragma unroll
        for (int p = 0; p < TL_PX; p++) {
            const long long sumI = sI[p];
            const long long num = K * (long long)acc[dy][p] - sumI * sumT;
            const long long varI = K * (long long)sQ[p] - sumI * sumI;
            g[p] = ncc_coef((float)num, (float)varI, varTf);
        }
        const size_t o = (size_t)y * a.op + xb;
        float *cp = a.coef + (size_t)t * plane + o;
        if (xb + TL_PX <= a.Wo) {
            __builtin_nontemporal_store((f4u){g[0], g[1], g[2], g[3]}, (f4u *)cp);
        } else {
#pragma unroll
            for (int p = 0; p < TL_PX; p++)
                if (xb + p < a.Wo) __builtin_nontemporal_store(g[p], cp + p);
        }
        if (a.sums) {
#pragma unroll
            for (int p = 0; p < TL_PX; p++) {
                if (xb + p >= a.Wo) break;
                if (t == 0) {
                    __builtin_nontemporal_store((int32_t)sI[p], a.sums + o + p);
                    __builtin_nontemporal_store((int32_t)sQ[p], a.sums + plane + o + p);
                }
                __builtin_nontemporal_store((int32_t)acc[dy][p], a.sums + (size_t)(2 + t) * plane + o + p);
            }
        }
    }
}

size_t tile_lds_bytes(int wT, int hT) {
    const int WT4 = (wT + 3) / 4, TW = (WT4 + 3) / 4 * 4, RT = TL_BY + hT - 1;
    return ((size_t)(RT + 3) * TL_P + 2 * (size_t)RT * TL_BX + (size_t)(hT + 6) * TW) * sizeof(uint32_t);
}

template <int WT4>
hipError_t launch_tile(const CorrArgs &a, int t, hipStream_t st) {
    static bool attr_set[2][NCC_MAX_DEVICES] = {};
    const bool a4 = ((uintptr_t)a.img & 3) == 0 && a.ip % 4 == 0;
    const size_t lds = tile_lds_bytes(a.wT, a.hT);
    hipError_t e = set_once(attr_set[a4], [a4] {
        const void *fn = a4 ? (const void *)corr_tile<WT4, true> : (const void *)corr_tile<WT4, false>;
        return hipFuncSetAttribute(fn, hipFuncAttributeMaxDynamicSharedMemorySize,
                                   (int)tile_lds_bytes(4 * TL_MAXW4, TL_MAXH));
    });
    if (e != hipSuccess) return e;
    const int ntx = (a.Wo + TL_BX - 1) / TL_BX, nty = (a.Ho + TL_BY - 1) / TL_BY;
    dim3 grid(xcd_grid(ntx * nty)), block(TL_NT);
    if (a4)
        hipLaunchKernelGGL((corr_tile<WT4, true>), grid, block, lds, st, a, t, ntx, nty);
    else
        hipLaunchKernelGGL((corr_tile<WT4, false>), grid, block, lds, st, a, t, ntx, nty);
    return hipGetLastError();
}

}  // namespace

bool corr_tile_supported(int wT, int hT) {
    return wT >= 1 && wT <= 4 * TL_MAXW4 && hT >= 1 && hT <= TL_MAXH;
}

hipError_t corr_tile_launch(const CorrArgs &a, int t, hipStream_t st) {
    switch ((a.wT + 3) / 4) {
        case 1: return launch_tile<1>(a, t, st);
        case 2: return launch_tile<2>(a, t, st);
        case 3: return launch_tile<3>(a, t, st);
        case 4: return launch_tile<4>(a, t, st);
        case 5: return launch_tile<5>(a, t, st);
        case 6: return launch_tile<6>(a, t, st);
        case 7: return launch_tile<7>(a, t, st);
        case 8: return launch_tile<8>(a, t, st);
        default: return hipErrorNotSupported;
    }
}

}  // namespace ncc
