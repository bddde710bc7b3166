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
// evaluated modulo 2^32: exact, since |num| <= K^2 * 127.5^2 < 2^31 for the
// K <= 256 this kernel takes.
//
// Operand layout (16x16x64, checked on the device): lane 16*g + m of the A
// operand holds 16 bytes of row m, lane 16*g + n of B the same 16 k-slots of
// column n, and lane 16*g + n of the result holds rows 4g..4g+3 of column n.
// The k order inside the 64 is the same for A and B, so chunk c = 4*kstep + g
// is a 16-byte piece of one template row (row c / NB16, bytes 16*(c % NB16)).
//
// A workgroup (4 wavefronts) owns 64 x 16 output positions and up to 64
// templates (4 blocks of 16).  The image tile + halo is staged in LDS; each
// wavefront takes groups of 16 positions of one row (the A rows), byte-aligns
// and offsets their chunks, and runs KSTEPS x 4 MFMAs.  Window sums SumI and
// SumISq of the 16 positions come from the same operands (v_dot4_i32_i8),
// once for all templates.
#include "ncc_internal.h"

namespace ncc {

namespace {

typedef int v4i __attribute__((ext_vector_type(4)));
typedef float f4u __attribute__((ext_vector_type(4), aligned(4)));

constexpr int BX = 64;  // positions per workgroup row
constexpr int BY = 16;  // rows per workgroup

template <int KSTEPS, bool FULL>
__global__ __launch_bounds__(256) void corr_bank(CorrArgs a, int nb16, int pitch, int rowsT) {
    extern __shared__ uint32_t tile[];  // rowsT x pitch bytes
    const int tid = threadIdx.x, w = tid >> 6, l = tid & 63;
    const int g = l >> 4, m = l & 15;
    const int x0 = blockIdx.x * BX, y0 = blockIdx.y * BY;
    const int pw = pitch / 4;
    const int K = a.wT * a.hT;

    // stage tile + halo (bytes outside the image are 0)
    for (int i = tid; i < rowsT * pw; i += 256) {
        const int r = i / pw, c = i % pw;
        const int y = y0 + r, xb = x0 + 4 * c;
        uint32_t v = 0;
        if (y < a.H) {
            const uint8_t *row = a.img + (size_t)y * a.W;
            if (xb + 3 < a.W && ((((uintptr_t)row + xb) & 3) == 0)) {
                v = *(const uint32_t *)(row + xb);
            } else {
#pragma unroll
                for (int b = 0; b < 4; b++)
                    if (xb + b < a.W) v |= (uint32_t)row[xb + b] << (8 * b);
            }
        }
        tile[i] = v;
    }

    // B operands and per-template constants of this workgroup's 4 blocks
    const int gbase = blockIdx.z * 4;
    const int ngroups = (a.nTpl + 15) / 16;
    v4i bop[4][KSTEPS];
    int ca[4], cb[4];
    float rT[4];
#pragma unroll
    for (int nb = 0; nb < 4; nb++) {
        const int gg = gbase + nb;
        const int tt = gg * 16 + m;  // this lane's template in block nb (lane n = m)
        if (gg < ngroups) {
#pragma unroll
            for (int ks = 0; ks < KSTEPS; ks++)
                bop[nb][ks] = *(const v4i *)(a.mfma + (((size_t)gg * KSTEPS + ks) * 64 + l) * 16);
        } else {
#pragma unroll
            for (int ks = 0; ks < KSTEPS; ks++) bop[nb][ks] = (v4i){0, 0, 0, 0};
        }
        if (gg < ngroups && tt < a.nTpl) {
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
    const int nblk = min(4, ngroups - gbase);

    // byte masks of this lane's chunks (only for shapes that pad)
    uint32_t msk[KSTEPS][4];
#pragma unroll
    for (int ks = 0; ks < KSTEPS; ks++) {
        const int c = 4 * ks + g, j = c / nb16, ib = c % nb16;
        const int nbytes = (j < a.hT) ? min(16, a.wT - 16 * ib) : 0;
#pragma unroll
        for (int k = 0; k < 4; k++) {
            const int nbk = nbytes - 4 * k;
            msk[ks][k] = nbk <= 0 ? 0u : byte_mask(nbk);
        }
    }
    __syncthreads();

    const size_t plane = (size_t)a.Ho * a.Wo;
    // 16 rows x 4 groups of 16 positions; wavefront w takes rows w, w+4, ...
    for (int it = 0; it < BY / 4 * (BX / 16); it++) {
        const int yy = w + 4 * (it / (BX / 16));
        const int xg = 16 * (it % (BX / 16));
        const int y = y0 + yy;
        if (y >= a.Ho) break;
        if (x0 + xg >= a.Wo) continue;

        // A operands: row m = position xg + m, chunk c = 4*ks + g
        v4i A[KSTEPS];
        int sI = 0, sQ = 0;
        const int px = xg + m;
#pragma unroll
        for (int ks = 0; ks < KSTEPS; ks++) {
            const int c = 4 * ks + g, j = c / nb16, ib = c % nb16;
            const int jj = j < a.hT ? j : 0;
            const int off = (yy + jj) * pitch + px + 16 * ib;
            const uint32_t *p = tile + (off >> 2);
            const uint32_t sh = (uint32_t)(off & 3);
            uint32_t d0 = p[0], d1 = p[1], d2 = p[2], d3 = p[3], d4 = p[4];
            uint32_t v[4];
            v[0] = align_bytes(d1, d0, sh) ^ 0x80808080u;
            v[1] = align_bytes(d2, d1, sh) ^ 0x80808080u;
            v[2] = align_bytes(d3, d2, sh) ^ 0x80808080u;
            v[3] = align_bytes(d4, d3, sh) ^ 0x80808080u;
#pragma unroll
            for (int k = 0; k < 4; k++) {
                const uint32_t vm = FULL ? v[k] : (v[k] & msk[ks][k]);
                sI = __builtin_amdgcn_sdot4((int)vm, 0x01010101, sI, false);
                sQ = __builtin_amdgcn_sdot4((int)vm, (int)vm, sQ, false);
            }
            A[ks] = (v4i){(int)v[0], (int)v[1], (int)v[2], (int)v[3]};
        }
        // sums over the four chunk groups of position m
        sI += __shfl_xor(sI, 16);
        sI += __shfl_xor(sI, 32);
        sQ += __shfl_xor(sQ, 16);
        sQ += __shfl_xor(sQ, 32);
        const int sumI = sI + 128 * K;
        const int sumISq = sQ + 256 * sI + 16384 * K;
        const unsigned varI = (unsigned)K * (unsigned)sumISq - (unsigned)sumI * (unsigned)sumI;
        const float rI = varI ? __builtin_amdgcn_rsqf((float)varI) : 0.0f;
        // this lane's result rows are positions 4g .. 4g+3
        int sumIi[4];
        float rIi[4];
#pragma unroll
        for (int i = 0; i < 4; i++) {
            sumIi[i] = __shfl(sumI, 4 * g + i);
            rIi[i] = __shfl(rI, 4 * g + i);
        }
        const int xb = x0 + xg + 4 * g;  // first output column of this lane
        const size_t orow = (size_t)y * a.Wo;
        if (a.sums && blockIdx.z == 0 && g == 0) {
            const int xm = x0 + xg + m;
            if (xm < a.Wo) {
                __builtin_nontemporal_store(sumI, a.sums + orow + xm);
                __builtin_nontemporal_store(sumISq, a.sums + plane + orow + xm);
            }
        }

        v4i acc[4];
#pragma unroll
        for (int nb = 0; nb < 4; nb++) acc[nb] = (v4i){0, 0, 0, 0};
#pragma unroll
        for (int ks = 0; ks < KSTEPS; ks++)
#pragma unroll
            for (int nb = 0; nb < 4; nb++)
                if (nb < nblk)
                    acc[nb] = __builtin_amdgcn_mfma_i32_16x16x64_i8(A[ks], bop[nb][ks], acc[nb], 0, 0, 0);

#pragma unroll
        for (int nb = 0; nb < 4; nb++) {
            if (nb >= nblk) break;
            const int tt = (gbase + nb) * 16 + m;
            if (tt >= a.nTpl) continue;
            float gv[4];
#pragma unroll
            for (int i = 0; i < 4; i++) {
                const int num = (int)((unsigned)K * (unsigned)acc[nb][i] +
                                      (unsigned)sumIi[i] * (unsigned)ca[nb] + (unsigned)cb[nb]);
                const float gm = (float)num * (rIi[i] * rT[nb]);
                gv[i] = __builtin_amdgcn_fmed3f(gm, -1.0f, 1.0f);
            }
            float *dst = a.coef + (size_t)tt * plane + orow + xb;
            if (xb + 3 < a.Wo) {
                f4u vv = {gv[0], gv[1], gv[2], gv[3]};
                __builtin_nontemporal_store(vv, (f4u *)dst);
            } else {
#pragma unroll
                for (int i = 0; i < 4; i++)
                    if (xb + i < a.Wo) __builtin_nontemporal_store(gv[i], dst + i);
            }
            if (a.sums) {
                int32_t *sd = a.sums + (size_t)(2 + tt) * plane + orow + xb;
                const TStat ts = a.stats[tt];
#pragma unroll
                for (int i = 0; i < 4; i++)
                    if (xb + i < a.Wo)
                        __builtin_nontemporal_store(
                            (int)(acc[nb][i] + 128 * (sumIi[i] + (int)ts.sumT) - 16384 * K), sd + i);
            }
        }
    }
}

void bank_geometry(int wT, int hT, int *pitch, int *rowsT) {
    const int nb16 = (wT + 15) / 16;
    *pitch = ((BX + 16 * nb16 + 4) + 15) / 16 * 16;
    *rowsT = BY + hT - 1;
}

}  // namespace

bool corr_bank_supported(int wT, int hT, int nTpl) {
    const int chunks = hT * ((wT + 15) / 16);
    return nTpl > 1 && chunks <= 16 && wT * hT <= 256;
}

hipError_t corr_bank_launch(const CorrArgs &a, hipStream_t st) {
    const int nb16 = (a.wT + 15) / 16;
    const int ks = (a.hT * nb16 + 3) / 4;
    int pitch, rowsT;
    bank_geometry(a.wT, a.hT, &pitch, &rowsT);
    const size_t lds = (size_t)pitch * rowsT;
    const bool full = (a.wT % 16 == 0) && ((a.hT * nb16) % 4 == 0);
    dim3 grid((a.Wo + BX - 1) / BX, (a.Ho + BY - 1) / BY, ((a.nTpl + 15) / 16 + 3) / 4);
#define NCC_BANK_CASE(KS)                                                                    \
    case KS:                                                                                 \
        if (full)                                                                            \
            hipLaunchKernelGGL((corr_bank<KS, true>), grid, dim3(256), lds, st, a, nb16, pitch, \
                               rowsT);                                                       \
        else                                                                                 \
            hipLaunchKernelGGL((corr_bank<KS, false>), grid, dim3(256), lds, st, a, nb16,    \
                               pitch, rowsT);                                                \
        break;
    switch (ks) {
        NCC_BANK_CASE(1)
        NCC_BANK_CASE(2)
        NCC_BANK_CASE(3)
        NCC_BANK_CASE(4)
        default:
            return hipErrorNotSupported;
    }
#undef NCC_BANK_CASE
    return hipGetLastError();
}

}  // namespace ncc
