// Template constants and packed template operands.
//
// The correlation coefficient needs, per template, SumT, SumTSq and the
// template-only denominator factor (the corrShared_kernel listing of The
// CUDA Handbook ch. 15 "Image in shared memory" passes g_SumT, cPixels and
// fDenomExp in).  Here they are exact int64 sums, varT = K*SumTSq - SumT^2
// and its float forms.  The kernel also packs the template rows into the
// layouts the correlation kernels read.
#include "ncc_internal.h"

namespace ncc {

namespace {

constexpr int WG = 1024;

// One workgroup per template (1024 lanes: a large template's loads spread
// over many wavefronts instead of long per-lane loops).
__global__ __launch_bounds__(WG) void tpl_prep(const uint8_t *__restrict__ tpl, int wT, int hT,
                                               uint32_t *__restrict__ rows,
                                               int8_t *__restrict__ mfma, int ksteps,
                                               TStat *__restrict__ stats) {
    const int t = blockIdx.x, tid = threadIdx.x;
    const int K = wT * hT;
    const uint8_t *T = tpl + (size_t)t * K;

    // exact sums
    unsigned long long s1 = 0, s2 = 0;
#pragma unroll 4
    for (int i = tid; i < K; i += WG) {
        unsigned v = T[i];
        s1 += v;
        s2 += v * v;
    }
    __shared__ unsigned long long red[2][WG];
    red[0][tid] = s1;
    red[1][tid] = s2;
    __syncthreads();
    for (int h = WG / 2; h > 0; h >>= 1) {
        if (tid < h) {
            red[0][tid] += red[0][tid + h];
            red[1][tid] += red[1][tid + h];
        }
        __syncthreads();
    }
    if (tid == 0) {
        long long sumT = (long long)red[0][0], sumTSq = (long long)red[1][0];
        long long varT = (long long)K * sumTSq - sumT * sumT;
        TStat st;
        st.sumT = sumT;
        st.sumTSq = sumTSq;
        st.varT = varT;
        st.varTf = (float)varT;
        st.rT = varT > 0 ? (float)(1.0 / sqrt((double)varT)) : 0.0f;
        stats[t] = st;
    }

    // rows padded to whole dwords
    const int wt4 = (wT + 3) / 4;
    uint32_t *R = rows + (size_t)t * hT * wt4;
#pragma unroll 2
    for (int i = tid; i < hT * wt4; i += WG) {
        const int j = i / wt4, k = i % wt4;
        uint32_t v = 0;
        for (int b = 0; b < 4; b++) {
            int c = 4 * k + b;
            if (c < wT) v |= (uint32_t)T[j * wT + c] << (8 * b);
        }
        R[i] = v;
    }

    // matrix-core operands: group g16 of 16 templates, lane = 16*q + n
    if (mfma != nullptr) {
        const int nb16 = (wT + 15) / 16;
        const int g16 = t / 16, n = t % 16;
        int8_t *M = mfma + (size_t)g16 * ksteps * 64 * 16;
        for (int i = tid; i < ksteps * 4 * 16; i += WG) {
            const int kstep = i / 64, q = (i / 16) % 4, byte = i % 16;
            const int c = 4 * kstep + q;  // chunk
            const int j = c / nb16, col = 16 * (c % nb16) + byte;
            int8_t v = 0;
            if (j < hT && col < wT) v = (int8_t)((int)T[j * wT + col] - 128);
            M[((size_t)kstep * 64 + 16 * q + n) * 16 + byte] = v;
        }
    }
}

// Zero operands of the padding templates of the last group of 16.
__global__ void tpl_pad_zero(int8_t *mfma, size_t off, size_t n) {
    for (size_t i = (size_t)blockIdx.x * blockDim.x + threadIdx.x; i < n;
         i += (size_t)gridDim.x * blockDim.x)
        mfma[off + i] = 0;
}

}  // namespace

size_t tpl_rows_bytes(int wT, int hT, int nTpl) {
    return (size_t)nTpl * hT * ((wT + 3) / 4) * 4;
}

static int bank_ksteps(int wT, int hT) {
    int chunks = hT * ((wT + 15) / 16);
    return (chunks + 3) / 4;
}

size_t tpl_mfma_bytes(int wT, int hT, int nTpl) {
    int groups = (nTpl + 15) / 16;
    return (size_t)groups * bank_ksteps(wT, hT) * 64 * 16;
}

hipError_t tpl_prep_launch(const uint8_t *tpl, int wT, int hT, int nTpl, uint32_t *rows,
                           int8_t *mfma, TStat *stats, hipStream_t st) {
    const int ks = bank_ksteps(wT, hT);
    if (mfma != nullptr && (nTpl % 16) != 0) {
        // templates nTpl .. 16*groups-1 do not exist: their operands must be 0
        // in every lane slot they own, which is every slot with n >= nTpl % 16
        // of the last group; clear the whole last group, then let the real
        // templates overwrite their own slots.
        size_t per = (size_t)ks * 64 * 16;
        size_t off = (size_t)(nTpl / 16) * per;
        hipLaunchKernelGGL(tpl_pad_zero, dim3(64), dim3(256), 0, st, mfma, off, per);
        hipError_t e = hipGetLastError();
        if (e != hipSuccess) return e;
    }
    hipLaunchKernelGGL(tpl_prep, dim3(nTpl), dim3(WG), 0, st, tpl, wT, hT, rows, mfma, ks, stats);
    return hipGetLastError();
}

}  // namespace ncc
