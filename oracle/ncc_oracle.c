/*
 * Plain CPU oracle for normalized cross-correlation (NCC) template matching
 * of 8-bit images with summed-area-table denominators.
 *
 * TEST INFRASTRUCTURE ONLY.  This file is the slow, obviously correct
 * definition that the GPU library is checked against.  Only the test suite,
 * the smoke check and the benchmark's CPU-baseline leg may load it.  It
 * shares no code, header, table or helper with the GPU library, and the GPU
 * library never calls it.
 *
 * Sources (the pages this follows):
 *   [HB-SAT]  The CUDA Handbook, ch. 15, section 15.8 "The Denominator:
 *             Summed Area Tables": the table definition (the sum of every
 *             pixel above and to the left, inclusive), the four-corner
 *             box-sum identity (Figure 15-7), and the width analysis (int64
 *             table, uint32 row running sums).  The table and the box query
 *             are written here from those definitions: the table by the 2-D
 *             inclusion-exclusion recurrence over a zero border, the query
 *             as the identity's four signed corners.
 *   [HB-SM]   The CUDA Handbook, ch. 15, "Image in shared memory": the
 *             corrShared_kernel listing, whose per-window loop accumulates
 *             SumI, SumISq and SumIT over a wTemplate x hTemplate window
 *             anchored at the window's top-left pixel, then calls
 *             CorrelationValue(SumI, SumISq, SumIT, SumT, cPixels, ...).
 *
 * Readings taken where the pages are silent:
 *   - CorrelationValue's body is not on the pages.  The coefficient is the
 *     textbook Pearson / Lewis normalized cross-correlation in sum form:
 *       num  = K*SumIT - SumI*SumT
 *       varI = K*SumISq - SumI^2,  varT = K*SumTSq - SumT^2
 *       gamma = num / sqrt(varI * varT)
 *     with K = wT*hT the pixel count.  gamma = 0 when varI == 0 or
 *     varT == 0.  num, varI and varT are exact int64 integers; the only
 *     rounding is one IEEE double evaluation, then one rounding to float.
 *   - Output is valid mode: Wo = W-wT+1 by Ho = H-hT+1 positions, position
 *     (x,y) covering rows y..y+hT-1 and columns x..x+wT-1.
 *   - The table is inclusive: S(x,y) sums rows 0..y and columns 0..x.
 *   - satBox accepts 0 <= x0 <= x1 <= W, 0 <= y0 <= y1 <= H; an empty box
 *     (x0 == x1 or y0 == y1) sums to 0.
 *
 * Every function loops in the plainest order.  The only parallelism is an
 * optional OpenMP split over output rows in oracle_correlate (each row is
 * computed independently, so results do not depend on the thread count).
 */
#include <stdint.h>
#include <stddef.h>
#include <math.h>
#include <stdlib.h>
#ifdef _OPENMP
#include <omp.h>
#endif

/* [HB-SAT] width analysis: each row's running sum is at most W*255^2 and is
 * stored as uint32.  Writes the inclusive row running sums of I and I^2. */
void oracle_row_partials(const uint8_t *img, int W, int H,
                         uint32_t *R1, uint32_t *R2)
{
    for (int y = 0; y < H; y++) {
        uint32_t s1 = 0, s2 = 0;
        for (int x = 0; x < W; x++) {
            uint32_t v = img[(size_t)y * W + x];
            s1 += v;
            s2 += v * v;
            R1[(size_t)y * W + x] = s1;
            R2[(size_t)y * W + x] = s2;
        }
    }
}

/* Table element (x, y), with everything left of column 0 or above row 0
 * read as zero: the zero border that [HB-SAT] gives the table's two leading
 * edges. */
static int64_t tbl_at(const int64_t *T, int W, int x, int y)
{
    return (x < 0 || y < 0) ? 0 : T[(size_t)y * W + x];
}

/* [HB-SAT] summed-area tables S (of I) and Q (of I^2), int64, row-major with
 * pitch W, inclusive: S(x,y) is the sum of I over every pixel (x',y') with
 * x' <= x and y' <= y.  Filled in row-major order from the identity
 *   S(x,y) = I(x,y) + S(x-1,y) + S(x,y-1) - S(x-1,y-1)
 * (the box [0,x] x [0,y] is its last pixel plus the box ending one column to
 * the left plus the box ending one row up, minus the box both of those
 * contain), with the zero border.  Returns 0, or -1 on bad sizes. */
int oracle_sat_build(const uint8_t *img, int W, int H, int64_t *S, int64_t *Q)
{
    if (W < 1 || H < 1 || !img || !S || !Q) return -1;
    for (int y = 0; y < H; y++)
        for (int x = 0; x < W; x++) {
            int64_t v = img[(size_t)y * W + x];
            S[(size_t)y * W + x] = v + tbl_at(S, W, x - 1, y) + tbl_at(S, W, x, y - 1)
                                   - tbl_at(S, W, x - 1, y - 1);
            Q[(size_t)y * W + x] = v * v + tbl_at(Q, W, x - 1, y) + tbl_at(Q, W, x, y - 1)
                                   - tbl_at(Q, W, x - 1, y - 1);
        }
    return 0;
}

/* [HB-SAT] four-corner identity (Figure 15-7): the sum over the half-open
 * box [x0,x1) x [y0,y1) is the table at the box's last pixel, minus the
 * table at the pixel above its top-right corner and at the pixel left of its
 * bottom-left corner (each of those boxes covers one strip outside the box),
 * plus the table at the pixel diagonally above-left of its first pixel (the
 * part both strips removed), every corner read through the zero border.
 * Empty boxes sum to 0.  Rectangles outside the domain abort (a caller bug
 * in a test). */
int64_t oracle_sat_box(const int64_t *S, int W, int H,
                       int x0, int y0, int x1, int y1)
{
    if (x0 < 0 || y0 < 0 || x1 > W || y1 > H || x0 > x1 || y0 > y1) abort();
    if (x0 == x1 || y0 == y1) return 0;
    return tbl_at(S, W, x1 - 1, y1 - 1) - tbl_at(S, W, x1 - 1, y0 - 1)
           - tbl_at(S, W, x0 - 1, y1 - 1) + tbl_at(S, W, x0 - 1, y0 - 1);
}

/* Batch of box queries; rects holds n records {x0, y0, x1, y1}. */
void oracle_box_batch(const int64_t *S, int W, int H,
                      const int32_t *rects, int64_t n, int64_t *out)
{
    for (int64_t i = 0; i < n; i++)
        out[i] = oracle_sat_box(S, W, H, rects[4 * i + 0], rects[4 * i + 1],
                                rects[4 * i + 2], rects[4 * i + 3]);
}

/* Template constants: SumT, SumTSq and varT = K*SumTSq - SumT^2 (exact). */
void oracle_template_stats(const uint8_t *tpl, int wT, int hT,
                           int64_t *sumT, int64_t *sumTSq, int64_t *varT)
{
    int64_t K = (int64_t)wT * hT, s1 = 0, s2 = 0;
    for (int j = 0; j < hT; j++)
        for (int i = 0; i < wT; i++) {
            int64_t t = tpl[(size_t)j * wT + i];
            s1 += t;
            s2 += t * t;
        }
    *sumT = s1;
    *sumTSq = s2;
    *varT = K * s2 - s1 * s1;
}

/* The coefficient from the exact integer sums (reading of CorrelationValue
 * stated in the file header). */
float oracle_coefficient(int64_t K, int64_t sumI, int64_t sumISq,
                         int64_t sumIT, int64_t sumT, int64_t sumTSq)
{
    int64_t num = K * sumIT - sumI * sumT;
    int64_t varI = K * sumISq - sumI * sumI;
    int64_t varT = K * sumTSq - sumT * sumT;
    if (varI == 0 || varT == 0) return 0.0f;
    double g = (double)num / sqrt((double)varI * (double)varT);
    return (float)g;
}

/* [HB-SM] the per-window product sum: SumIT(x,y) = sum over j < hT,
 * i < wT of I[y+j][x+i] * T[j][i]. */
static int64_t window_sum_it(const uint8_t *img, int W, const uint8_t *t,
                             int wT, int hT, int x, int y)
{
    int64_t s = 0;
    for (int j = 0; j < hT; j++)
        for (int i = 0; i < wT; i++)
            s += (int64_t)img[(size_t)(y + j) * W + (x + i)] *
                 (int64_t)t[(size_t)j * wT + i];
    return s;
}

/* One position: SumI and SumISq from the tables by the four-corner rule,
 * SumIT by the direct double loop, then the coefficient for every template.
 * sums (nullable) receives {SumI, SumISq, SumIT_0 .. SumIT_{nTpl-1}};
 * coef receives nTpl values. */
static void one_position(const uint8_t *img, int W, int H,
                         const int64_t *S, const int64_t *Q,
                         const uint8_t *tpl, int wT, int hT, int nTpl,
                         const int64_t *sT, const int64_t *sTSq,
                         int x, int y, int64_t *sums, float *coef)
{
    int64_t K = (int64_t)wT * hT;
    int64_t sumI = oracle_sat_box(S, W, H, x, y, x + wT, y + hT);
    int64_t sumISq = oracle_sat_box(Q, W, H, x, y, x + wT, y + hT);
    if (sums) { sums[0] = sumI; sums[1] = sumISq; }
    for (int t = 0; t < nTpl; t++) {
        const uint8_t *T = tpl + (size_t)t * wT * hT;
        int64_t sumIT = window_sum_it(img, W, T, wT, hT, x, y);
        if (sums) sums[2 + t] = sumIT;
        coef[t] = oracle_coefficient(K, sumI, sumISq, sumIT, sT[t], sTSq[t]);
    }
}

/* Valid-mode correlation of an H x W image with nTpl templates of hT x wT.
 *   sums_out (nullable): int32 planes [(2+nTpl)][Ho][Wo]: SumI, SumISq,
 *                        then SumIT of each template.
 *   coef_out:            float planes [nTpl][Ho][Wo].
 * nthreads <= 0 uses the OpenMP default.  Returns 0, or -1 on bad sizes or
 * an allocation failure. */
int oracle_correlate(const uint8_t *img, int W, int H,
                     const uint8_t *tpl, int wT, int hT, int nTpl,
                     int32_t *sums_out, float *coef_out, int nthreads)
{
    if (W < 1 || H < 1 || wT < 1 || hT < 1 || wT > W || hT > H || nTpl < 1)
        return -1;
    int Wo = W - wT + 1, Ho = H - hT + 1;
    size_t plane = (size_t)Wo * Ho;
    int64_t *S = malloc(sizeof(int64_t) * (size_t)W * H);
    int64_t *Q = malloc(sizeof(int64_t) * (size_t)W * H);
    int64_t *sT = malloc(sizeof(int64_t) * nTpl);
    int64_t *sTSq = malloc(sizeof(int64_t) * nTpl);
    if (!S || !Q || !sT || !sTSq) {
        free(S); free(Q); free(sT); free(sTSq);
        return -1;
    }
    oracle_sat_build(img, W, H, S, Q);
    for (int t = 0; t < nTpl; t++) {
        int64_t v;
        oracle_template_stats(tpl + (size_t)t * wT * hT, wT, hT,
                              &sT[t], &sTSq[t], &v);
    }
#ifdef _OPENMP
    if (nthreads <= 0) nthreads = omp_get_max_threads();
#pragma omp parallel for schedule(dynamic, 1) num_threads(nthreads)
#endif
    for (int y = 0; y < Ho; y++) {
        int64_t *sums = malloc(sizeof(int64_t) * (2 + (size_t)nTpl));
        float *coef = malloc(sizeof(float) * (size_t)nTpl);
        for (int x = 0; x < Wo; x++) {
            one_position(img, W, H, S, Q, tpl, wT, hT, nTpl, sT, sTSq,
                         x, y, sums, coef);
            size_t o = (size_t)y * Wo + x;
            for (int t = 0; t < nTpl; t++) coef_out[(size_t)t * plane + o] = coef[t];
            if (sums_out)
                for (int p = 0; p < 2 + nTpl; p++)
                    sums_out[(size_t)p * plane + o] = (int32_t)sums[p];
        }
        free(sums);
        free(coef);
    }
    free(S); free(Q); free(sT); free(sTSq);
    return 0;
}

/* The same computation at n chosen positions only, for checking outputs of
 * images too large to correlate in full on the CPU.  S and Q are the tables
 * from oracle_sat_build.  pos holds n records {x, y} with 0 <= x < Wo and
 * 0 <= y < Ho.  sums (nullable) receives n records of (2+nTpl) int64;
 * coef receives n records of nTpl floats.  Returns 0, or -1 on bad input. */
int oracle_correlate_at(const uint8_t *img, int W, int H,
                        const int64_t *S, const int64_t *Q,
                        const uint8_t *tpl, int wT, int hT, int nTpl,
                        const int32_t *pos, int64_t n,
                        int64_t *sums, float *coef, int nthreads)
{
    if (W < 1 || H < 1 || wT < 1 || hT < 1 || wT > W || hT > H || nTpl < 1)
        return -1;
    int Wo = W - wT + 1, Ho = H - hT + 1;
    for (int64_t i = 0; i < n; i++)
        if (pos[2 * i] < 0 || pos[2 * i] >= Wo || pos[2 * i + 1] < 0 ||
            pos[2 * i + 1] >= Ho)
            return -1;
    int64_t *sT = malloc(sizeof(int64_t) * nTpl);
    int64_t *sTSq = malloc(sizeof(int64_t) * nTpl);
    if (!sT || !sTSq) { free(sT); free(sTSq); return -1; }
    for (int t = 0; t < nTpl; t++) {
        int64_t v;
        oracle_template_stats(tpl + (size_t)t * wT * hT, wT, hT,
                              &sT[t], &sTSq[t], &v);
    }
#ifdef _OPENMP
    if (nthreads <= 0) nthreads = omp_get_max_threads();
#pragma omp parallel for schedule(dynamic, 64) num_threads(nthreads)
#endif
    for (int64_t i = 0; i < n; i++)
        one_position(img, W, H, S, Q, tpl, wT, hT, nTpl, sT, sTSq,
                     pos[2 * i], pos[2 * i + 1],
                     sums ? sums + (size_t)i * (2 + nTpl) : NULL,
                     coef + (size_t)i * nTpl);
    free(sT); free(sTSq);
    return 0;
}

/* Threads an OpenMP region started with nthreads would use (1 without
 * OpenMP): lets the benchmark report the cores the baseline actually used. */
int oracle_threads(int nthreads)
{
#ifdef _OPENMP
    int used = 1;
    if (nthreads <= 0) nthreads = omp_get_max_threads();
#pragma omp parallel num_threads(nthreads)
    {
#pragma omp single
        used = omp_get_num_threads();
    }
    return used;
#else
    (void)nthreads;
    return 1;
#endif
}
