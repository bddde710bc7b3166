/*
 * ncc.h -- C ABI of libncc.so: normalized cross-correlation (NCC) template
 * matching of 8-bit images, with window sums from summed-area tables, on
 * AMD Instinct MI355X (gfx950).
 *
 * The operations follow The CUDA Handbook, chapter 15:
 *   - "Image in shared memory": the per-window accumulation of SumI, SumISq
 *     and SumIT over a wT x hT template (corrShared_kernel listing) and the
 *     coefficient computed from them (CorrelationValue, whose body the page
 *     does not print; this library uses the textbook Pearson coefficient,
 *     stated at ncc_correlate below).
 *   - Section 15.8 "The Denominator: Summed Area Tables": the inclusive
 *     summed-area table of I and of I^2 (int64, uint32 row running sums,
 *     built as a row scan then a column scan) and the four-corner satBox
 *     query with the table's two leading edges read as zero.
 *
 * Conventions for every entry point:
 *   - Images are H rows x W columns of uint8, row-major, dense (pitch = W),
 *     except where an entry point takes a pitch.
 *   - Buffer arguments are DEVICE pointers (memory from hipMalloc or from a
 *     framework allocator on the current device).  The caller allocates and
 *     owns them; the library never frees or keeps them.
 *   - `stream` is a hipStream_t passed as void* (NULL = the null stream).
 *     Work is enqueued on it and the call returns without waiting for it.
 *   - Arguments are validated on the host before anything is launched; a
 *     rejected call launches nothing and leaves every output untouched.
 *   - Return value: NCC_OK or a negative NCC_E* code (ncc_strerror names it).
 *   - The library keeps a per-device, per-stream workspace cache (growing,
 *     freed by ncc_release).  Calls on one stream are ordered by the stream;
 *     calls on different streams use different workspaces.
 *   - HIP graphs: a call recorded into a graph during stream capture keeps
 *     using that stream's workspace when the graph is replayed.  A block
 *     that a later call outgrows is retired, not freed, so replays stay
 *     valid until ncc_release (after which graphs must be captured again).
 *     A replay shares the workspace with every other call made on the
 *     capturing stream: replays and such calls must not run concurrently.
 *   - Routes and tuning: process-wide settings of ncc_set_option, read at
 *     every call; the defaults need no setting.  Nothing is read from the
 *     environment.
 */
#ifndef NCC_H
#define NCC_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

#define NCC_OK 0
#define NCC_EINVAL (-1)        /* null pointer, size < 1, template larger than image ... */
#define NCC_ERANGE (-2)        /* sizes past the integer widths the method relies on */
#define NCC_ENOMEM (-3)        /* workspace allocation failed */
#define NCC_EHIP (-4)          /* a HIP runtime call or kernel launch failed */
#define NCC_EUNSUPPORTED (-5)  /* shape this build has no kernel for (see ncc_correlate) */

/* Largest image width: one row's running sum of squares, at most W*255^2,
 * must fit the uint32 row partials of the table build (section 15.8 width
 * analysis): W*65025 <= 2^32 - 1. */
#define NCC_MAX_WIDTH 66051
/* Largest template pixel count: SumISq <= K*255^2 and SumIT <= K*255^2 must
 * fit the int32 sums of the window loop (corrShared_kernel accumulates in
 * int): K*65025 <= 2^31 - 1. */
#define NCC_MAX_TEMPLATE_PIXELS 33025

/*
 * ncc_sat_build -- summed-area tables of an image (section 15.8: table
 * definition, width analysis, row-scan-then-column-scan build).
 *
 *   img  [H][W] uint8, device.
 *   S    [H][W] int64, device, written: S(x,y) = sum of I over rows 0..y and
 *        columns 0..x (inclusive).
 *   Q    [H][W] int64, device, written: the same sum of I^2.
 *
 * The default build is two passes with no waiting between workgroups.  The
 * single-pass build (ncc_set_option(NCC_OPT_SAT_BUILD, NCC_SAT_SINGLE_PASS);
 * section 15.8's decoupled look-back, one read of the image) has bounded
 * waits: if one gives up, or the stream's build state was left inconsistent,
 * the tiles concerned are written as INT64_MIN and the failure is reported
 * as NCC_EHIP by ncc_stream_status, or by the next call on that stream that
 * uses the single-pass build, which also resets the state.
 *
 * Errors: NCC_EINVAL (null pointer, W < 1, H < 1), NCC_ERANGE (W >
 * NCC_MAX_WIDTH, or W*H*65025 past int64), NCC_ENOMEM, NCC_EHIP (including
 * an earlier single-pass failure on this stream, see above).
 */
int ncc_sat_build(const uint8_t *img, int W, int H, int64_t *S, int64_t *Q,
                  void *stream);

/* Largest build scratch of ncc_sat_build_noalloc, in bytes (16 MiB): the
 * two-pass build needs about W*H/8 bytes, so images up to about 133 million
 * pixels (a square image up to 11520 x 11520). */
#define NCC_NOALLOC_SCRATCH_BYTES (16u << 20)

/*
 * ncc_sat_build_noalloc -- ncc_sat_build for callers that cannot allocate
 * device memory: code under HIP graph capture, tight serving loops, and
 * harnesses that forbid hipMalloc.  Same arguments, tables and errors as
 * ncc_sat_build (always its two-pass build; NCC_OPT_SAT_BUILD is not read),
 * plus NCC_ERANGE when the image's build scratch exceeds
 * NCC_NOALLOC_SCRATCH_BYTES.  It allocates nothing: the scratch is a fixed
 * device array of that size, which each GPU the library runs on holds until
 * the process ends (its address is looked up once per device, at the first
 * call there).  Every call on a GPU shares that GPU's array, so calls that
 * overlap on one GPU (on different streams, or a graph replayed beside other
 * calls) race: the caller must order them.  Nothing in the array needs to
 * start at zero.
 */
int ncc_sat_build_noalloc(const uint8_t *img, int W, int H, int64_t *S,
                          int64_t *Q, void *stream);

/*
 * ncc_box -- batched four-corner box sums on one table (section 15.8:
 * four-corner equation and satBox listing).
 *
 *   S      [H][W] int64 table from ncc_sat_build (S or Q), device.
 *   rects  [n][4] int32 {x0, y0, x1, y1}, device: the half-open box
 *          [x0,x1) x [y0,y1).
 *   out    [n] int64, device, written: D - B - C + A, with corners outside
 *          the table's leading edges read as zero.  An empty box
 *          (x0 == x1 or y0 == y1) gives 0.  A box outside
 *          0 <= x0 <= x1 <= W, 0 <= y0 <= y1 <= H gives INT64_MIN (the
 *          check runs on the device; there is no error return for it).
 *   n      number of boxes; n == 0 launches nothing and returns NCC_OK.
 *
 * Errors: NCC_EINVAL (null pointer with n > 0, W < 1, H < 1, n < 0),
 * NCC_EHIP.
 */
int ncc_box(const int64_t *S, int W, int H, const int32_t *rects, int64_t n,
            int64_t *out, void *stream);

/*
 * ncc_correlate -- valid-mode normalized cross-correlation of an image with
 * one template or a bank of templates ("Image in shared memory":
 * corrShared_kernel's window sums; section 15.8: window sums from the tables
 * by the four-corner rule, one table serving every window, every template in
 * a bank and every shift of an FFT search).
 *
 *   img       [H][W] uint8, device.
 *   tpl       [nTpl][hT][wT] uint8, device.
 *   sums_out  nullable; [(2+nTpl)][Ho][Wo] int32, device: plane 0 SumI,
 *             plane 1 SumISq, plane 2+t SumIT of template t, with
 *             Wo = W-wT+1, Ho = H-hT+1.  Position (x,y) covers rows
 *             y..y+hT-1 and columns x..x+wT-1.
 *   coef_out  [nTpl][Ho][Wo] float32, device:
 *               num  = K*SumIT - SumI*SumT,   K = wT*hT
 *               varI = K*SumISq - SumI^2,     varT = K*SumTSq - SumT^2
 *               gamma = num / sqrt(varI*varT), and 0 when varI or varT is 0.
 *             num, varI and varT are exact integers; the float evaluation
 *             after them is within 1e-5 of the correctly rounded value.
 *   S, Q      nullable pair (both or neither); [H][W] int64, device: the
 *             summed-area tables of img (as ncc_sat_build writes them), read
 *             only.  NULL: routes that read tables build them in the
 *             workspace.
 *
 * Window sums SumI and SumISq are exact integers by the four-corner rule.
 * The generic and FFT routes read them from the full tables (the caller's S,
 * Q when given).  The specialised kernels form the same integers from the
 * image strip they stage on chip (a table of the strip, or per-window sums)
 * and do not read S, Q: reading four int64 corners of two tables per
 * position would make them HBM-bound well below their compute rate.  A bank
 * (nTpl > 1) of templates with at most 16 rows of at most 16 pixels runs
 * SumIT as an int8 matrix-core contraction; one template of 16 rows and 13
 * to 16 columns runs on the int8 matrix cores as a banded Toeplitz product
 * streamed down image strips; other templates up to 32 x 32, and 16-row
 * ones in small launches (under about 1.5 M positions), run on the int8
 * matrix cores in 16 x 16 output tiles (one banded product per template
 * row), those up to 32 x 64 on the vector units; larger ones run
 * the generic kernel or, where estimated
 * faster (about 48 x 48 and up on a 4096 x 4096 image), a product of 2-D
 * Fourier transforms in double precision rounded to the integer SumIT it
 * equals (the "FFT numerator" section 15.8 names; images whose padded
 * transform exceeds 8192 x 8192 always run the generic kernel).
 * ncc_set_option(NCC_OPT_CORR_ROUTE, ...) forces a route.
 *
 * Errors: NCC_EINVAL (null img/tpl/coef_out, exactly one of S, Q null, W or
 * H < 1, wT or hT < 1, wT > W, hT > H, nTpl < 1), NCC_ERANGE (W >
 * NCC_MAX_WIDTH, wT*hT > NCC_MAX_TEMPLATE_PIXELS, outputs past 2^62 bytes),
 * NCC_EUNSUPPORTED (called during stream capture before the stream's
 * workspace was sized by an uncaptured call), NCC_ENOMEM, NCC_EHIP.
 */
int ncc_correlate(const uint8_t *img, int W, int H, const uint8_t *tpl,
                  int wT, int hT, int nTpl, int32_t *sums_out,
                  float *coef_out, const int64_t *S, const int64_t *Q,
                  void *stream);

/* Largest output row pitch of ncc_correlate_rect, in elements. */
#define NCC_MAX_OUT_PITCH (1 << 24)

/*
 * ncc_correlate_rect -- the same correlation over a rectangle of positions
 * only, read in place from a pitched image, written to pitched output
 * ("Image in shared memory": the sample program's corrShared_kernel computes
 * a w x h rectangle of coefficients whose upper-left position is offset into
 * the image, into rows CorrPitch apart; the two offsets the listing adds to
 * every image coordinate enter here as their sum, x0 and y0).
 *
 *   img        H rows of W uint8 pixels, device; row y starts at
 *              img + y*img_pitch (img_pitch >= W bytes).
 *   tpl        [nTpl][hT][wT] uint8, device.
 *   x0, y0     the first position: its window covers rows y0..y0+hT-1 and
 *              columns x0..x0+wT-1.
 *   w, h       positions x0..x0+w-1 by y0..y0+h-1; every window must lie
 *              inside the image: 0 <= x0, x0+w <= W-wT+1, 0 <= y0,
 *              y0+h <= H-hT+1 (valid mode, as ncc_correlate).  w == 0 or
 *              h == 0 writes nothing and returns NCC_OK.
 *   out_pitch  elements from one output row to the next (>= w); planes are
 *              h*out_pitch elements apart.  Elements between w and
 *              out_pitch of each row are not written.
 *   sums_out   nullable; [(2+nTpl)][h][out_pitch] int32, device, planes as in
 *              ncc_correlate: element [p][v][u] belongs to position
 *              (x0+u, y0+v).
 *   coef_out   [nTpl][h][out_pitch] float32, device, likewise (may be NULL
 *              when w or h is 0).
 *   S, Q       nullable pair; [H][W] int64 summed-area tables of the whole
 *              H x W image (row pitch W elements, as ncc_sat_build writes
 *              them for the dense image), read in place by the routes that
 *              read tables; NULL: those routes build tables of the
 *              rectangle's windows in the workspace.
 *
 * Every value equals ncc_correlate's at the same position, bit for bit for
 * the sums.  Only the image rows and columns that the rectangle's windows
 * cover are read (the streaming kernel may also read up to 15 bytes on each
 * side of them within the same image row).
 *
 * Errors: NCC_EINVAL (null img/tpl, null coef_out with w, h > 0, exactly
 * one of S, Q null, W or H < 1, wT or hT < 1, wT > W, hT > H, nTpl < 1,
 * img_pitch < W, w or h < 0, out_pitch < w),
 * NCC_ERANGE (the rectangle outside the valid positions,
 * wT*hT > NCC_MAX_TEMPLATE_PIXELS, w+wT-1 > NCC_MAX_WIDTH,
 * (w+wT-1)*(h+hT-1) > 2^40, img_pitch*H > 2^48,
 * out_pitch > NCC_MAX_OUT_PITCH, outputs past 2^62 bytes), and the rest as
 * ncc_correlate.
 */
int ncc_correlate_rect(const uint8_t *img, int W, int H, size_t img_pitch,
                       const uint8_t *tpl, int wT, int hT, int nTpl,
                       int x0, int y0, int w, int h, size_t out_pitch,
                       int32_t *sums_out, float *coef_out, const int64_t *S,
                       const int64_t *Q, void *stream);

/*
 * Options: process-wide settings read at every call (no environment
 * variables are read).  ncc_set_option returns NCC_OK, or NCC_EINVAL for an
 * unknown option or value (the setting is then unchanged); ncc_get_option
 * writes the current value.
 *
 *   NCC_OPT_CORR_ROUTE    correlation route: NCC_ROUTE_AUTO (default: the
 *                         choice described at ncc_correlate), or one forced
 *                         route: NCC_ROUTE_GENERIC (tables + generic kernel,
 *                         any shape), NCC_ROUTE_FFT (tables + FFT numerator,
 *                         images up to 8192 x 8192 padded), NCC_ROUTE_SINGLE
 *                         (one template at a time; the matrix-core kernels
 *                         wherever the shape fits), NCC_ROUTE_DOT4 (the
 *                         vector-unit streaming kernel for 16-row templates
 *                         13 to 16 wide), NCC_ROUTE_TILE (the
 *                         vector-unit tile kernel).  A forced route runs
 *                         every template on its own (no bank kernel); where
 *                         its kernel does not take the shape, the generic
 *                         kernel runs (NCC_ROUTE_SINGLE takes the
 *                         matrix-core strip kernel for 16-row templates 13
 *                         to 16 wide at any launch size, else the
 *                         matrix-core tile kernel).
 *   NCC_OPT_SAT_BUILD     NCC_SAT_TWO_PASS (default) or NCC_SAT_SINGLE_PASS.
 *   NCC_OPT_TZ_STRIP      rows per workgroup of the matrix-core single-
 *                         template kernel: 0 (default: chosen per launch),
 *                         16 or 32.
 *   NCC_OPT_STREAM_ROWS   rows per workgroup of the vector-unit streaming
 *                         kernel: 0 (default: chosen per launch), 16, 32, 64.
 *   NCC_OPT_SAT_SPIN      polls of a single-pass look-back wait before it
 *                         gives up: >= 0, default 4194304.
 *   NCC_OPT_SAT_STALE     for tests of the failure report: 1 makes the next
 *                         single-pass build (on any stream) start from a
 *                         state whose tile ticket counter is past the end, as
 *                         a call that never finished would leave it; that
 *                         build resets the option to 0.  Default 0.
 */
#define NCC_OPT_CORR_ROUTE 1
#define NCC_OPT_SAT_BUILD 2
#define NCC_OPT_TZ_STRIP 3
#define NCC_OPT_STREAM_ROWS 4
#define NCC_OPT_SAT_SPIN 5
#define NCC_OPT_SAT_STALE 6

#define NCC_ROUTE_AUTO 0
#define NCC_ROUTE_GENERIC 1
#define NCC_ROUTE_FFT 2
#define NCC_ROUTE_SINGLE 3
#define NCC_ROUTE_DOT4 4
#define NCC_ROUTE_TILE 5

#define NCC_SAT_TWO_PASS 0
#define NCC_SAT_SINGLE_PASS 1

int ncc_set_option(int option, int value);
int ncc_get_option(int option, int *value);

/*
 * ncc_stream_status -- waits for `stream` and reports a failure of a
 * single-pass table build enqueued on it since the last report (a bounded
 * look-back wait that gave up, or a build state left inconsistent): NCC_EHIP
 * then, after resetting the stream's build state, else NCC_OK; also
 * NCC_EHIP if the wait itself fails.  Tables written by a failed build hold
 * INT64_MIN in the tiles concerned (or are not written at all).
 */
int ncc_stream_status(void *stream);

/* Static string naming a status code. */
const char *ncc_strerror(int status);

/* Frees every cached workspace on every device, including blocks retired by
 * growth.  Waits for the devices that used them.  Later calls allocate
 * again; HIP graphs that recorded earlier calls must be captured again. */
void ncc_release(void);

/* ABI version of this header (major*100 + minor): 201. */
int ncc_version(void);

#ifdef __cplusplus
}
#endif

#endif /* NCC_H */
