/*
 * TEST INFRASTRUCTURE ONLY.  This is the slow, plain CPU oracle that the HIP
 * library is checked against.  Only the tests, the smoke check and the
 * bench's cpu_baseline leg may load it; no product code path calls it.  It
 * shares no source, header or table with the library under
 * exact_reductions_amd/.
 *
 * What it computes: for one luma frame pair, the five double accumulators of
 * the CPU feature extractors float_psnr and float_moment, in the CPU's own
 * arithmetic, sample by sample, rows top to bottom and columns left to right.
 *
 * Sources (web pages; cited by title and section):
 *   [PSNR]   "ADR-1440: float_psnr_hip adds its squared differences as
 *            integers and returns the CPU's score bit for bit" -- Context.
 *            The CPU turns both planes into float samples divided by
 *            scaler = 2^(bpc-8), forms the float square of every sample
 *            difference and accumulates those squares in one double,
 *            visiting the rows from the top.
 *   [MOMENT] "ADR-1447: float_moment_hip adds the float squares the CPU
 *            adds, and is bit-identical while the CPU's own sum is exact" --
 *            Context.  One double per output collects the (scaled) samples
 *            or their float squares; the mean is that double over the pixel
 *            count.
 *   [HVS]    "ADR-1397: GPU psnr_hvs twins reproduce the CPU's running
 *            float sum bit for bit" -- Decision.  The CPU reference is
 *            built with contraction off, so no product is fused with an add.
 *
 * Build: gcc -O2 -ffp-contract=off -fno-fast-math -shared -fPIC.  On x86-64
 * a float expression is evaluated in binary32 (SSE), so `a * b` on two
 * floats is one IEEE product rounded to nearest, ties to even.
 *
 * Readings where the pages are silent:
 *   - "row by row" is one running double per output, visited in raster
 *     order (not per-row partials).
 *   - The difference is taken between the two scaled float samples, as the
 *     CPU does; it is exact because both are multiples of 1/scaler below 2^8.
 *   - A uint16 sample above 2^bpc - 1 is not an error: it is converted and
 *     squared like any other value.
 */

#include <stddef.h>
#include <stdint.h>

/* Sample i of a plane as the CPU's float: the stored integer converted to
 * float, then divided by the scaler [PSNR, Context; MOMENT, Context]. */
static float scaled_sample(const void *plane, size_t i, int bpc, float scaler)
{
    float v;
    if (bpc == 8)
        v = (float)((const uint8_t *)plane)[i];
    else
        v = (float)((const uint16_t *)plane)[i];
    return v / scaler;
}

/*
 * One frame.  out[0] = noise (sum of squared differences), out[1] = sum of
 * ref samples, out[2] = sum of dist samples, out[3] = sum of squared ref
 * samples, out[4] = sum of squared dist samples; all on the 8-bit scale
 * (samples divided by the scaler), exactly as the CPU's accumulators hold
 * them before the final division by w*h.
 *
 * Returns 0, or -1 on a bad argument (then out is untouched).
 */
int oracle_frame_sums(const void *ref, const void *dist, int w, int h, int bpc, double *out)
{
    if (!ref || !dist || !out || w < 1 || h < 1 || bpc < 8 || bpc > 16)
        return -1;

    const float scaler = (float)(1 << (bpc - 8));
    double noise = 0.0;     /* float_psnr: one double [PSNR, Context] */
    double ref_sum = 0.0;   /* float_moment: one double per output [MOMENT, Context] */
    double dist_sum = 0.0;
    double ref_sq_sum = 0.0;
    double dist_sq_sum = 0.0;

    for (int y = 0; y < h; ++y) {
        for (int x = 0; x < w; ++x) {
            const size_t i = (size_t)y * (size_t)w + (size_t)x;
            const float r = scaled_sample(ref, i, bpc, scaler);
            const float d = scaled_sample(dist, i, bpc, scaler);

            const float diff = r - d;
            const float diff_sq = diff * diff;   /* float square of the difference */
            noise += (double)diff_sq;

            ref_sum += (double)r;
            dist_sum += (double)d;

            const float r_sq = r * r;            /* the moment's float square */
            const float d_sq = d * d;
            ref_sq_sum += (double)r_sq;
            dist_sq_sum += (double)d_sq;
        }
    }

    out[0] = noise;
    out[1] = ref_sum;
    out[2] = dist_sum;
    out[3] = ref_sq_sum;
    out[4] = dist_sq_sum;
    return 0;
}

/*
 * nframes frames stored back to back, [nframes][h][w]; frame f's five sums go
 * to out[5*f .. 5*f+4].  Each frame starts its accumulators from zero.
 */
int oracle_batch_sums(const void *ref, const void *dist, int w, int h, int bpc, int nframes,
                      double *out)
{
    if (!ref || !dist || !out || w < 1 || h < 1 || bpc < 8 || bpc > 16 || nframes < 1)
        return -1;
    const size_t bytes = (size_t)w * (size_t)h * (bpc == 8 ? 1u : 2u);
    for (int f = 0; f < nframes; ++f) {
        const char *r = (const char *)ref + (size_t)f * bytes;
        const char *d = (const char *)dist + (size_t)f * bytes;
        int rc = oracle_frame_sums(r, d, w, h, bpc, out + 5 * (size_t)f);
        if (rc != 0)
            return rc;
    }
    return 0;
}
