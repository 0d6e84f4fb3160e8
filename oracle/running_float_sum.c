/*
 * TEST INFRASTRUCTURE ONLY.  The plain CPU oracle of the running float sum;
 * only the tests, the smoke check and the bench's cpu_baseline leg may load
 * it, and it shares no source with the library under exact_reductions_amd/.
 *
 * What it computes: the value one binary32 accumulator holds after a buffer
 * of float terms has been added into it one by one, in buffer order,
 * starting from zero.
 *
 * Source (web page, cited by title and section):
 *   [HVS] "ADR-1397: GPU psnr_hvs twins reproduce the CPU's running float
 *         sum bit for bit" -- Context: calc_psnrhvs() accumulates all of a
 *         plane's masked coefficient errors (an 8x8 block gives 64) in a
 *         single float, so the rounding of each add depends on the value
 *         accumulated before it; Decision: the terms are laid out row-major
 *         inside a block with the blocks in raster order, the host folds
 *         them into one float in that order, and the reference code is
 *         compiled without contraction.
 *
 * Build: gcc -O2 -ffp-contract=off -fno-fast-math.  On x86-64 a float add is
 * one SSE binary32 addition, rounded to nearest, ties to even; nothing here
 * lets the compiler reorder the adds.
 */

#include <stddef.h>

/* The running sum of n terms. */
float oracle_running_float_sum(const float *terms, long long n)
{
    float s = 0.0f;
    for (long long i = 0; i < n; ++i)
        s += terms[i];
    return s;
}

/*
 * nsums buffers of n terms each, stored one after another; sum k goes to
 * out[k].  Returns 0, or -1 on a bad argument (then out is untouched).
 */
int oracle_running_float_sums(const float *terms, long long n, int nsums, float *out)
{
    if (!terms || !out || n < 0 || nsums < 1)
        return -1;
    for (int k = 0; k < nsums; ++k)
        out[k] = oracle_running_float_sum(terms + (size_t)k * (size_t)n, n);
    return 0;
}
