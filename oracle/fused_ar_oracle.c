/*
 * Oracle for the fused all-reduce + residual-add + RMSNorm epilogue (one GPU's share).
 *
 * TEST INFRASTRUCTURE, NOT PART OF THE PRODUCT. Only the test suite, the package smoke check and
 * the benchmark's CPU-baseline leg may load this library. The HIP path never calls it, and the two
 * share no code: no header, helper, table or constant.
 *
 * It is plain, single-threaded C, written to be checked by eye against the pages it follows.
 * Build it with -ffp-contract=off and without fast-math, so that every float operation below is
 * one IEEE binary32 (or binary64) operation with round-to-nearest-even.
 *
 * What it computes, for an [m, hidden] problem with n partial-sum buffers in[0..n-1] (bf16),
 * a residual [m, hidden] (bf16) and a weight [hidden] (bf16):
 *
 *   1. Reduce. "perf: optimize fused AllReduce + RMSNorm (custom_all_reduce)" (ROCm/aiter PR #3817),
 *      Technical Details > 2stage > reduce-scatter: each element is summed over the n buffers in
 *      fp32, in the buffer order ptrs[0..ngpus-1], and the fp32 sum is rounded to bf16.
 *      The accumulator starts from the first rank's value and each further rank is added with
 *      one fp32 addition.
 *   2. Residual. "perf(comm): add opt-in Triton AR+RMSNorm backend" (lightseekorg/tokenspeed PR #968),
 *      Summary (AI) and the fused operator it adds (all-reduce + residual + RMSNorm, bf16 tensors of
 *      shape (tokens, hidden), bf16 weight): the reduced bf16 value plus the bf16 residual, rounded
 *      once to bf16, is the residual output.
 *   3. RMSNorm of each row of that residual output, the normalisation that both pages fuse after the
 *      all-reduce (aiter PR #3817, Motivation and Technical Details > 2stage > stage-2 RMSNorm reduce,
 *      where it is a per-row square-sum reduction). The pages name RMSNorm without printing its
 *      formula; this is its usual definition, with eps added to the mean of squares inside the root
 *      and the weight applied as a plain factor:
 *      out[j] = bf16( x[j] / sqrt(mean_j(x[j]^2) + eps) * w[j] ).
 *
 * Precision. The pages fix fp32 for the reduce (step 1), so it runs in binary32 here. They fix
 * nothing for steps 2 and 3, so those run in binary64 and are rounded once to bf16; this is the
 * exact result to within binary64 rounding (see the comments at each step).
 *
 * Rounding to bf16 is round-to-nearest, ties to even, with overflow to infinity, subnormals kept
 * and NaN returned as a quiet NaN with the operand's sign. The pages name no rounding mode for the
 * conversion; this is the IEEE default.
 *
 * Layout: every [m, hidden] array is row-major and contiguous; bf16 values travel as their raw
 * 16-bit patterns (uint16_t).
 */
#include <math.h>
#include <stdint.h>
#include <string.h>

/* The binary32 value of a bf16 bit pattern: bf16 is the upper half of a binary32. */
static float bf16_to_float(uint16_t b)
{
    uint32_t bits = (uint32_t)b << 16;
    float f;
    memcpy(&f, &bits, sizeof f);
    return f;
}

/*
 * Round a real number (given as a binary64) to the nearest bf16, ties to even.
 * bf16 has 8 significant bits and the exponent range of binary32: normal values from 2^-126,
 * subnormal values spaced 2^-133, largest finite value (2 - 2^-7) * 2^127.
 */
uint16_t oracle_bf16_round(double x)
{
    uint16_t sign = signbit(x) ? 0x8000u : 0u;
    if (isnan(x))
        return (uint16_t)(sign | 0x7FC0u);
    double a = fabs(x);
    if (isinf(a))
        return (uint16_t)(sign | 0x7F80u);
    if (a == 0.0)
        return sign;

    int e;
    frexp(a, &e);            /* a = f * 2^e with 0.5 <= f < 1, so 2^(e-1) <= a < 2^e       */
    int q = e - 8;           /* bf16 values in [2^(e-1), 2^e) are spaced 2^q apart          */
    if (q < -133)
        q = -133;            /* below 2^-126 the spacing stays at the subnormal step 2^-133 */

    double units = ldexp(a, -q);       /* a in steps of 2^q; a power-of-two scaling, exact  */
    double lower = floor(units);
    double frac = units - lower;       /* exact                                             */
    double k = lower;
    if (frac > 0.5 || (frac == 0.5 && fmod(lower, 2.0) == 1.0))
        k = lower + 1.0;               /* nearest; on a tie the even neighbour              */

    double r = ldexp(k, q);            /* the rounded magnitude                             */
    if (r >= 0x1p128)
        return (uint16_t)(sign | 0x7F80u);   /* beyond the largest finite bf16: infinity   */
    float rf = (float)r;               /* exact: at most 8 significant bits, in range       */
    uint32_t bits;
    memcpy(&bits, &rf, sizeof bits);
    return (uint16_t)(sign | (bits >> 16));
}

/* Step 1 for one element: fp32 sum over the ranks in order 0..n-1, then one rounding to bf16. */
static uint16_t reduce_element(const uint16_t *const *inputs, int n, size_t i)
{
    float acc = bf16_to_float(inputs[0][i]);
    for (int k = 1; k < n; ++k)
        acc = acc + bf16_to_float(inputs[k][i]);
    return oracle_bf16_round((double)acc);
}

/*
 * Step 1 alone over `count` elements: reduced[i] = bf16(fp32 sum of inputs[0..n-1][i]).
 * Returns 0, or -1 on a bad argument.
 */
int oracle_reduce(const uint16_t *const *inputs, int n, long long count, uint16_t *reduced)
{
    if (inputs == NULL || n < 1 || count < 0 || reduced == NULL)
        return -1;
    for (long long i = 0; i < count; ++i)
        reduced[i] = reduce_element(inputs, n, (size_t)i);
    return 0;
}

/*
 * Steps 1-3 over an [m, hidden] problem. Writes residual_out and out, both [m, hidden].
 * Returns 0, or -1 on a bad argument.
 */
int oracle_fused_ar_rmsnorm(const uint16_t *const *inputs, int n, const uint16_t *residual,
                            const uint16_t *weight, float eps, int m, int hidden,
                            uint16_t *residual_out, uint16_t *out)
{
    if (inputs == NULL || n < 1 || residual == NULL || weight == NULL || m < 0 || hidden < 1 ||
        residual_out == NULL || out == NULL)
        return -1;

    for (int r = 0; r < m; ++r) {
        size_t row = (size_t)r * (size_t)hidden;

        /* Steps 1 and 2. Both addends of the residual add are bf16 values; their binary64 sum
         * differs from the exact sum only when their exponents differ by more than 45, and then
         * the exact sum lies within 2^-45 (relative) of the larger addend, far from any bf16
         * rounding tie, so rounding the binary64 sum gives the correctly rounded exact sum. */
        for (int j = 0; j < hidden; ++j) {
            size_t i = row + (size_t)j;
            uint16_t red = reduce_element(inputs, n, i);
            double sum = (double)bf16_to_float(red) + (double)bf16_to_float(residual[i]);
            residual_out[i] = oracle_bf16_round(sum);
        }

        /* Step 3: mean of squares of the bf16 residual output. Each square of a bf16 value is
         * exact in binary64 (16 significant bits), and a row sum of them needs at most
         * 16 + log2(hidden) + (exponent spread) bits, so this is the exact sum except for rows
         * whose values span a very wide exponent range. */
        double sumsq = 0.0;
        for (int j = 0; j < hidden; ++j) {
            double x = (double)bf16_to_float(residual_out[row + (size_t)j]);
            sumsq = sumsq + x * x;
        }
        double mean = sumsq / (double)hidden;
        double rstd = 1.0 / sqrt(mean + (double)eps);

        for (int j = 0; j < hidden; ++j) {
            double x = (double)bf16_to_float(residual_out[row + (size_t)j]);
            double w = (double)bf16_to_float(weight[j]);
            out[row + (size_t)j] = oracle_bf16_round(x * rstd * w);
        }
    }
    return 0;
}
