/*
 * Check of the correctly rounded fp32 square root the GPU kernels use
 * (CPU; test infrastructure).  The hardware square root is only known to be
 * within 1 ulp, so the check starts from each of the three values within 1 ulp
 * of the true root -- RN(sqrt x) and its two neighbours -- and applies the
 * kernels' refinement:
 *   xs = x < 2^-96 ? x * 2^32 : x          (exact scaling of small inputs)
 *   s  = start value for sqrt(xs)
 *   s- = s with its bit pattern minus 1, s+ = plus 1
 *   if fma(-s-, s, xs) <= 0: s = s-      (root below the lower midpoint)
 *   else if fma(-s+, s, xs) > 0: s = s+  (root above the upper midpoint)
 *   result = x < 2^-96 ? s * 2^-16 : s
 * and compares the result with the C library's correctly rounded sqrtf.  (The
 * 1-ulp bound covers finite inputs; the root of +inf is +inf exactly.)
 *
 * Argument "all": every finite x >= 0 (2^31 - 2^23 values); otherwise the
 * exponents that exercise every distinct path: all denormals, the scaled
 * range around 2^-96, two whole binades of each exponent parity ([1, 4)), and
 * the largest binades.  Prints: inputs checked, mismatches.
 */
#include <math.h>
#include <stdint.h>
#include <stdio.h>
#include <string.h>

static float from_bits(uint32_t u) { float f; memcpy(&f, &u, sizeof f); return f; }
static uint32_t to_bits(float f) { uint32_t u; memcpy(&u, &f, sizeof u); return u; }

static float refine(float x, float s)
{
    const int tiny = x < 0x1p-96f;
    const float xs = tiny ? x * 0x1p+32f : x;
    const float sp = from_bits(to_bits(s) - 1), sn = from_bits(to_bits(s) + 1);
    if (fmaf(-sp, s, xs) <= 0.0f)
        s = sp;
    else if (fmaf(-sn, s, xs) > 0.0f)
        s = sn;
    return tiny ? s * 0x1p-16f : s;
}

static long long check_range(uint32_t lo, uint32_t hi, long long *bad)
{
    long long n = 0, b = 0;
#pragma omp parallel for schedule(dynamic, 65536) reduction(+ : n, b)
    for (long long u = lo; u < (long long)hi; ++u) {
        const float x = from_bits((uint32_t)u);
        const float y = sqrtf(x);
        const float xs = x < 0x1p-96f ? x * 0x1p+32f : x;
        const float ys = sqrtf(xs);
        for (int d = -1; d <= 1; ++d) {
            if ((ys == 0.0f && d < 0) || (isinf(x) && d != 0))
                continue;   /* nothing below +0; the hardware root of +inf is +inf exactly */
            const float s0 = from_bits(to_bits(ys) + d);
            const float r = refine(x, s0);
            n++;
            b += to_bits(r) != to_bits(y);
        }
    }
    *bad += b;
    return n;
}

int main(int argc, char **argv)
{
    long long n = 0, bad = 0;
    if (argc > 1 && !strcmp(argv[1], "all")) {
        n += check_range(0, 0x7f800001u, &bad);   /* every finite x >= 0, and +inf */
    } else {
        n += check_range(0, 0x00800000u, &bad);             /* zero and all denormals */
        n += check_range(0x0f000000u, 0x10800000u, &bad);   /* around the 2^-96 scaling edge */
        n += check_range(0x3f800000u, 0x40800000u, &bad);   /* [1, 4): both exponent parities */
        n += check_range(0x7e800000u, 0x7f800001u, &bad);   /* the two largest binades, +inf */
    }
    printf("%lld %lld\n", n, bad);
    return 0;
}
