/*
 * Exhaustive check of the reciprocal-and-correction quotient that the int8
 * and int4 block quantizers use in place of a division (CPU; test
 * infrastructure).  The argument is the largest code Q: 127 (int8, the
 * default) or 7 (int4).
 *
 * For every positive finite bf16 absmax with s = RN(absmax / Q) >= 2^-100 and
 * every bf16 x with 0 <= x <= absmax:
 *   r  = RN(1 / s)
 *   q0 = RN(x * r);  rem = RN(x - q0 * s) (fused);  q1 = RN(q0 + rem * r) (fused)
 * and the code clamp(rint(q1), -Q, Q) is compared with the definition
 * clamp(rint(RN(x / s)), -Q, Q).  Negative x need no separate pass: every
 * step is odd in x under round-to-nearest-even, so the code of -x is minus the
 * code of x.
 *
 * Prints: pairs, code mismatches, quotient mismatches with q >= 1/4, and code
 * mismatches of the uncorrected product rint(q0) (which must be non-zero, or
 * the check would not discriminate).
 */
#include <math.h>
#include <stdint.h>
#include <stdio.h>
#include <stdlib.h>
#include <string.h>

static float from_bits(uint32_t u) { float f; memcpy(&f, &u, sizeof f); return f; }
static uint32_t to_bits(float f) { uint32_t u; memcpy(&u, &f, sizeof u); return u; }
static float Q = 127.0f;
static float code(float t) { return fminf(fmaxf(rintf(t), -Q), Q); }

int main(int argc, char **argv)
{
    if (argc > 1)
        Q = (float)atoi(argv[1]);
    long long pairs = 0, bad_code = 0, bad_quot = 0, bad_plain = 0;
#pragma omp parallel for schedule(dynamic, 64) reduction(+ : pairs, bad_code, bad_quot, bad_plain)
    for (int a = 1; a < 0x7f80; ++a) {
        const float amax = from_bits((uint32_t)a << 16);
        const float s = amax / Q;
        if (to_bits(s) < 0x0d800000u)  /* s < 2^-100: the quantizer divides */
            continue;
        const float r = 1.0f / s;
        for (uint32_t xb = 0; xb <= (uint32_t)a; ++xb) {  /* 0 <= x <= amax */
            const float x = from_bits(xb << 16);
            const float q = x / s;
            const float q0 = x * r;
            const float rem = fmaf(-q0, s, x);
            const float q1 = fmaf(rem, r, q0);
            pairs++;
            bad_code += code(q1) != code(q);
            bad_quot += q >= 0.25f && q1 != q;
            bad_plain += code(q0) != code(q);
        }
    }
    printf("%lld %lld %lld %lld\n", pairs, bad_code, bad_quot, bad_plain);
    return 0;
}
