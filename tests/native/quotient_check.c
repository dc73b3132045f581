/*
 * Exhaustive check of the quotient used by the HIP quantization kernels.
 *
 * A quantization code is q = rne(fl32(x / s)) with s = fl32(a / 127), where
 * a is the absmax (an fp16 magnitude) of the vector x belongs to, so
 * |x| <= a.  The kernels replace the per-element IEEE division by
 *     r  = fl32(1 / s)                 (once per vector, IEEE division)
 *     q0 = fl32(x * r)                 (on the GPU fma(x, r, +0): the same
 *                                       value for every x != 0, and x = 0
 *                                       gives code 0 either way)
 *     e  = fma(-q0, s, x)              (exact residual)
 *     q1 = fma(e, r, q0)
 * This program checks q1 == fl32(x / s) bit for bit for every positive
 * finite fp16 a and every fp16 x with 0 < x <= a (the formula is odd in x,
 * and x = 0 gives 0 on both sides), and reports the number of mismatches.
 * It also checks the two facts the kernels use to turn q1 into a code:
 * rounding by adding 1.5 * 2^23 leaves rne(q1) in the low mantissa bits
 * (the sum's low byte is the two's complement code byte, for q1 and -q1),
 * and |rne(q1)| <= 127, so no clamp is needed.
 *
 * Build: gcc -O2 -fopenmp -ffp-contract=off quotient_check.c -lm
 */
#include <math.h>
#include <stdint.h>
#include <stdio.h>
#include <string.h>

static float half_value(uint16_t h)
{
    int e = (h >> 10) & 31, m = h & 1023;
    if (e == 0)
        return ldexpf((float)m, -24);
    return ldexpf((float)(m | 1024), e - 25);
}

int main(void)
{
    static float vals[0x7c00];
    for (int i = 0; i < 0x7c00; i++)
        vals[i] = half_value((uint16_t)i);
    long long bad = 0, checked = 0;
#pragma omp parallel for schedule(dynamic, 64) reduction(+ : bad, checked)
    for (int ia = 1; ia < 0x7c00; ia++) {
        volatile float a = vals[ia];
        float s = a / 127.0f;
        float r = 1.0f / s;
        for (int ix = 1; ix <= ia; ix++) {
            float x = vals[ix];
            float ref = x / s;
            float q0 = x * r;
            float e = fmaf(-q0, s, x);
            float q1 = fmaf(e, r, q0);
            uint32_t b1, b2;
            memcpy(&b1, &ref, 4);
            memcpy(&b2, &q1, 4);
            bad += (b1 != b2);
            /* rounding through the magic constant, and the code range */
            float rq = rintf(q1);
            float m1 = q1 + 12582912.0f, m2 = -q1 + 12582912.0f;
            uint32_t u1, u2;
            memcpy(&u1, &m1, 4);
            memcpy(&u2, &m2, 4);
            bad += (rq > 127.0f);
            bad += ((int8_t)(u1 & 0xffu) != (int8_t)rq);
            bad += ((int8_t)(u2 & 0xffu) != (int8_t)(-rq));
            checked++;
        }
    }
    printf("checked %lld pairs, mismatches %lld\n", checked, bad);
    return bad != 0;
}
