/* Host check of the division the activation-quantisation kernels use:
 * with y = RN(1/d), q0 = RN(a*y), r = fma(-q0, d, a), q1 = fma(r, y, q0),
 * q1 must equal the IEEE quotient RN(a/d) (Markstein's correction).  Pairs
 * are drawn over the kernels' operating range (d = scale + 1e-5 >= 1e-5,
 * below 2^100; |a/d| <= 127), half of them with a/d next to k + 1/2 where
 * the int8 code could flip.  Also checks the binary64 route of the GEMM
 * epilogue, RN32(RN64(p * RN64(1/127))) == RN32(p / 127), on random binary32
 * p over the whole finite range (subnormals included) and on every mantissa
 * of three binades.  Prints "<pairs> <quotient mismatches>". */
#include <math.h>
#include <stdint.h>
#include <stdio.h>
#include <stdlib.h>
#include <string.h>

static uint64_t st = 0x9E3779B97F4A7C15ull;
static uint64_t next(void) {
    st ^= st << 13;
    st ^= st >> 7;
    st ^= st << 17;
    return st;
}
static float unit(void) { return (float)((next() >> 40) * (1.0 / 16777216.0)); }

int main(int argc, char **argv) {
    long n = argc > 1 ? atol(argv[1]) : 10000000L;
    long bad = 0;
    for (long i = 0; i < n; ++i) {
        float d = ldexpf(1.0f + unit(), (int)(next() % 117) - 17); /* 2^-17 .. 2^100 */
        if (d < 1e-5f) d = 1e-5f;
        float a;
        if (i & 1) {
            float k = (float)((int)(next() % 255) - 127) + 0.5f;
            a = k * d;
            uint32_t u;
            memcpy(&u, &a, 4);
            u += (uint32_t)((int)(next() % 9) - 4);
            memcpy(&a, &u, 4);
        } else {
            a = (unit() * 254.0f - 127.0f) * d;
        }
        float y = 1.0f / d;
        float q0 = a * y;
        float r = fmaf(-q0, d, a);
        float q1 = fmaf(r, y, q0);
        if (q1 != a / d) ++bad;
    }
    /* division by the constant 127 (dequantisation), products over the
     * normal range handled by the fast path (|p| >= 2^-100) */
    const float d127 = 127.0f, y127 = 1.0f / 127.0f;
    for (long i = 0; i < n; ++i) {
        float p = ldexpf(1.0f + unit(), (int)(next() % 227) - 100); /* 2^-100 .. 2^127 */
        if (i & 2) p = -p;
        if (i & 1) { /* near k + 1/2 multiples of 127 ulps: random low bits */
            uint32_t u;
            memcpy(&u, &p, 4);
            u ^= (uint32_t)(next() & 0xff);
            memcpy(&p, &u, 4);
        }
        if (isinf(p)) continue;
        float q0 = p * y127;
        float r = fmaf(-q0, d127, p);
        float q1 = fmaf(r, y127, q0);
        if (q1 != p / d127) ++bad;
    }
    /* binary64 product route for the division by 127 */
    const double r127 = 1.0 / 127.0;
    for (long i = 0; i < n; ++i) {
        uint32_t u = (uint32_t)next();
        float p;
        memcpy(&p, &u, 4);
        if (isnan(p) || isinf(p)) continue;
        if ((float)((double)p * r127) != p / 127.0f) ++bad;
    }
    const int exps[3] = {-140, 0, 100}; /* subnormal quotients, ordinary, large */
    for (int e = 0; e < 3; ++e)
        for (uint32_t m = 0; m < (1u << 23); ++m) {
            float p = ldexpf(1.0f + (float)m / 8388608.0f, exps[e]);
            if ((float)((double)p * r127) != p / 127.0f) ++bad;
        }
    printf("%ld %ld\n", n, bad);
    return 0;
}
