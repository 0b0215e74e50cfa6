/*
 * Exhaustive checks of two division shortcuts in the GPU kernels (test
 * infrastructure).  Prints one line per check: "<name> checked N bad B".
 *
 * 1. Division by the constants 6 and 448 (group and row scales): for every
 *    finite non-negative bf16 x (subnormals included) the kernels compute
 *        y0 = RN(x * rc),  y = RN(fma(RN(fma(-y0, d, x)), rc, y0)),  rc = RN(1/d)
 *    and rely on y == RN(x / d).  The constant rc is given here as the hex
 *    literal the kernels use, and checked to be RN(1/d).
 * 2. Reciprocal of an e4m3fn scale: for every positive finite e4m3fn value s
 *    and every starting r0 within 2 ulp of RN(1/s), one Newton step
 *        r = RN(fma(r0, RN(fma(-s, r0, 1)), r0))
 *    gives RN(1/s).  (The hardware reciprocal the kernels start from is
 *    within 1 ulp.)
 * RN(a / b) is computed independently from a float64 candidate corrected by
 * exact midpoint tests.
 */
#include <math.h>
#include <stdint.h>
#include <stdio.h>
#include <string.h>

static float u2f(uint32_t u) { float f; memcpy(&f, &u, 4); return f; }
static uint32_t f2u(float f) { uint32_t u; memcpy(&u, &f, 4); return u; }

/* RN(a / b) for finite a >= 0 and b > 0: a float64 candidate, moved to the
 * neighbouring float while the exact quotient lies beyond a midpoint.  A
 * midpoint of two floats has at most 25 significant bits, so midpoint * b is
 * exact in float64 and each comparison is exact (subnormal floats included);
 * at an exact tie the candidate, rounded from the exact float64 quotient, is
 * already the even neighbour. */
static float div_rn(float a, float b) {
    float c = (float)((double)a / (double)b);
    for (int it = 0; it < 3; ++it) {
        const uint32_t u = f2u(c);
        const double hi = 0.5 * ((double)c + (double)u2f(u + 1));
        const double lo = u ? 0.5 * ((double)c + (double)u2f(u - 1)) : 0.0;
        if ((double)a > hi * (double)b) c = u2f(u + 1);
        else if (u && (double)a < lo * (double)b) c = u2f(u - 1);
    }
    return c;
}

static void check_const(const char* name, float d, uint32_t rc_bits) {
    const float rc = u2f(rc_bits);
    long n = 0, bad = 0;
    if (f2u(div_rn(1.0f, d)) != rc_bits) bad++;
    for (uint32_t b = 0; b < 0x7F80u; ++b) {  /* every non-negative finite bf16 */
        const float x = u2f(b << 16);
        const float y0 = x * rc;
        const float y = fmaf(fmaf(-y0, d, x), rc, y0);
        ++n;
        if (f2u(y) != f2u(div_rn(x, d))) bad++;
    }
    printf("%s checked %ld bad %ld\n", name, n, bad);
}

static void check_e4m3_reciprocal(void) {
    long n = 0, bad = 0;
    for (int c = 1; c < 0x7F; ++c) {          /* every positive finite e4m3fn code */
        const int E = (c >> 3) & 15, m = c & 7;
        const float s = E == 0 ? (float)m * 0x1p-9f : ldexpf((float)(8 + m), E - 10);
        const float exact = div_rn(1.0f, s);
        for (int k = -2; k <= 2; ++k) {
            const float r0 = u2f(f2u(exact) + k);
            const float r = fmaf(r0, fmaf(-s, r0, 1.0f), r0);
            ++n;
            if (f2u(r) != f2u(exact)) bad++;
        }
    }
    printf("e4m3_reciprocal checked %ld bad %ld\n", n, bad);
}

int main(void) {
    check_const("div6", 6.0f, 0x3E2AAAABu);     /* 0x1.555556p-3f */
    check_const("div448", 448.0f, 0x3B124925u); /* 0x1.24924ap-9f */
    check_e4m3_reciprocal();
    return 0;
}
