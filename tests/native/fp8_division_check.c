/*
 * Exhaustive check of the FP8 fp32-scale quotient used by the GPU kernels
 * (test infrastructure).  For x a bf16 value and s a positive normal fp32,
 * the kernels compute
 *     r = RN(1/s),  y0 = RN(x * r),  y = RN(fma(RN(fma(-y0, s, x)), r, y0))
 * and rely on y == RN(x / s).  Both sides scale with the exponents of x and
 * s (away from underflow and overflow), so it suffices to run every bf16
 * significand (1.m, 7 bits) against every fp32 significand in [1, 2).
 * RN(x / s) is computed independently: a float64 candidate corrected by exact
 * midpoint tests (products of a 24-bit and a 25-bit significand are exact in
 * float64; an exact tie is impossible for these operands).
 * Usage: fp8_division_check MANT_BEGIN MANT_END  -> prints "checked N bad B".
 */
#include <math.h>
#include <stdint.h>
#include <stdio.h>
#include <stdlib.h>
#include <string.h>

static float u2f(uint32_t u) { float f; memcpy(&f, &u, 4); return f; }
static uint32_t f2u(float f) { uint32_t u; memcpy(&u, &f, 4); return u; }

static float div_rn(float x, float s) {
    float c = (float)((double)x / (double)s);
    for (int it = 0; it < 3; ++it) {
        uint32_t b = f2u(c);
        double hi = 0.5 * ((double)c + (double)u2f(b + 1));
        double lo = 0.5 * ((double)c + (double)u2f(b - 1));
        if ((double)x > hi * (double)s) c = u2f(b + 1);
        else if ((double)x < lo * (double)s) c = u2f(b - 1);
        else break;
    }
    return c;
}

int main(int argc, char** argv) {
    if (argc != 3) return 2;
    uint32_t m0 = (uint32_t)strtoul(argv[1], 0, 10), m1 = (uint32_t)strtoul(argv[2], 0, 10);
    long n = 0, bad = 0;
    for (uint32_t sm = m0; sm < m1; ++sm) {
        const float s = u2f((127u << 23) | sm);
        const float r = div_rn(1.0f, s);
        for (uint32_t xm = 0; xm < 128; ++xm) {
            const float x = u2f((127u << 23) | (xm << 16));
            const float y0 = x * r;
            const float e = fmaf(-y0, s, x);
            const float y = fmaf(e, r, y0);
            ++n;
            if (f2u(y) != f2u(div_rn(x, s))) ++bad;
        }
    }
    printf("checked %ld bad %ld\n", n, bad);
    return bad != 0;
}
