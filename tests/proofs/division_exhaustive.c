/* Exhaustive check of the one-correction FMA division the quantize kernels
 * use for bf16 / f16 inputs: for every binary32 divisor significand s in
 * [1, 2) and every dividend significand x in [1, 2) with FBITS fraction bits
 * (7: bf16, 10: f16),
 *     y = RN(1/s); q0 = RN(x*y); r = RN(q0*s - x); q = RN(q0 - r*y)
 * (the last two as fused multiply-adds) equals the IEEE quotient RN(x/s).
 * Rounding is scale-invariant while every intermediate stays normal, so the
 * significand pairs cover every exponent inside that range.
 * Prints the number of mismatches; exit status 0 iff there are none. */
#include <math.h>
#include <stdint.h>
#include <stdio.h>
#include <stdlib.h>
#include <string.h>

static float from_bits(uint32_t b) { float f; memcpy(&f, &b, 4); return f; }
static uint32_t to_bits(float f) { uint32_t b; memcpy(&b, &f, 4); return b; }

int main(int argc, char** argv)
{
    const int fbits = argc > 1 ? atoi(argv[1]) : 7;
    long bad = 0;
#pragma omp parallel for reduction(+ : bad) schedule(static, 4096)
    for (long ms = 0; ms < (1L << 23); ++ms) {
        const float s = from_bits(0x3f800000u | (uint32_t)ms);
        const float y = 1.0f / s;
        for (uint32_t mx = 0; mx < (1u << fbits); ++mx) {
            const float x = from_bits(0x3f800000u | (mx << (23 - fbits)));
            const float q0 = x * y;
            const float r = fmaf(q0, s, -x);
            const float q = fmaf(-r, y, q0);
            if (to_bits(q) != to_bits(x / s)) ++bad;
        }
    }
    printf("fraction bits %d: %ld mismatches\n", fbits, bad);
    return bad != 0;
}
