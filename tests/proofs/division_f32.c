/* Two-correction FMA division in binary32, against IEEE a / b.
 *
 *   y  = RN(1/b)                       (the kernels' reciprocal equals it:
 *                                       tests/proofs/rcp_probe.hip)
 *   q0 = RN(a*y)
 *   q1 = RN(q0 - RN(q0*b - a)*y)        (the remainder by one FMA: exact)
 *   q2 = RN(q1 - RN(q1*b - a)*y)
 *
 * This is the quotient the quantize kernels form for binary32 dividends
 * (an f32 input element, or the asymmetric range mx - mn) inside their fast
 * range 2^-40 <= |b| <= 2^40, 2^-78 <= |a| <= 2^86.  q1 is faithful and
 * Markstein's theorem (y within half an ulp of 1/b, q within one ulp of a/b
 * => RN(q + r*y) = RN(a/b)) makes q2 correctly rounded while the
 * intermediates stay normal.  Checked here on random operands spread over
 * the whole guarded range and on the hardest ones: quotients within about
 * 15 * 2^-48 (relative) of a midpoint between two binary32 numbers, where
 * a faithful but wrong quotient shows.  The program also counts the pairs
 * where the first correction alone is wrong: none were found (q0 = RN(a*y)
 * is itself faithful, so the theorem already applies after one step); the
 * kernels keep the second step for binary32 dividends as the margin this
 * check covers.
 *
 * usage: division_f32 <n>   (n random pairs and n near-midpoint pairs)
 */
#include <math.h>
#include <stdint.h>
#include <stdio.h>
#include <stdlib.h>
#include <string.h>

static uint64_t sm_next(uint64_t* s)
{
    uint64_t z = (*s += 0x9e3779b97f4a7c15ull);
    z = (z ^ (z >> 30)) * 0xbf58476d1ce4e5b9ull;
    z = (z ^ (z >> 27)) * 0x94d049bb133111ebull;
    return z ^ (z >> 31);
}

static float from_sig(uint32_t sig24, int e)   /* sig24 in [2^23, 2^24): value sig24 * 2^(e - 23) */
{
    return ldexpf((float)sig24, e - 23);
}

/* returns 1 when q2 differs from IEEE a / b; *wrong1 = q1 differs */
static int check(float a, float b, int* wrong1)
{
    volatile float one = 1.0f;
    const float y = one / b;
    const float q0 = a * y;
    const float q1 = fmaf(-fmaf(q0, b, -a), y, q0);
    const float q2 = fmaf(-fmaf(q1, b, -a), y, q1);
    volatile float va = a, vb = b;
    const float ref = va / vb;
    *wrong1 = memcmp(&q1, &ref, 4) != 0;
    if (memcmp(&q2, &ref, 4) != 0) {
        printf("mismatch a=%a b=%a q2=%a ref=%a\n", a, b, q2, ref);
        return 1;
    }
    return 0;
}

int main(int argc, char** argv)
{
    const long long n = argc > 1 ? atoll(argv[1]) : 1000000;
    const uint32_t top = 1u << 23, mask = top - 1;
    long long bad2 = 0, bad1 = 0, hard = 0, bad1_hard = 0;
    uint64_t st = 20240611;
    for (long long i = 0; i < n; ++i) {
        const uint64_t r = sm_next(&st);
        /* divisor exponent in [-40, 39], dividend exponent in [-78, 85] */
        const int eb = (int)(r % 80) - 40;
        const int ea = (int)((r >> 8) % 164) - 78;
        float a = from_sig(top | ((uint32_t)sm_next(&st) & mask), ea);
        float b = from_sig(top | ((uint32_t)sm_next(&st) & mask), eb);
        if (r & (1ull << 20)) a = -a;
        if (r & (1ull << 21)) b = -b;
        int w1;
        bad2 += check(a, b, &w1);
        bad1 += w1;
        /* quotients of a group: a scale b and elements |a| <= 255 * |b| */
        const float a2 = b * ldexpf((float)((r >> 32) & 0xffff) / 65536.0f, (int)((r >> 48) % 8));
        bad2 += check(a2, b, &w1);
        bad1 += w1;
        if (bad2 > 10) break;
    }
    for (long long i = 0; i < n && bad2 <= 10; ++i) {
        /* a/b within |d| * 2^-48 of the midpoint m / 2^24 (m odd, 25 bits):
         * A * 2^24 = B * m + d with B odd, d small and odd, so
         * m = -d * B^-1 mod 2^24 (+ 2^24) and A = (B * m + d) / 2^24. */
        const uint64_t B = top | ((uint32_t)sm_next(&st) & mask) | 1u;
        uint64_t inv = B;                                   /* B^-1 mod 2^64 by Newton */
        for (int k = 0; k < 6; ++k) inv *= 2 - B * inv;
        const int64_t d = (int64_t)(sm_next(&st) % 16) * 2 - 15;   /* odd, -15..15 */
        const uint64_t m = (((uint64_t)(-d) * inv) & ((1ull << 24) - 1)) | (1ull << 24);
        const int64_t num = (int64_t)(B * m) + d;
        if (num & ((1ll << 24) - 1)) return 2;              /* construction broken */
        const int64_t A = num >> 24;
        if (A < (int64_t)top || A >= (int64_t)(1u << 24)) continue;
        const uint64_t r = sm_next(&st);
        const int eb = (int)(r % 80) - 40;                  /* |b| in [2^-40, 2^40) */
        const int ea = eb + (int)((r >> 8) % 41) - 20;      /* |a| within 2^+-20 of |b| */
        int w1;
        bad2 += check(from_sig((uint32_t)A, ea), from_sig((uint32_t)B, eb), &w1);
        bad1_hard += w1;
        bad2 += check(-from_sig((uint32_t)A, ea), from_sig((uint32_t)B, eb), &w1);
        bad1_hard += w1;
        hard += 2;
    }
    printf("%lld random pairs; first correction alone: %lld wrong\n", 2 * n, bad1);
    printf("%lld near-midpoint pairs; first correction alone: %lld wrong\n", hard, bad1_hard);
    printf("two corrections: %lld mismatches\n", bad2);
    return bad2 != 0;
}
