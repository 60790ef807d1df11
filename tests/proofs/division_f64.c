/* Two-correction FMA division in binary64, against IEEE a / b.
 *
 *   y  = RN(1/b)
 *   q0 = RN(a*y)
 *   q1 = RN(q0 - RN(a - b*q0)*y)      (the remainder by one FMA: exact)
 *   q2 = RN(q1 - RN(a - b*q1)*y)
 *
 * q1 is faithful (within one ulp of a/b), and then Markstein's theorem
 * (y within half an ulp of 1/b, q within one ulp of a/b => RN(q + r*y) is
 * RN(a/b)) makes q2 the correctly rounded quotient, for operands whose
 * intermediates stay normal.  This program checks that on random operands
 * and on the hardest ones: quotients within about 2^-107 of a midpoint
 * between two binary64 numbers.  It also counts how often the first
 * correction alone is wrong, to show the cases bite.
 *
 * usage: division_f64 <n>   (n cases of each kind; prints "<m> mismatches")
 */
#include <math.h>
#include <stdint.h>
#include <stdio.h>
#include <stdlib.h>
#include <string.h>

static uint64_t sm_state;
static uint64_t splitmix64(void)
{
    uint64_t z = (sm_state += 0x9e3779b97f4a7c15ull);
    z = (z ^ (z >> 30)) * 0xbf58476d1ce4e5b9ull;
    z = (z ^ (z >> 27)) * 0x94d049bb133111ebull;
    return z ^ (z >> 31);
}

static double from_sig(uint64_t sig53, int e)   /* sig53 in [2^52, 2^53) */
{
    return ldexp((double)sig53, e - 52);
}

static long long bad2 = 0, bad1 = 0, hard = 0;

static void check(double a, double b)
{
    const double y = 1.0 / b;
    const double q0 = a * y;
    const double q1 = fma(-fma(b, q0, -a), y, q0);
    const double q2 = fma(-fma(b, q1, -a), y, q1);
    const double ref = a / b;
    if (memcmp(&q2, &ref, 8) != 0) {
        if (bad2 < 10) printf("mismatch a=%a b=%a q2=%a ref=%a\n", a, b, q2, ref);
        ++bad2;
    }
    if (memcmp(&q1, &ref, 8) != 0) ++bad1;
}

int main(int argc, char** argv)
{
    const long long n = argc > 1 ? atoll(argv[1]) : 1000000;
    sm_state = 12345;
    const uint64_t top = 1ull << 52, mask = top - 1;
    for (long long i = 0; i < n; ++i) {
        /* random significands, exponents spread over +-60 and the signs */
        const uint64_t r = splitmix64();
        double a = from_sig(top | (splitmix64() & mask), (int)(r % 121) - 60);
        double b = from_sig(top | (splitmix64() & mask), (int)((r >> 8) % 121) - 60);
        if (r & (1ull << 20)) a = -a;
        if (r & (1ull << 21)) b = -b;
        check(a, b);
        /* quotients in the code range of a group: |a/b| <= 255 */
        check(ldexp(a, -(int)ilogb(a)) * (double)(r >> 56), from_sig(top | (splitmix64() & mask), -7));
    }
    for (long long i = 0; i < n; ++i) {
        /* a/b within d * 2^-105 of the midpoint m / 2^53 (m odd, 54 bits):
         * A * 2^53 = B * m + d with B odd, d small and odd, so
         * m = -d * B^-1 mod 2^53 (+ 2^53) and A = (B * m + d) / 2^53. */
        const uint64_t B = top | (splitmix64() & mask) | 1ull;
        uint64_t inv = B;                                   /* B^-1 mod 2^64 by Newton */
        for (int k = 0; k < 6; ++k) inv *= 2 - B * inv;
        const int64_t d = (int64_t)(splitmix64() % 16) * 2 - 15;   /* odd, -15..15 */
        const uint64_t m = (((uint64_t)(-d) * inv) & ((1ull << 53) - 1)) | (1ull << 53);
        const __int128 num = (__int128)((unsigned __int128)B * m) + d;
        if (num & (((__int128)1 << 53) - 1)) return 2;      /* construction broken */
        const __int128 A = num >> 53;
        if (A < (__int128)top || A >= ((__int128)1 << 53)) continue;
        const int e = (int)(splitmix64() % 41) - 20;
        check(from_sig((uint64_t)A, e), from_sig(B, e));
        check(-from_sig((uint64_t)A, e + 3), from_sig(B, e - 1));
        ++hard;
    }
    printf("%lld near-midpoint pairs; first correction alone: %lld wrong\n", hard, bad1);
    printf("two corrections: %lld mismatches\n", bad2);
    return bad2 != 0;
}
