/* div_refined_check.c -- host check of the shared-divisor division the NVFP4
 * quantizers use on the GPU (test infrastructure, not part of the library).
 *
 * The kernels divide every value a of a block by the block step b as
 *     y  = y0 + y0 (1 - b y0)            (y0: the hardware reciprocal of b)
 *     q0 = a y;  q1 = q0 - (b q0 - a) y;  q = q1 - (b q1 - a) y   (each step an FMA)
 * and expect q to carry the sign of a, also for a = -0.
 * This program checks, for divisors b in [2^-59, 2^59] and numerators that
 * matter for the codes, that q equals the correctly rounded a / b for every y0
 * within one ulp of 1/b (the hardware reciprocal's stated accuracy), on random
 * operands and on operands built to sit at or next to rounding boundaries of
 * the quotient.  Usage: div_refined_check <seed> <divisors> <values-per-divisor>.
 * Prints one line and exits 0 when every quotient matched, 1 otherwise. */
#include <math.h>
#include <stdint.h>
#include <stdio.h>
#include <stdlib.h>
#include <string.h>

static uint64_t st;
static uint64_t next(void) /* splitmix64 */
{
    uint64_t z = (st += 0x9E3779B97F4A7C15ull);
    z = (z ^ (z >> 30)) * 0xBF58476D1CE4E5B9ull;
    z = (z ^ (z >> 27)) * 0x94D049BB133111EBull;
    return z ^ (z >> 31);
}
static float bits(uint32_t u) { float f; memcpy(&f, &u, 4); return f; }
static uint32_t ubits(float f) { uint32_t u; memcpy(&u, &f, 4); return u; }

static float refine(float b, float y0) { return fmaf(fmaf(-b, y0, 1.0f), y0, y0); }
static float divr(float a, float b, float y)
{
    volatile float q0 = a * y;
    float q1 = fmaf(-fmaf(b, q0, -a), y, q0);
    return fmaf(-fmaf(b, q1, -a), y, q1);
}

int main(int argc, char **argv)
{
    st = argc > 1 ? strtoull(argv[1], 0, 10) : 1;
    long nb = argc > 2 ? atol(argv[2]) : 2000, na = argc > 3 ? atol(argv[3]) : 2000;
    static const float thr[] = {0.25f, 0.75f, 1.25f, 1.75f, 2.5f, 3.5f, 5.0f, 0.5f, 1.0f, 1.5f, 2.0f, 3.0f,
                                4.0f, 6.0f, 448.0f, 0x1p-10f, 0x1.8p-9f, 0x1p-6f};
    long checked = 0, bad = 0;
    for (long i = 0; i < nb; ++i) {
        /* divisor: random mantissa, exponent in [-59, 58] */
        const int e = (int)(next() % 118) - 59;
        const float b = bits(((uint32_t)(e + 127) << 23) | (uint32_t)(next() & 0x7FFFFF));
        const float r = 1.0f / b;
        const float ys[3] = {nextafterf(r, 0.0f), r, nextafterf(r, INFINITY)};
        for (long j = 0; j < na; ++j) {
            float a;
            const uint64_t k = next();
            switch (k % 4) {
            case 0: /* random quotient in [2^-12, 2^5) */
                a = b * bits(((uint32_t)(115 + (k >> 8) % 17) << 23) | (uint32_t)((k >> 32) & 0x7FFFFF));
                break;
            case 1: { /* next to t b, t a code threshold or grid point */
                const float t = thr[(k >> 8) % (sizeof thr / sizeof thr[0])];
                a = t * b;
                for (int n = (int)((k >> 16) % 5) - 2; n; n += n > 0 ? -1 : 1)
                    a = nextafterf(a, n > 0 ? INFINITY : 0.0f);
                break;
            }
            case 2: { /* a / b close to a midpoint between two floats */
                const float q = bits(((uint32_t)(115 + (k >> 8) % 17) << 23) | (uint32_t)((k >> 32) & 0x7FFFFF));
                const double mid = ((double)q + (double)nextafterf(q, INFINITY)) / 2.0;
                a = (float)(mid * (double)b);
                for (int n = (int)((k >> 20) % 3) - 1; n; n = 0) a = nextafterf(a, n > 0 ? INFINITY : 0.0f);
                break;
            }
            default: /* tiny or zero numerators: only the code 0 matters, checked as q < 0.25 */
                a = (k >> 8) % 2 ? 0.0f : bits((uint32_t)((k >> 9) & 0x7FFFFFFF) % ubits(b * 0x1p-12f));
                break;
            }
            if (!isfinite(a)) continue;
            if ((k >> 40) & 1) a = -a;  /* both signs, -0 included */
            const float want = a / b;
            for (int m = 0; m < 3; ++m) {
                const float got = divr(a, b, refine(b, ys[m]));
                ++checked;
                const int tiny = fabsf(want) < 0x1p-11f;
                const int sign_ok = signbit(got) == signbit(want);
                if (!sign_ok || (tiny ? !(fabsf(got) < 0.125f) : ubits(got) != ubits(want))) {
                    if (bad < 5)
                        fprintf(stderr, "mismatch a=%a b=%a y0=%a got %a want %a\n", a, b, ys[m], got, want);
                    ++bad;
                }
            }
        }
    }
    printf("div_refined_check: %ld quotients, %ld mismatches\n", checked, bad);
    return bad != 0;
}
