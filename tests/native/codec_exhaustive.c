/* Exhaustive check of the oracle's element encoders (test infrastructure).
 *
 * For every fp32 bit pattern (NaNs excepted) the oracle's E2M1 encoder must
 * return the code of the nearest of the magnitudes {0, 0.5, 1, 1.5, 2, 3, 4, 6}
 * ("NVFP4" wiki, section on the technical principle: E2M1 elements), ties going
 * to the code with an even mantissa bit, magnitudes past 6 saturating to 6, and
 * the sign bit kept; and for every non-negative fp32 pattern the E4M3 encoder
 * must return the nearest finite E4M3FN byte (0x00 .. 0x7E), ties to the even
 * byte, values past 448 saturating to 448.
 *
 * The reference here is written independently of the oracle's: it decodes every
 * candidate code from its bit fields, then takes the nearest candidate by fp64
 * distance (E2M1: all 8 magnitudes below 6, the largest one from 6 up; E4M3: a
 * binary search over the 127 finite magnitudes in increasing order, then the
 * nearer neighbour).
 *
 * usage: codec_exhaustive <path to libfp4oracle.so> [e2m1]
 * prints "<n> mismatches" per encoder and exits 0 when all are 0; with "e2m1"
 * only the E2M1 encoder is checked. */
#include <dlfcn.h>
#include <math.h>
#include <stdint.h>
#include <stdio.h>
#include <stdlib.h>
#include <string.h>

typedef void (*enc_fn)(const float *, int64_t, uint8_t *);

static double e2m1_mag(int c) /* magnitude of code c (0..7) from its fields */
{
    const int e = (c >> 1) & 3, m = c & 1;
    return e == 0 ? 0.5 * m : ldexp(1.0 + 0.5 * m, e - 1);
}

static uint8_t ref_e2m1(float f)
{
    const double a = fabs((double)f);
    int best = 7;  /* a >= 6 (and +inf): 6 is the nearest magnitude */
    if (a < 6.0) {
        /* a < 6 and every magnitude <= 6, so each distance is exact in fp64
         * wherever two of them could be close (a near a midpoint has an ulp of
         * at least 2^-25) */
        double bd = INFINITY;
        for (int c = 0; c < 8; ++c) {
            const double d = fabs(a - e2m1_mag(c));
            if (d < bd || (d == bd && (c & 1) == 0 && (best & 1) == 1)) {
                bd = d;
                best = c;
            }
        }
    }
    return (uint8_t)((signbit(f) ? 8 : 0) | best);
}

static double e4m3_tab[127]; /* magnitude of byte b, b = 0 .. 0x7E, increasing */

static uint8_t ref_e4m3(float f)
{
    const double q = (double)f;
    if (q >= e4m3_tab[126]) return 0x7E; /* 448 and above (and +inf) */
    int lo = 0, hi = 126;                /* e4m3_tab[lo] <= q < e4m3_tab[hi] */
    while (hi - lo > 1) {
        const int mid = (lo + hi) / 2;
        if (e4m3_tab[mid] <= q) lo = mid;
        else hi = mid;
    }
    const double dl = q - e4m3_tab[lo], dh = e4m3_tab[hi] - q;
    if (dl < dh) return (uint8_t)lo;
    if (dh < dl) return (uint8_t)hi;
    return (uint8_t)((lo & 1) == 0 ? lo : hi);
}

int main(int argc, char **argv)
{
    if (argc < 2) {
        fprintf(stderr, "usage: %s libfp4oracle.so\n", argv[0]);
        return 2;
    }
    void *h = dlopen(argv[1], RTLD_NOW);
    if (!h) {
        fprintf(stderr, "dlopen: %s\n", dlerror());
        return 2;
    }
    const int only_e2m1 = argc > 2 && strcmp(argv[2], "e2m1") == 0;
    enc_fn e2m1 = (enc_fn)dlsym(h, "fp4o_e2m1_encode_f32");
    enc_fn e4m3 = (enc_fn)dlsym(h, "fp4o_e4m3_encode_f32");
    if (!e2m1 || !e4m3) {
        fprintf(stderr, "missing symbols\n");
        return 2;
    }
    for (int b = 0; b < 127; ++b) {
        const int e = (b >> 3) & 15, m = b & 7;
        e4m3_tab[b] = e == 0 ? ldexp((double)m, -9) : ldexp(1.0 + m / 8.0, e - 7);
    }
    for (int b = 1; b < 127; ++b)
        if (!(e4m3_tab[b] > e4m3_tab[b - 1])) {
            fprintf(stderr, "E4M3 table not increasing at %d\n", b);
            return 2;
        }

    const int64_t chunk = (int64_t)1 << 22;
    const int64_t nchunks = ((int64_t)1 << 32) / chunk;
    long long bad2 = 0, bad3 = 0, seen2 = 0, seen3 = 0;
#pragma omp parallel reduction(+ : bad2, bad3, seen2, seen3)
    {
        float *v = malloc(sizeof(float) * chunk);
        uint8_t *o = malloc(chunk);
        if (!v || !o) abort();
#pragma omp for schedule(dynamic)
        for (int64_t c = 0; c < nchunks; ++c) {
            int64_t n = 0;
            for (int64_t i = 0; i < chunk; ++i) {
                const uint32_t u = (uint32_t)(c * chunk + i);
                float f;
                memcpy(&f, &u, 4);
                if (!isnan(f)) v[n++] = f;
            }
            e2m1(v, n, o);
            for (int64_t i = 0; i < n; ++i) {
                if (o[i] != ref_e2m1(v[i])) {
                    if (bad2 < 5) {
                        uint32_t u;
                        memcpy(&u, &v[i], 4);
                        printf("E2M1 mismatch at 0x%08x: oracle %u reference %u\n", u, o[i], ref_e2m1(v[i]));
                    }
                    ++bad2;
                }
            }
            seen2 += n;
            /* E4M3 takes non-negative inputs: the first half of the patterns */
            if (!only_e2m1 && c < nchunks / 2) {
                e4m3(v, n, o);
                for (int64_t i = 0; i < n; ++i) {
                    if (o[i] != ref_e4m3(v[i])) {
                        if (bad3 < 5) {
                            uint32_t u;
                            memcpy(&u, &v[i], 4);
                            printf("E4M3 mismatch at 0x%08x: oracle %u reference %u\n", u, o[i], ref_e4m3(v[i]));
                        }
                        ++bad3;
                    }
                }
                seen3 += n;
            }
        }
        free(v);
        free(o);
    }
    printf("E2M1: %lld patterns, %lld mismatches\n", seen2, bad2);
    printf("E4M3: %lld patterns, %lld mismatches\n", seen3, bad3);
    return (bad2 == 0 && bad3 == 0) ? 0 : 1;
}
