/* CPU check of the arithmetic the GPU quantizer uses in place of divisions
 * (Q8_0 activation blocks, minfer README on the nano-inference page, M3.5 and
 * M14: d = max|x| / 127, q = round(x / d)).  It emulates the kernel's steps
 * with IEEE fp32 operations and fmaf, and compares them with the definitions:
 *
 *  scale   d = RN(a / 127) from q = RN(a * RN(1/127)), r = fma(-q, 127, a),
 *          d = fma(r, RN(1/127), q): every a in [1, 2), every a of the two
 *          binades at the guard ends, and a spread of binades in between.
 *  codes   for a reciprocal rc anywhere within one ulp of 1/d, wherever the
 *          kernel's test |fma(x, rc, -n)| < 1/2 - 2^-13 passes, the byte from
 *          fma(x, rc, 1.5 * 2^23) equals (int8) roundf(RN(x / d)).  Inputs:
 *          random blocks, and every x within 200 ulps of (k + 1/2) d and of
 *          k d, for every k, over many scales.
 *
 * Prints "ok <fast> <slow>" (counts of values the fast test accepted and
 * rejected) or the first mismatch, and exits non-zero on a mismatch.
 * Build: gcc -O2 -ffp-contract=off quant_fastpath_check.c -lm
 */
#include <math.h>
#include <stdint.h>
#include <stdio.h>
#include <string.h>

static float bits_f(uint32_t u) { float f; memcpy(&f, &u, 4); return f; }
static uint32_t f_bits(float f) { uint32_t u; memcpy(&u, &f, 4); return u; }

static float scale_fast(float a) {
    const float y = 1.0f / 127.0f;
    const float q = a * y;
    const float r = fmaf(-q, 127.0f, a);
    return fmaf(r, y, q);
}

static int check_scale_range(uint32_t lo, uint32_t hi) {  /* bit patterns [lo, hi) */
    for (uint32_t u = lo; u < hi; ++u) {
        const float a = bits_f(u);
        const float want = a / 127.0f;
        const float got = scale_fast(a);
        if (f_bits(got) != f_bits(want)) {
            printf("scale mismatch a=%a got=%a want=%a\n", a, got, want);
            return 1;
        }
    }
    return 0;
}

static long n_fast, n_slow;

/* One value x of a block with scale dd and reciprocal rc; returns 1 on a mismatch. */
static int check_value(float x, float dd, float rc) {
    const float magic = 0x1.8p23f;
    const float m = fmaf(x, rc, magic);
    const float dist = fmaf(x, rc, -(m - magic));
    if (!(fabsf(dist) < 0.5f - 0x1p-13f)) { ++n_slow; return 0; }
    ++n_fast;
    const int8_t got = (int8_t)(uint8_t)(f_bits(m) & 0xFFu);
    const int8_t want = (int8_t)(int)roundf(x / dd);
    if (got != want) {
        printf("code mismatch x=%a d=%a rc=%a got=%d want=%d\n", x, dd, rc, got, want);
        return 1;
    }
    return 0;
}

static uint64_t rng_state = 0x9E3779B97F4A7C15ull;
static uint64_t rng_next(void) {  /* splitmix64 */
    uint64_t z = (rng_state += 0x9E3779B97F4A7C15ull);
    z = (z ^ (z >> 30)) * 0xBF58476D1CE4E5B9ull;
    z = (z ^ (z >> 27)) * 0x94D049BB133111EBull;
    return z ^ (z >> 31);
}
static float rng_unit(void) { return (float)(rng_next() >> 40) * 0x1p-24f; }

static int check_codes_for(float a) {
    const float dd = a / 127.0f;
    if (!(dd >= 0x1p-125f && dd <= 0x1p125f)) return 0;  /* the kernel divides there */
    const float r0 = 1.0f / dd;
    const float rcs[3] = {nextafterf(r0, 0.0f), r0, nextafterf(r0, INFINITY)};
    for (int ri = 0; ri < 3; ++ri) {
        const float rc = rcs[ri];
        if (check_value(a, dd, rc) || check_value(-a, dd, rc)) return 1;
        for (int k = -127; k <= 127; ++k) {
            const float centers[2] = {((float)k + 0.5f) * dd, (float)k * dd};
            for (int c = 0; c < 2; ++c) {
                float x = centers[c];
                for (int s = 0; s < 200; ++s) x = nextafterf(x, -INFINITY);
                for (int s = 0; s <= 400; ++s, x = nextafterf(x, INFINITY))
                    if (fabsf(x) <= a && check_value(x, dd, rc)) return 1;
            }
        }
        for (int s = 0; s < 2000; ++s) {
            const float x = (2.0f * rng_unit() - 1.0f) * a;
            if (check_value(x, dd, rc)) return 1;
        }
    }
    return 0;
}

int main(void) {
    /* scale: [1, 2) exhaustively, both guard binades, and a spread between */
    if (check_scale_range(f_bits(1.0f), f_bits(2.0f))) return 1;
    if (check_scale_range(f_bits(0x1p-96f), f_bits(0x1p-95f))) return 1;
    if (check_scale_range(f_bits(0x1p95f), f_bits(0x1p96f))) return 1;
    for (int e = -96; e < 96; e += 7)
        for (int s = 0; s < 20000; ++s) {
            const float a = ldexpf(1.0f + rng_unit(), e);
            if (f_bits(scale_fast(a)) != f_bits(a / 127.0f)) {
                printf("scale mismatch a=%a\n", a);
                return 1;
            }
        }
    /* codes: scales from 2^-120 to 2^40, random mantissas, plus the block maxima
       whose scales sit exactly on powers of two */
    for (int e = -120; e <= 40; e += 1) {
        for (int s = 0; s < 3; ++s)
            if (check_codes_for(ldexpf(1.0f + rng_unit(), e))) return 1;
        if (check_codes_for(ldexpf(127.0f, e - 7))) return 1;
    }
    printf("ok %ld %ld\n", n_fast, n_slow);
    return 0;
}
