/* The kernels' activation-code rule for one element, restated in C on the host
 * and compared with rint(h / sx) by IEEE division.
 *
 * Rule (scale sx >= 2^-100, inv = fp32(1/sx)): round the two products of h with
 * inv (1 -+ 2^-22) to integers by adding 1.5 * 2^23 with one rounding (an FMA);
 * where both give the same integer that is the code, otherwise the code comes
 * from the corrected quotient q2 (q0 = fp32(h inv), then twice
 * q <- fp32(q + fp32(h - sx q) inv), the residual by an FMA) rounded to the
 * nearest integer, ties to even.
 *
 *   rule_check SAMPLES     random scales and elements, |h| <= 127.01 sx
 *   rule_check exhaustive  every float h with sx/4 <= |h| <= 127.01 sx for a
 *                          set of scales (edge mantissas, powers of two,
 *                          maxima of bf16 rows divided by 127)
 * Prints one summary line; exit status 1 on any difference. */
#include <math.h>
#include <stdint.h>
#include <stdio.h>
#include <stdlib.h>
#include <string.h>

static const float kMagic = 12582912.0f; /* 1.5 * 2^23 */

static float from_bits(uint32_t u) { float f; memcpy(&f, &u, 4); return f; }
static uint32_t to_bits(float f) { uint32_t u; memcpy(&u, &f, 4); return u; }

static float corrected_quotient(float h, float sx, float inv) {
    float q0 = h * inv;
    float q1 = fmaf(fmaf(-sx, q0, h), inv, q0);
    return fmaf(fmaf(-sx, q1, h), inv, q1);
}

/* the code as an integer, and whether the corrected quotient decided it */
static int32_t rule_code(float h, float sx, float inv, float inv_lo, float inv_hi, int* corrected) {
    float lo = fmaf(h, inv_lo, kMagic), hi = fmaf(h, inv_hi, kMagic);
    *corrected = lo != hi;
    float c = *corrected ? corrected_quotient(h, sx, inv) + kMagic : lo;
    return (int32_t)(to_bits(c) - to_bits(kMagic));
}

static long n_checked = 0, n_corrected = 0, n_bad = 0;

static void check(float h, float sx, float inv, float inv_lo, float inv_hi) {
    int corr = 0;
    int32_t got = rule_code(h, sx, inv, inv_lo, inv_hi, &corr);
    int32_t want = (int32_t)rintf(h / sx);
    ++n_checked;
    n_corrected += corr;
    if (got != want) {
        if (n_bad < 8) printf("mismatch h=%a sx=%a rule %d division %d\n", h, sx, got, want);
        ++n_bad;
    }
}

static void check_scale(float sx) {
    float inv = 1.0f / sx;
    float inv_lo = inv * 0x1.fffff8p-1f, inv_hi = inv * 0x1.000004p+0f;
    uint32_t lo = to_bits(0.25f * sx), hi = to_bits(127.01f * sx);
    for (uint32_t u = lo; u <= hi; ++u) {
        check(from_bits(u), sx, inv, inv_lo, inv_hi);
        if ((u & 7u) == 0) check(-from_bits(u), sx, inv, inv_lo, inv_hi);
    }
}

static uint64_t state = 0x9E3779B97F4A7C15ull;
static uint64_t next(void) {
    state ^= state << 13; state ^= state >> 7; state ^= state << 17;
    return state;
}

int main(int argc, char** argv) {
    if (argc > 1 && strcmp(argv[1], "exhaustive") == 0) {
        const uint32_t scales[] = {
            0x3F7FFFFFu, 0x3F800000u, 0x3F800001u, /* around 1 */
            0x0D800000u, 0x0D800001u,              /* 2^-100 and the next float */
            0x7A7FFFFFu,                            /* large */
        };
        for (size_t i = 0; i < sizeof scales / sizeof scales[0]; ++i) check_scale(from_bits(scales[i]));
        /* bf16 row maxima over 127: 3.625, 1 and 255 (bf16 mantissas 0x68, 0, 0x7F) */
        check_scale(3.625f / 127.0f);
        check_scale(1.0f / 127.0f);
        check_scale(255.0f / 127.0f);
    } else {
        long samples = argc > 1 ? atol(argv[1]) : 1000000L;
        for (long i = 0; i < samples; ++i) {
            int e = (int)(next() % 201) - 100;
            float sx = ldexpf(1.0f + (float)(next() & 0x7FFFFFu) * 0x1p-23f, e);
            float inv = 1.0f / sx;
            float inv_lo = inv * 0x1.fffff8p-1f, inv_hi = inv * 0x1.000004p+0f;
            float h;
            switch (next() % 3) {
                case 0: /* uniform in [-127.01, 127.01] sx */
                    h = (float)(((double)(next() >> 11) * 0x1p-53 * 254.02 - 127.01) * (double)sx);
                    break;
                case 1: { /* within six floats of (n + 1/2) sx */
                    int n = (int)(next() % 255) - 127;
                    h = (float)(((double)n + 0.5) * (double)sx);
                    if (h != 0.0f) h = from_bits(to_bits(h) + (uint32_t)((int)(next() % 13) - 6));
                    break;
                }
                default: /* the row maximum 127 sx (rounded) over a power of two, either sign */
                    h = ldexpf((float)(127.0 * (double)sx), -(int)(next() % 8));
                    if (next() & 1) h = -h;
            }
            if (isfinite(h) && fabsf(h) <= 127.01f * sx) check(h, sx, inv, inv_lo, inv_hi);
        }
    }
    printf("checked %ld corrected %ld mismatches %ld\n", n_checked, n_corrected, n_bad);
    return n_bad != 0;
}
