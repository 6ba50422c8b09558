/*
 * CPU check of the identity the KV-cache write uses for its division by
 * k_scale / v_scale: with y = RN(1/b), q = RN(a*y), r = a - b*q (exact in
 * one FMA) and q' = RN(q + r*y), q' equals the IEEE float32 quotient RN(a/b)
 * (Markstein's correction), as long as |a| and |q| lie in the ranges below
 * and y is normal (b in [2^-100, 2^100]).  Outside them the kernel divides.
 *
 * Usage: quotient_identity SAMPLES_PER_SCALE; prints "tested N mismatches M"
 * and exits non-zero on any mismatch.  Needs a hardware FMA (built with -mfma).
 */
#include <math.h>
#include <stdint.h>
#include <stdio.h>
#include <stdlib.h>
#include <string.h>

static uint64_t st = 0x9E3779B97F4A7C15ull;
static uint32_t rnd(void) { st ^= st << 13; st ^= st >> 7; st ^= st << 17; return (uint32_t)st; }
static float fbits(uint32_t u) { float f; memcpy(&f, &u, 4); return f; }
static uint32_t ubits(float f) { uint32_t u; memcpy(&u, &f, 4); return u; }

static float fast_quotient(float a, float b, float y) {
    float q = a * y;
    float aq = fabsf(q), aa = fabsf(a);
    if (aq >= 0x1p-100f && aq <= 0x1p100f && aa >= 0x1p-96f && aa <= 0x1p100f)
        return fmaf(fmaf(-q, b, a), y, q);
    return a / b;
}

int main(int argc, char **argv) {
    long n = argc > 1 ? atol(argv[1]) : 1000000;
    float scales[48];
    int ns = 0;
    const float fixed[] = {0.05f, 0.04f, 0.37f, 3.1f, 1.0f / 3.0f, 0.1f, 7.0f, 0x1p-100f, 0x1p100f, 0x1.fffffep-1f};
    for (int i = 0; i < 10; ++i) scales[ns++] = fixed[i];
    while (ns < 48)   /* random significands, exponents across [2^-100, 2^100) */
        scales[ns++] = fbits((rnd() & 0x007fffffu) | ((uint32_t)(27 + rnd() % 200) << 23));
    long tested = 0, bad = 0;
    for (int si = 0; si < ns; ++si) {
        const float b = scales[si];
        volatile float yv = 1.0f / b;
        const float y = yv;
        for (long k = 0; k < n; ++k) {
            /* random bit patterns, and values near quotients of small integers */
            float a = (k & 1) ? fbits(rnd()) : (float)((double)(rnd() % 4096) * b + (double)((int)(rnd() % 5) - 2) * 0x1p-20);
            if (!isfinite(a)) continue;
            float ref = a / b, got = fast_quotient(a, b, y);
            if (ubits(ref) != ubits(got) && !(isnan(ref) && isnan(got))) {
                if (bad < 5) printf("a=%a b=%a ieee=%a fast=%a\n", a, b, ref, got);
                ++bad;
            }
            ++tested;
        }
    }
    printf("tested %ld mismatches %ld\n", tested, bad);
    return bad != 0;
}
