/* Host check of the division steps the quantize kernel uses in place of an
 * IEEE fp32 division per element.
 *
 * Reciprocal: for a divisor b with a 16-bit significand, the hardware
 * reciprocal y0 (within one ulp of 1/b) refined by one Newton step,
 * fma(fma(-b, y0, 1), y0, y0), must be RN(1/b): checked from each of the
 * three floats around RN(1/b) (which include every float within one ulp of
 * 1/b), for every fp16 divisor and every bf16 divisor >= 1e-7.
 *
 * Quotient: with y = RN(1/b), q = RN(a*y) and the exact residual
 * r = fma(-q, b, a), RN(q + r*y) = fma(r, y, q) is compared with the IEEE
 * quotient a / b computed by the host's division.  Zeros are compared by
 * value (a signed zero does not change a code).
 *
 * Usage: division_check STRIDE
 *   part 0: the reciprocal, as above;
 *   part 1: every fp16 divisor >= 2^-24 against every numerator within four
 *           ulps of each half-integer quotient k + 1/2, k = 0..300, both signs
 *           (the quotients where a one-ulp difference could move a code), and
 *           every fp16 numerator whose quotient is at most 300;
 *   part 2: every bf16 divisor >= 1e-7 against the same half-integer
 *           neighbourhoods;
 *   part 3: the constant divisors 2^bits - 1 (bits 2..8) and 127 against every
 *           STRIDE-th non-negative finite fp32 value.
 * Prints one line per part: checks and mismatches. */
#include <math.h>
#include <stdint.h>
#include <stdio.h>
#include <stdlib.h>
#include <string.h>

static float u2f(uint32_t u) { float f; memcpy(&f, &u, 4); return f; }
static uint32_t f2u(float f) { uint32_t u; memcpy(&u, &f, 4); return u; }
static float h2f(uint32_t h) {
    const uint32_t e = (h >> 10) & 31, m = h & 1023;
    float v = e == 0 ? ldexpf((float)m, -24) : ldexpf((float)(m | 1024), (int)e - 25);
    return (h >> 15) ? -v : v;
}
static float step(float a, float b, float y) {
    const float q = a * y;
    const float r = fmaf(-q, b, a);
    return fmaf(r, y, q);
}
static int same(float x, float z) { return x == z || (isnan(x) && isnan(z)); }

static void near_halves(float b, long* n, long* bad) {
    const float y = 1.0f / b;
    for (int k = 0; k <= 300; ++k) {
        const float t = ((float)k + 0.5f) * b;
        if (!isfinite(t)) break;
        const uint32_t u = f2u(t);
        for (int d = -4; d <= 4; ++d) {
            for (int sg = 0; sg < 2; ++sg) {
                const float a = sg ? -u2f(u + d) : u2f(u + d);
                ++*n;
                if (!same(step(a, b, y), a / b)) ++*bad;
            }
        }
    }
}

static void recip_check(float b, long* n, long* bad) {
    const float r = 1.0f / b;
    for (int d = -1; d <= 1; ++d) {
        const float y0 = u2f(f2u(r) + d);
        const float y = fmaf(fmaf(-b, y0, 1.0f), y0, y0);
        ++*n;
        if (f2u(y) != f2u(r)) ++*bad;
    }
}

int main(int argc, char** argv) {
    const long stride = argc > 1 ? atol(argv[1]) : 97;
    long n = 0, bad = 0;
    for (uint32_t h = 1; h < 0x7c00; ++h) recip_check(h2f(h), &n, &bad);
    for (uint32_t h = 1; h < 0x7f80; ++h) {
        const float b = u2f(h << 16);
        if (b >= 1e-7f) recip_check(b, &n, &bad);
    }
    printf("recip %ld %ld\n", n, bad);
    n = bad = 0;
#pragma omp parallel for reduction(+ : n, bad) schedule(dynamic, 64)
    for (int hb = 1; hb < 0x7c00; ++hb) {
        const float b = h2f((uint32_t)hb);
        near_halves(b, &n, &bad);
        const float y = 1.0f / b;
        for (int ha = 0; ha < 0x7c00; ++ha) {
            const float a = h2f((uint32_t)ha);
            if (a / b > 300.0f) break;
            n += 2;
            if (!same(step(a, b, y), a / b)) ++bad;
            if (!same(step(-a, b, y), -a / b)) ++bad;
        }
    }
    printf("fp16 %ld %ld\n", n, bad);
    n = bad = 0;
#pragma omp parallel for reduction(+ : n, bad) schedule(dynamic, 64)
    for (int hb = 1; hb < 0x7f80; ++hb) {
        const float b = u2f((uint32_t)hb << 16);
        if (b < 1e-7f) continue;
        near_halves(b, &n, &bad);
    }
    printf("bf16 %ld %ld\n", n, bad);
    n = bad = 0;
    const int cs[8] = {3, 7, 15, 31, 63, 127, 255, 127};
    for (int ci = 0; ci < 8; ++ci) {
        const float b = (float)cs[ci], y = 1.0f / b;
#pragma omp parallel for reduction(+ : n, bad) schedule(static)
        for (long u = ci; u < 0x7f800000L; u += stride) {
            const float x = u2f((uint32_t)u);
            ++n;
            if (!same(step(x, b, y), x / b)) ++bad;
        }
    }
    printf("const %ld %ld\n", n, bad);
    return 0;
}
