/* Checks the division sequence the scale sweep uses against IEEE fp32
 * division (test infrastructure; built and run by tests/test_division.py).
 *
 * Sequence: y = RN(1/b); q = RN(a*y); r = fma(-q, b, a); q' = RN(fma(r, y, q)).
 * Markstein's theorem (fma-based division; Handbook of Floating-Point
 * Arithmetic, "Newton-Raphson-based division with an FMA") states that q' is
 * RN(a/b) when y = RN(1/b), q is within one ulp of a/b and nothing
 * overflows or underflows.  Checked here: every significand of b in [1, 2)
 * against a spread of numerators, then random pairs over the exponent range
 * the sweep uses (|a| up to 2^24, b in [2^-100, 2^101]).  Prints the number
 * of mismatches (0 expected). */
#include <math.h>
#include <stdint.h>
#include <stdio.h>
#include <string.h>

static float bits(uint32_t u) { float f; memcpy(&f, &u, 4); return f; }
static uint32_t ubits(float f) { uint32_t u; memcpy(&u, &f, 4); return u; }

static float div_seq(float a, float b)
{
    const float y = 1.0f / b;
    const float q = a * y;
    const float r = fmaf(-q, b, a);
    return fmaf(r, y, q);
}

static uint64_t state = 0x9E3779B97F4A7C15ull;
static uint32_t rnd(void)
{
    state ^= state << 13; state ^= state >> 7; state ^= state << 17;
    return (uint32_t)(state >> 11);
}

int main(void)
{
    uint64_t bad = 0, n = 0;
    /* all significands of b in [1, 2), 6 numerators each */
    for (uint32_t m = 0; m < (1u << 23); ++m) {
        const float b = bits(0x3F800000u | m);
        for (int k = 0; k < 6; ++k) {
            const float a = bits(0x3F800000u | (rnd() & 0x7FFFFFu)) * (float)(1 << (rnd() % 20));
            const float want = a / b, got = div_seq(a, b);
            bad += ubits(want) != ubits(got);
            ++n;
        }
    }
    /* random exponents: a in [2^-20, 2^24), b in [2^-100, 2^101] */
    for (int k = 0; k < 20000000; ++k) {
        const float a = ldexpf(bits(0x3F800000u | (rnd() & 0x7FFFFFu)), (int)(rnd() % 44) - 20) * ((rnd() & 1) ? -1.0f : 1.0f);
        const float b = ldexpf(bits(0x3F800000u | (rnd() & 0x7FFFFFu)), (int)(rnd() % 202) - 100);
        const float want = a / b, got = div_seq(a, b);
        if (isnormal(want)) {
            bad += ubits(want) != ubits(got);
            ++n;
        }
    }
    printf("%llu %llu\n", (unsigned long long)bad, (unsigned long long)n);
    return 0;
}
