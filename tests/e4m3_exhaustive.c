/*
 * Exhaustive pin of the oracle's fp32 -> OCP E4M3FN encoder (test program).
 *
 * Every finite fp32 bit pattern (2^32 minus infinities and NaNs) goes through
 * oracle_f32_to_e4m3 and through an independent nearest-code search written
 * here from the format's closed form: a non-negative code c = E*8 + M
 * (4 exponent bits, 3 mantissa bits, bias 7) decodes to 2^(E-7) * (1 + M/8)
 * for E > 0 and to 2^-6 * M/8 for E = 0; 0x7E (448) is the largest finite
 * value and 0x7F is NaN.  The nearest code to |v| is the one whose value is
 * closest, ties to the code with an even mantissa (an even code); values at
 * or above 448 saturate to 0x7E; the sign bit is copied, so -0 -> 0x80.
 * The search locates the largest code not above |v| with frexp (no table,
 * no bisection, unlike the oracle) and compares it with the next code.
 * Distances are exact in double (both operands are short binary fractions).
 *
 * Prints the number of patterns checked and of mismatches (the first few in
 * full); exits 0 only when every pattern matches.
 */
#include <math.h>
#include <stdint.h>
#include <stdio.h>
#include <string.h>

#include "oracle.h"

static double code_value(int c) /* c in 0..0x7E */
{
    const int E = c >> 3, M = c & 7;
    return E == 0 ? ldexp((double)M / 8.0, -6) : ldexp(1.0 + (double)M / 8.0, E - 7);
}

static uint8_t nearest_code(float f)
{
    const uint8_t sign = signbit(f) ? 0x80 : 0x00;
    const double a = fabs((double)f);
    if (a >= 448.0) return (uint8_t)(sign | 0x7E);
    int lo; /* largest code whose value is <= a */
    if (a < ldexp(1.0, -6)) {
        lo = (int)floor(a * 512.0);               /* subnormal codes, spacing 2^-9 */
    } else {
        int e2;
        const double m = frexp(a, &e2);           /* a = m * 2^e2, m in [0.5, 1) */
        const int E = e2 - 1 + 7;                 /* a in [2^(E-7), 2^(E-6)) */
        const int M = (int)floor((2.0 * m - 1.0) * 8.0);
        lo = E * 8 + M;
    }
    if (code_value(lo) > a || (lo < 0x7E && code_value(lo + 1) <= a)) return 0xFF; /* search bug */
    const double dlo = a - code_value(lo), dhi = code_value(lo + 1) - a;
    int pick;
    if (dlo < dhi) pick = lo;
    else if (dhi < dlo) pick = lo + 1;
    else pick = (lo % 2 == 0) ? lo : lo + 1;
    return (uint8_t)(sign | pick);
}

int main(void)
{
    long long checked = 0, bad = 0;
    (void)oracle_f32_to_e4m3(1.0f);   /* the oracle builds its value table on first use */
#pragma omp parallel for reduction(+ : checked, bad) schedule(static)
    for (long long hi = 0; hi < 65536; ++hi) {
        for (uint32_t lo = 0; lo < 65536; ++lo) {
            const uint32_t u = ((uint32_t)hi << 16) | lo;
            if ((u & 0x7F800000u) == 0x7F800000u) continue; /* infinities and NaNs */
            float f;
            memcpy(&f, &u, 4);
            const uint8_t want = nearest_code(f), got = oracle_f32_to_e4m3(f);
            ++checked;
            if (want != got) {
                ++bad;
                if (bad <= 5) {
#pragma omp critical
                    printf("mismatch: bits 0x%08x (%.9g): oracle 0x%02x, nearest 0x%02x\n", u,
                           (double)f, got, want);
                }
            }
        }
    }
    printf("checked %lld finite fp32 patterns, %lld mismatches\n", checked, bad);
    return bad == 0 && checked == 4278190080LL ? 0 : 1;
}
