/* Test helper (not part of the library or the oracle): the quantiser's
 * binary32 quotient |x| / s restated in C from its description, and plain
 * IEEE division, so that a CPU test can compare the two.
 *
 * Restated steps: k = 2^64 when s < 2^-62, else 1; sk = s k; r = RN(1 / sk)
 * (0 when s = 0); with a = |x| k: q = RN(a r); e = RN(a - q sk) by one fused
 * multiply-add; q' = RN(q + e r) by one fused multiply-add; result min(q', 448).
 * Built with -ffp-contract=off so that only the written fmaf calls fuse. */
#include <math.h>

void quotient_fma(const float *x, const float *s, float *out, long n)
{
    long i;
    for (i = 0; i < n; ++i) {
        float si = s[i];
        float k = si < 0x1p-62f ? 0x1p64f : 1.0f;
        float sk = si * k;
        float r = si == 0.0f ? 0.0f : 1.0f / sk;
        float a = fabsf(x[i]) * k;
        float q = a * r;
        float e = fmaf(-q, sk, a);
        float qq = fmaf(e, r, q);
        out[i] = fminf(qq, 448.0f);
    }
}

void quotient_div(const float *x, const float *s, float *out, long n)
{
    long i;
    for (i = 0; i < n; ++i)
        out[i] = s[i] == 0.0f ? 0.0f : fminf(fabsf(x[i]) / s[i], 448.0f);
}
