/* Exhaustive check of the division-free quotient used by the GPU kernels.
 *
 * For a scale S > 0 the kernels compute R = fl(1/S) once, then per element
 *   q0 = fl(a * R);  r = fma(-q0, S, a);  q = fma(r, R, q0)
 * and round q onto the E2M1 grid.  The specification rounds fl(a / S).
 * q is within one ulp of fl(a/S) (the FMA residual is exact and the
 * correction leaves less than 0.51 ulp of error), so the two can only land
 * in different E2M1 bins when a/S is within an ulp or two of a bin boundary
 * t in {0.25, 0.75, 1.25, 1.75, 2.5, 3.5, 5}, or decide the
 * straight-through mask |a/S| <= 6 differently.  In the normal range the
 * rounding of both sequences is invariant under a -> 2^j a, S -> 2^j S, so
 * checking every S in [1, 2) (all 2^23 mantissas) and every a within a few
 * ulps of t * S covers every scale in [2^-100, 2^100].
 *
 * Compile with FMA (gcc -O2 -mfma -ffp-contract=off); fmaf and the IEEE
 * operations of the CPU round exactly like the GPU's.  Returns the number
 * of bin mismatches and counts the quotient mismatches (both 0 expected:
 * with a correctly rounded reciprocal the corrected quotient is itself
 * correctly rounded).
 */
#include <math.h>
#include <stdint.h>
#include <stdio.h>
#include <string.h>

static float fb(uint32_t u) { float f; memcpy(&f, &u, 4); return f; }
static uint32_t bf(float f) { uint32_t u; memcpy(&u, &f, 4); return u; }

/* E2M1 bin of a non-negative quotient, by comparison with the boundaries
 * (ties to the even code: > for 0.25, 1.25, 2.5, 5; >= for 0.75, 1.75, 3.5) */
static int bin(float u)
{
    if (isnan(u)) return -1;
    return (u > 0.25f) + (u >= 0.75f) + (u > 1.25f) + (u >= 1.75f) + (u > 2.5f) + (u >= 3.5f) + (u > 5.0f);
}

int check_markstein(uint32_t mant_lo, uint32_t mant_hi, int radius, uint64_t* n_checked,
                    uint64_t* quot_mismatch)
{
    static const float T[8] = {0.25f, 0.75f, 1.25f, 1.75f, 2.5f, 3.5f, 5.0f, 6.0f};
    int bad = 0;
    uint64_t n = 0, qm = 0;
    for (uint32_t m = mant_lo; m < mant_hi; ++m) {
        float S = fb(0x3F800000u | m);
        float R = 1.0f / S;
        for (int k = 0; k < 8; ++k) {
            uint32_t c = bf(T[k] * S);
            for (int d = -radius; d <= radius; ++d) {
                float a = fb(c + d);
                float ref = a / S;
                float q0 = a * R;
                float r = fmaf(-q0, S, a);
                float q = fmaf(r, R, q0);
                ++n;
                if (q != ref) ++qm;
                if (bin(q) != bin(ref)) {
                    if (bad < 10) printf("mismatch S=%a a=%a ref=%a q=%a\n", S, a, ref, q);
                    ++bad;
                }
            }
        }
    }
    *n_checked = n;
    *quot_mismatch = qm;
    return bad;
}

/* The same quotient for the scale code of a block, s = RNE_E4M3(fl(a / d))
 * (E4M3, UE5M3) with d = fl(6 g) or fl(4 g) and R = fl(1/d) computed once
 * per call.  The 3-bit-mantissa rounding of two adjacent fp32 quotients can
 * only differ when one of them is a grid point or a midpoint of that
 * format; relative to their binade these are the values 1 + k/16, k = 0..15
 * (the subnormal codes of both formats land on the same relative values).
 * Every divisor mantissa and every dividend within `radius` ulps of
 * fl((1 + k/16) d) is checked: the quotients must be identical. */
int check_markstein_scale(uint32_t mant_lo, uint32_t mant_hi, int radius, uint64_t* n_checked)
{
    int bad = 0;
    uint64_t n = 0;
    for (uint32_t m = mant_lo; m < mant_hi; ++m) {
        float S = fb(0x3F800000u | m);
        float R = 1.0f / S;
        for (int k = 0; k < 16; ++k) {
            uint32_t c = bf((1.0f + (float)k / 16.0f) * S);
            for (int d = -radius; d <= radius; ++d) {
                float a = fb(c + d);
                float ref = a / S;
                float q0 = a * R;
                float r = fmaf(-q0, S, a);
                float q = fmaf(r, R, q0);
                ++n;
                if (q != ref) {
                    if (bad < 10) printf("scale quotient mismatch S=%a a=%a ref=%a q=%a\n", S, a, ref, q);
                    ++bad;
                }
            }
        }
    }
    *n_checked = n;
    return bad;
}
