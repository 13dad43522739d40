/*
 * Test infrastructure, not product code: a float32 CPU model of the
 * software exp2 used by the attention path (degree 3, and the degree-4 and
 * degree-5 variants). Only the test suite, the smoke check and the bench's
 * CPU-baseline leg load it.
 *
 * Source: "FlashAttention-4's Softmax Tricks: A Degree-3 exp2 on the FMA
 * Pipe, and a Lagging Max That Saturated FP8", section "The emulated exp2";
 * the KernelWiki page "Software-Emulated Exponential" describes the same
 * method in prose (Cody-Waite reduction, Horner polynomial, integer part
 * through the exponent).
 *
 * The mathematics: for x >= -127, write x = n + f with n = floor(x) an
 * integer and f in [0, 1). Then 2^x = 2^n * 2^f. The factor 2^f in [1, 2)
 * is approximated by a polynomial q(f) with q(0) = 1 (a relative-error
 * minimax fit on [0, 1]), evaluated by Horner's rule; the factor 2^n needs
 * no arithmetic at all, since multiplying a float32 by 2^n adds n to its
 * biased exponent field, i.e. adds n << 23 to its bit pattern. Inputs below
 * -127 are raised to -127 first, which keeps n within the exponent field and
 * sends -inf (a masked score) to exactly +0.
 *
 * Each Horner step is one correctly rounded fused multiply-add (fmaf), the
 * operation the GPU's v_fma_f32 performs. Build with -ffp-contract=off so
 * the compiler adds no other contraction.
 */
#include <math.h>
#include <stdint.h>
#include <string.h>

/* q(f) = sum_k c[k] f^k, constant term first.
 * Degree 3: the coefficients the first page prints (each exactly
 * representable in float32).
 * Degrees 4 and 5: not printed on the pages (their error rows are); fitted
 * the same way, relative-error minimax with c[0] = 1, rounded to float32
 * (oracle/fit_ex2_poly.py). */
static const float kDeg3[4] = {1.0f, 0.695146143436431884765625f, 0.227564394474029541015625f,
                               0.077119089663028717041015625f};
static const float kDeg4[5] = {1.0f, 0.693044841289520263671875f, 0.2412802278995513916015625f,
                               0.05224247276782989501953125f, 0.013426683843135833740234375f};
static const float kDeg5[6] = {1.0f, 0.693151295185089111328125f, 0.2401644885540008544921875f,
                               0.055799908936023712158203125f, 0.009017030708491802215576171875f,
                               0.001867130049504339694976806640625f};

static uint32_t float_bits(float f) { uint32_t u; memcpy(&u, &f, 4); return u; }
static float bits_float(uint32_t u) { float f; memcpy(&f, &u, 4); return f; }

/* 2^x with the polynomial c of the given degree. */
static float pow2_split(float x, const float* c, int degree)
{
    const float xc = fmaxf(x, -127.0f);
    const float n = floorf(xc);
    /* exact except for -0.5 < xc < 0, where 1 + xc rounds to the 2^-24
     * grid (and to 1.0 when xc >= -2^-25) */
    const float f = xc - n;
    float q = c[degree];
    for (int k = degree - 1; k >= 0; --k) q = fmaf(q, f, c[k]);
    /* scale by 2^n through the exponent field (two's-complement add of the
     * shifted integer; unsigned arithmetic keeps C well defined) */
    return bits_float(float_bits(q) + ((uint32_t)(int32_t)n << 23));
}

float ex2_emu_deg3_one(float x) { return pow2_split(x, kDeg3, 3); }

void ex2_emu_deg3(const float* x, float* y, long n)
{
    for (long i = 0; i < n; ++i) y[i] = pow2_split(x[i], kDeg3, 3);
}

/* Degree 3, 4 or 5; other degrees leave y untouched. */
void ex2_emu_poly(const float* x, float* y, long n, int degree)
{
    const float* c = degree == 3 ? kDeg3 : degree == 4 ? kDeg4 : degree == 5 ? kDeg5 : 0;
    if (!c) return;
    for (long i = 0; i < n; ++i) y[i] = pow2_split(x[i], c, degree);
}
