/*
 * Test infrastructure, not product code: a float32 CPU model of the
 * software exp2 used by the attention path (degree 3, and the degree-4 and
 * degree-5 variants). Only the test suite, the smoke check and the bench's
 * CPU-baseline leg load it.
 *
 * Source: "FlashAttention-4's Softmax Tricks: A Degree-3 exp2 on the FMA
 * Pipe, and a Lagging Max That Saturated FP8", section "The emulated exp2"
 * (the split 2^x = 2^floor(x) * 2^frac(x), the clamp at -127, the round-down
 * add of 2^23 + 2^22, the degree-3 Horner polynomial with p0 = 1 and the
 * integer shift-and-add into the exponent field); restated as prose on the
 * KernelWiki page "Software-Emulated Exponential" (Cody-Waite reduction,
 * Sollya polynomial in Horner form, integer part through the exponent).
 *
 * Each Horner step is one correctly rounded fused multiply-add (fmaf), the
 * operation the GPU's v_fma_f32 performs. Build with -ffp-contract=off so
 * the compiler adds no other contraction.
 */
#include <math.h>
#include <stdint.h>
#include <string.h>

/* Degree-3 coefficients printed on the first page (relative-error minimax,
 * constant term 1). Each is exactly representable in float32. */
static const float kP0 = 1.0f;
static const float kP1 = 0.695146143436431884765625f;
static const float kP2 = 0.227564394474029541015625f;
static const float kP3 = 0.077119089663028717041015625f;

/* Degree-4 and degree-5 coefficients, not printed on the pages (their error
 * rows are): fitted the same way, relative-error minimax with constant term
 * 1, rounded to float32 (oracle/fit_ex2_poly.py). */
static const float kQ4[5] = {1.0f, 0.693044841289520263671875f, 0.2412802278995513916015625f,
                             0.05224247276782989501953125f, 0.013426683843135833740234375f};
static const float kQ5[6] = {1.0f, 0.693151295185089111328125f, 0.2401644885540008544921875f,
                             0.055799908936023712158203125f, 0.009017030708491802215576171875f,
                             0.001867130049504339694976806640625f};

static uint32_t bits_of(float f) { uint32_t u; memcpy(&u, &f, 4); return u; }
static float float_of(uint32_t u) { float f; memcpy(&f, &u, 4); return f; }

float ex2_emu_deg3_one(float x)
{
    /* 1. clamp from below so the integer part stays in the exponent range */
    float xc = fmaxf(x, -127.0f);
    /* 2. round-down add of 2^23 + 2^22: the low mantissa bits of the sum
     *    hold floor(xc); floorf followed by an exact add is the same value */
    const float magic = 12582912.0f;            /* 2^23 + 2^22 */
    float x_rounded = floorf(xc) + magic;       /* exact: |floor| < 2^22 */
    /* 3. fractional part, exact, in [0, 1] */
    float x_frac = xc - (x_rounded - magic);
    /* 4. 2^frac by Horner, highest coefficient first, one FMA per step */
    float p = kP3;
    p = fmaf(p, x_frac, kP2);
    p = fmaf(p, x_frac, kP1);
    p = fmaf(p, x_frac, kP0);
    /* 5. shift the integer part into the exponent field and add (a 32-bit
     *    two's-complement add; unsigned here only to keep C well defined) */
    uint32_t e = bits_of(x_rounded) << 23;
    return float_of(e + bits_of(p));
}

void ex2_emu_deg3(const float* x, float* y, long n)
{
    for (long i = 0; i < n; ++i) y[i] = ex2_emu_deg3_one(x[i]);
}

/* The same steps with the degree-4 or degree-5 polynomial (Horner, one fmaf
 * per step, highest coefficient first). Other degrees leave y untouched. */
void ex2_emu_poly(const float* x, float* y, long n, int degree)
{
    const float* c = degree == 4 ? kQ4 : degree == 5 ? kQ5 : 0;
    if (degree == 3) { ex2_emu_deg3(x, y, n); return; }
    if (!c) return;
    for (long i = 0; i < n; ++i) {
        float xc = fmaxf(x[i], -127.0f);
        const float magic = 12582912.0f;
        float x_rounded = floorf(xc) + magic;
        float x_frac = xc - (x_rounded - magic);
        float p = c[degree];
        for (int k = degree - 1; k >= 0; --k) p = fmaf(p, x_frac, c[k]);
        y[i] = float_of((bits_of(x_rounded) << 23) + bits_of(p));
    }
}
