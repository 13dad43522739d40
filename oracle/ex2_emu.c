/*
 * Test infrastructure, not product code: a float32 CPU model of the
 * degree-3 software exp2 used by the attention forward path. Only the test
 * suite, the smoke check and the bench's CPU-baseline leg load it.
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
