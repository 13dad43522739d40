// attn_device.h -- device-side building blocks shared by the gfx950 attention
// kernels: vector types, the two exp2 paths, cross-half lane exchange and the
// workgroup -> tile mapping. Everything here is __device__ and inlined.
#pragma once
#include <hip/hip_runtime.h>
#include <stdint.h>

namespace attn {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x4 __attribute__((ext_vector_type(4)));
typedef float floatx16 __attribute__((ext_vector_type(16)));
typedef float floatx4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));
typedef int32_t i32x8 __attribute__((ext_vector_type(8)));

constexpr float kNegInf = -__builtin_huge_valf();

// ---------------------------------------------------------------------------
// exp2. The hardware path is one v_exp_f32. The software path is the
// degree-3 emulation of "FlashAttention-4's Softmax Tricks" (section "The
// emulated exp2"): clamp at -127, split x into floor(x) and a fraction in
// [0, 1), evaluate 2^frac with a relative-error minimax cubic (p0 = 1) in
// Horner form, then add floor(x) into the exponent field with an integer add.
// On gfx950 the split uses v_fract_f32 and a floor-convert instead of the
// round-down add of 2^23 + 2^22 (the VALU has no per-instruction rounding
// mode); both give the same floor and fraction. v_fract_f32 keeps the
// fraction below 1.0, so for x in [-2^-25, 0) it returns 1 - 2^-24 where an
// exact subtraction would round to 1.0; either lies within the cubic's error.
// Valid for x <= 127; returns +0 for x <= -127 and for -inf.
// ---------------------------------------------------------------------------
__device__ __forceinline__ float exp2_hw(float x) { return __builtin_amdgcn_exp2f(x); }

__device__ __forceinline__ float exp2_emu(float x) {
  const float c1 = 0.695146143436431884765625f;
  const float c2 = 0.227564394474029541015625f;
  const float c3 = 0.077119089663028717041015625f;
  float xc = __builtin_fmaxf(x, -127.0f);
  float fr = __builtin_amdgcn_fractf(xc);
  int fl = (int)__builtin_floorf(xc);
  float p = __builtin_fmaf(__builtin_fmaf(__builtin_fmaf(c3, fr, c2), fr, c1), fr, 1.0f);
  return __builtin_bit_cast(float, ((uint32_t)fl << 23) + __builtin_bit_cast(uint32_t, p));
}

// The MIX policy: element j (0..15) of each lane's 16-score group goes through
// the software path when j < EMU16.
template <int EMU16>
__device__ __forceinline__ float exp2_sel(float x, int j) {
  if (EMU16 >= 16) return exp2_emu(x);
  if (EMU16 <= 0) return exp2_hw(x);
  return (j < EMU16) ? exp2_emu(x) : exp2_hw(x);
}

// ---------------------------------------------------------------------------
// Reductions across the two 32-lane halves of a wave (lane l and l ^ 32 hold
// the two halves of one query row). Both halves get the same result.
// ---------------------------------------------------------------------------
__device__ __forceinline__ float other_half(float x) { return __shfl_xor(x, 32, 64); }
__device__ __forceinline__ float max_halves(float x) { return __builtin_fmaxf(x, other_half(x)); }
__device__ __forceinline__ float sum_halves(float x) {
  const float y = other_half(x);
  // same operand order in both halves, so both get bit-identical sums
  return (threadIdx.x & 32) ? y + x : x + y;
}

// ---------------------------------------------------------------------------
// Workgroup -> logical tile. The dispatcher deals workgroups round-robin over
// the 8 XCDs (workgroup i lands on XCD i % 8). Re-numbering so that each XCD
// gets a contiguous range of logical ids keeps the query tiles of one head on
// one XCD, where they share that XCD's L2 copy of the head's K and V.
// ---------------------------------------------------------------------------
__device__ __forceinline__ int xcd_logical_id(int wg, int n) {
  const int xcd = wg & 7, slot = wg >> 3;
  const int per = n >> 3, rem = n & 7;
  return xcd < rem ? xcd * (per + 1) + slot : rem * (per + 1) + (xcd - rem) * per + slot;
}

}  // namespace attn
