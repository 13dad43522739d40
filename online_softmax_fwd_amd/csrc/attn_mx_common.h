// attn_mx_common.h -- helpers shared by the MXFP8 (e4m3 + E8M0) kernels,
// forward and backward, for v_mfma_scale_f32_32x32x64_f8f6f4 on gfx950.
#pragma once

#include "attn_bf16_common.h"
#include "attn_device.h"

namespace attn {
namespace {

typedef int intx2 __attribute__((ext_vector_type(2)));
typedef __attribute__((address_space(3))) intx2 lds_intx2;

// S^T A-operand row m reads key mx_key_of_row(m) of its 32-key block: the 32x32
// output then holds keys 16h + e (e = 0..15) in lane half h.
__device__ __forceinline__ int mx_key_of_row(int m) { return 16 * ((m >> 2) & 1) + 4 * (m >> 3) + (m & 3); }

__device__ __forceinline__ float max16(const floatx16& x) {
  float t[16];
#pragma unroll
  for (int e = 0; e < 16; ++e) t[e] = x[e];
  return MaxTree3<16>::run(t);
}
__device__ __forceinline__ float sum16(const floatx16& x) {
  float t[8];
#pragma unroll
  for (int e = 0; e < 8; ++e) t[e] = x[e] + x[e + 8];
#pragma unroll
  for (int w = 4; w >= 1; w >>= 1)
#pragma unroll
    for (int e = 0; e < w; ++e) t[e] = t[e] + t[e + w];
  return t[0];
}

// A dword with no defined value: the old operand of the first of the two
// v_cvt_pk_fp8_f32 that write a dword's low and high halves (an empty asm
// defines it, so no register is cleared first).
__device__ __forceinline__ int undef_dword() {
  int v;
  asm volatile("" : "=v"(v));
  return v;
}

// E8M0 byte of the smallest power of two X with amax / X <= 448 (e4m3's
// largest finite value), read off the float32 bits of amax >= 0: with
// amax = 1.f * 2^e, X = 2^(e-8) when 1.f <= 1.75, else 2^(e-7). Zero gives
// X = 1. Clamped to [1, 253] so X and 1/X are normal floats.
__device__ __forceinline__ uint32_t e8m0_of(float amax) {
  const uint32_t u = __builtin_bit_cast(uint32_t, amax);
  const int eb = (int)((u >> 23) & 0xFF);
  int byte = eb - 8 + ((u & 0x7FFFFF) > 0x600000 ? 1 : 0);
  byte = eb == 0 ? 127 : byte;
  return (uint32_t)__builtin_amdgcn_fmed3f((float)byte, 1.0f, 253.0f);
}

}  // namespace
}  // namespace attn
