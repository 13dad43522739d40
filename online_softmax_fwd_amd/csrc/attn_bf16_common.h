// attn_bf16_common.h -- operand-layout helpers shared by the bf16 kernels
// (forward and backward) for v_mfma_f32_32x32x16_bf16 on gfx950.
#pragma once

#include "attn_device.h"

namespace attn {
namespace {

typedef short shortx4 __attribute__((ext_vector_type(4)));
typedef __attribute__((address_space(3))) shortx4 lds_shortx4;
typedef __attribute__((address_space(3))) bf16x8 lds_bf16x8;

// A-operand row m of the S^T MFMA reads key key_of_row(m) of its 32-key
// block. With the 32x32 output layout (lane half h, element j <-> row 8*(j/4)
// + 4*h + j%4), this leaves keys 8h..8h+7 in elements 0..7 and keys
// 16+8h..16+8h+7 in elements 8..15 of each lane.
__device__ __forceinline__ int key_of_row(int m) {
  const int g = m >> 3, h = (m >> 2) & 1, r = m & 3;
  return ((g >> 1) << 4) | (h << 3) | ((g & 1) << 2) | r;
}

__device__ __forceinline__ void wait_own_loads() { asm volatile("s_waitcnt vmcnt(0)" ::: "memory"); }

// Workgroup barrier without a memory fence. __syncthreads() releases at
// workgroup scope, which makes every wave wait for all of its outstanding
// vector-memory operations, tile DMAs included, at every barrier. Here each
// wave waits for its own DMA explicitly (wait_own_loads) at the barrier before
// the data is read, so the barriers in between do not stall on loads still in
// flight. The LDS reads a wave issued must have returned before it passes (a
// later DMA may overwrite the buffer), and the asm's memory clobber keeps the
// compiler from moving memory accesses across it.
__device__ __forceinline__ void block_sync() { asm volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory"); }

// Row maxima on v_maximum3_f32 / v_maximum_f32 (IEEE maximum, which returns
// NaN if either input is NaN). fmaxf's maxNum semantics make the compiler
// quiet each input that it cannot prove non-signalling -- every MFMA result --
// with an extra v_max_f32 x, x, x before the first level of the tree. maximum
// needs no such step, so a tree over N values costs about N/2 instructions.
// The scores here are finite or -inf, where the two agree.
__device__ __forceinline__ float vmax(float a, float b) { return __builtin_elementwise_maximum(a, b); }
__device__ __forceinline__ float vmax3(float a, float b, float c) { return vmax(vmax(a, b), c); }
template <int N>
struct MaxTree3 {
  static __device__ __forceinline__ float run(const float (&t)[N]) {
    constexpr int M = (N + 2) / 3;
    float u[M];
#pragma unroll
    for (int i = 0; i < N / 3; ++i) u[i] = vmax3(t[3 * i], t[3 * i + 1], t[3 * i + 2]);
    if constexpr (N % 3 == 1) u[M - 1] = t[N - 1];
    if constexpr (N % 3 == 2) u[M - 1] = vmax(t[N - 2], t[N - 1]);
    return MaxTree3<M>::run(u);
  }
};
template <>
struct MaxTree3<1> {
  static __device__ __forceinline__ float run(const float (&t)[1]) { return t[0]; }
};
// maximum of the KB x 16 accumulator elements of one lane
template <int KB>
__device__ __forceinline__ float tree_max(const floatx16 (&x)[KB]) {
  float t[16 * KB];
#pragma unroll
  for (int kb = 0; kb < KB; ++kb)
#pragma unroll
    for (int e = 0; e < 16; ++e) t[16 * kb + e] = x[kb][e];
  return MaxTree3<16 * KB>::run(t);
}

// Cross-half reductions with v_permlane32_swap: it exchanges the upper half of
// one register with the lower half of the other, so (r[0], r[1]) is
// (x[l], x[l ^ 32]) in some order in every lane, and max/sum of the pair is
// the pair's reduction (the sum is formed lower half + upper half in both).
__device__ __forceinline__ float pl_max_halves(float x) {
  const uint32_t u = __builtin_bit_cast(uint32_t, x);
  const auto r = __builtin_amdgcn_permlane32_swap(u, u, false, false);
  return vmax(__builtin_bit_cast(float, (uint32_t)r[0]), __builtin_bit_cast(float, (uint32_t)r[1]));
}
__device__ __forceinline__ float pl_sum_halves(float x) {
  const uint32_t u = __builtin_bit_cast(uint32_t, x);
  const auto r = __builtin_amdgcn_permlane32_swap(u, u, false, false);
  return __builtin_bit_cast(float, (uint32_t)r[0]) + __builtin_bit_cast(float, (uint32_t)r[1]);
}

}  // namespace
}  // namespace attn
