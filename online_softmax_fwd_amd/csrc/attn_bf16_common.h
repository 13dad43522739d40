// attn_bf16_common.h -- operand-layout helpers shared by the bf16 kernels
// (forward and backward) for v_mfma_f32_32x32x16_bf16 on gfx950.
#pragma once

#include "attn_device.h"

namespace attn {
namespace {

typedef short shortx4 __attribute__((ext_vector_type(4)));
typedef __attribute__((address_space(3))) shortx4 lds_shortx4;

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

// Cross-half reductions with v_permlane32_swap: it exchanges the upper half of
// one register with the lower half of the other, so (r[0], r[1]) is
// (x[l], x[l ^ 32]) in some order in every lane, and max/sum of the pair is
// the pair's reduction (the sum is formed lower half + upper half in both).
__device__ __forceinline__ float pl_max_halves(float x) {
  const uint32_t u = __builtin_bit_cast(uint32_t, x);
  const auto r = __builtin_amdgcn_permlane32_swap(u, u, false, false);
  return __builtin_fmaxf(__builtin_bit_cast(float, (uint32_t)r[0]), __builtin_bit_cast(float, (uint32_t)r[1]));
}
__device__ __forceinline__ float pl_sum_halves(float x) {
  const uint32_t u = __builtin_bit_cast(uint32_t, x);
  const auto r = __builtin_amdgcn_permlane32_swap(u, u, false, false);
  return __builtin_bit_cast(float, (uint32_t)r[0]) + __builtin_bit_cast(float, (uint32_t)r[1]);
}

}  // namespace
}  // namespace attn
