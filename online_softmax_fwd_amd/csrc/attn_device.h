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

// The polynomial has degree DEG: 3 uses the coefficients the page prints;
// 4 and 5 use the same kind of fit (relative-error minimax, p0 = 1, float32
// coefficients), whose errors the page's table lists (3.05e-6 and 1.44e-7
// maximum relative error against 8.77e-5 for degree 3).
template <int DEG>
__device__ __forceinline__ float exp2_emu_deg(float x) {
  static_assert(DEG >= 3 && DEG <= 5, "degree");
  float xc = __builtin_fmaxf(x, -127.0f);
  float fr = __builtin_amdgcn_fractf(xc);
  int fl = (int)__builtin_floorf(xc);
  float p;
  if (DEG == 3) {
    p = __builtin_fmaf(0.077119089663028717041015625f, fr, 0.227564394474029541015625f);
    p = __builtin_fmaf(p, fr, 0.695146143436431884765625f);
  } else if (DEG == 4) {
    p = __builtin_fmaf(0.013426683843135833740234375f, fr, 0.05224247276782989501953125f);
    p = __builtin_fmaf(p, fr, 0.2412802278995513916015625f);
    p = __builtin_fmaf(p, fr, 0.693044841289520263671875f);
  } else {
    p = __builtin_fmaf(0.001867130049504339694976806640625f, fr, 0.009017030708491802215576171875f);
    p = __builtin_fmaf(p, fr, 0.055799908936023712158203125f);
    p = __builtin_fmaf(p, fr, 0.2401644885540008544921875f);
    p = __builtin_fmaf(p, fr, 0.693151295185089111328125f);
  }
  p = __builtin_fmaf(p, fr, 1.0f);
  return __builtin_bit_cast(float, ((uint32_t)fl << 23) + __builtin_bit_cast(uint32_t, p));
}
__device__ __forceinline__ float exp2_emu(float x) { return exp2_emu_deg<3>(x); }

// The MIX policy: element j (0..15) of each lane's 16-score group goes through
// the software path when j < EMU16. Two more codes select full emulation with
// the higher-degree polynomials.
constexpr int kEmuDeg4 = 17, kEmuDeg5 = 18;
template <int EMU16>
__device__ __forceinline__ float exp2_sel(float x, int j) {
  if (EMU16 == kEmuDeg4) return exp2_emu_deg<4>(x);
  if (EMU16 == kEmuDeg5) return exp2_emu_deg<5>(x);
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

// Where a (batch, head) slice lives. Dense tensors are [B, H, N, d]: slice bh
// starts at bh * N * d with rows d apart. Packed variable-length batches
// (cu_q != nullptr) are [total, H, d]: sequence b holds rows cu[b] .. cu[b+1]-1
// of every head, so slice (b, h) starts at (cu[b] * H + h) * d with rows H * d
// apart; its LSE entries start at h * total_q + cu_q[b] of an [H, total_q] array.
// Sequence bounds are clamped to [0, total] so that inconsistent offsets can
// only shorten a sequence, never move an access outside the tensors.
struct Slice {
  size_t qbase, kbase, lse;  // element offsets of row 0 (Q and O share a layout)
  int Nq, Nk;                // rows of this slice
  int rs;                    // elements between consecutive rows
};
__device__ __forceinline__ Slice slice_of(int bh, int H, int d, int Nq, int Nk, const int* cu_q, const int* cu_k,
                                          int total_q, int total_k) {
  Slice s;
  if (cu_q == nullptr) {
    s.qbase = (size_t)bh * Nq * d;
    s.kbase = (size_t)bh * Nk * d;
    s.lse = (size_t)bh * Nq;
    s.Nq = Nq;
    s.Nk = Nk;
    s.rs = d;
  } else {
    const int b = bh / H, h = bh - b * H;
    const int q0 = min(max(cu_q[b], 0), total_q), k0 = min(max(cu_k[b], 0), total_k);
    s.Nq = min(max(cu_q[b + 1], q0), total_q) - q0;
    s.Nk = min(max(cu_k[b + 1], k0), total_k) - k0;
    s.qbase = ((size_t)q0 * H + h) * d;
    s.kbase = ((size_t)k0 * H + h) * d;
    s.lse = (size_t)h * total_q + q0;
    s.rs = H * d;
  }
  return s;
}

// E8M0 scales of slice (b, h), one byte per 32x32 block of rows x d. Dense
// tensors are [B, H, N/32, d/32]. Packed batches address scales apart from
// the data ("Quantization along both axes and jagged tensors" on the MXFP8
// page: the FP8 data stays compact, only the scale tensors follow a layout
// of their own): scales are [rows, H, d/32] with sequence b's 32-row blocks
// starting at scale row off[b], so sequences may start at padded scale rows
// while their data rows are packed. Block r of the slice holds the scales
// of its rows 32r .. 32r+31; a sequence's last block may be partial. The
// offsets are clamped to [0, rows] and blocks past rows read as absent, so
// inconsistent offsets never move a read outside the scale tensor.
struct ScaleSlice {
  size_t qbase, kbase;  // byte offset of block 0 (K and V share a layout)
  int qblocks, kblocks; // blocks present
  uint32_t stride;      // bytes between consecutive blocks of the slice
};
__device__ __forceinline__ ScaleSlice scale_slice_of(int bh, int H, int d, int Nq, int Nk, const int* off_q,
                                                     const int* off_k, int rows_q, int rows_k) {
  ScaleSlice s;
  const int w = d / 32;
  const int nqb = (Nq + 31) / 32, nkb = (Nk + 31) / 32;
  if (off_q == nullptr) {
    s.qbase = (size_t)bh * nqb * w;
    s.kbase = (size_t)bh * nkb * w;
    s.qblocks = nqb;
    s.kblocks = nkb;
    s.stride = w;
  } else {
    const int b = bh / H, h = bh - b * H;
    const int q0 = min(max(off_q[b], 0), rows_q), k0 = min(max(off_k[b], 0), rows_k);
    s.qbase = ((size_t)q0 * H + h) * w;
    s.kbase = ((size_t)k0 * H + h) * w;
    s.qblocks = min(nqb, rows_q - q0);
    s.kblocks = min(nkb, rows_k - k0);
    s.stride = (uint32_t)(H * w);
  }
  return s;
}

// Causal query tiles differ in length: tile qt of a head needs its first
// qt+1 tiles' worth of keys. When the heads split evenly over the 8 XCDs, XCD
// x takes the heads bh = x (mod 8), all of whose tiles therefore share that
// XCD's L2, and hands them to its compute units longest first (all heads'
// last tiles, then their second-to-last, ...), so the short tiles fill the
// gaps at the end instead of a long tile starting last. Otherwise the tiles
// follow xcd_logical_id, longest first within each head. Either way the map
// from workgroup to (head, tile) is a bijection.
__device__ __forceinline__ void causal_tile_of(int wg, int n_wg, int n_qt, int& bh, int& qt) {
  const int n_bh = n_wg / n_qt;
  if ((n_bh & 7) == 0) {
    const int xcd = wg & 7, slot = wg >> 3, per = n_bh >> 3;
    qt = n_qt - 1 - slot / per;
    bh = (slot % per) * 8 + xcd;
  } else {
    const int logical = xcd_logical_id(wg, n_wg);
    bh = logical / n_qt;
    qt = n_qt - 1 - (logical - bh * n_qt);
  }
}

// ---------------------------------------------------------------------------
// K/V tile DMA: buffer_load_dwordx4 ... lds copies 16 bytes per lane from a
// buffer straight into LDS (lane i's bytes land at the LDS address in M0 plus
// 16 * i), with no VGPR staging. The buffer resource makes it a raw byte
// buffer of nbytes: offsets are 32-bit and range-checked (the check covers
// the whole offset), and bytes at or past nbytes arrive as zeros.
//
// The instruction is written as inline asm rather than through the compiler
// builtin: the compiler cannot tell which LDS buffer a DMA writes, so before
// an LDS read it waits for every DMA still in flight, whichever buffer it
// targets, which would serialise the prefetch of the next tile with the reads
// of the current one. The kernels order DMA and reads themselves: the issuing
// wave waits on its vector-memory counter (s_waitcnt vmcnt) before the
// workgroup barrier that precedes the reads, and no DMA targets a buffer
// before the barrier after its last read. The asm sets M0 itself; no compiler
// builtin that depends on M0 runs in these kernels. An SALU write of M0 needs
// one wait state before an LDS DMA reads it (the compiler puts the same s_nop
// between the two for its own LDS-DMA builtins on gfx950), hence the s_nop.
// ---------------------------------------------------------------------------
__device__ __forceinline__ u32x4 raw_buffer_rsrc(const void* base, uint32_t nbytes) {
  const uint64_t p = (uint64_t)base;
  return u32x4{(uint32_t)p, (uint32_t)(p >> 32) & 0xFFFFu, nbytes, 0x00020000u};
}
__device__ __forceinline__ uint32_t lds_address(const void* p) {
  return (uint32_t)(uintptr_t)(const __attribute__((address_space(3))) void*)p;
}
__device__ __forceinline__ void dma16(const u32x4& rs, const char* lds, uint32_t off) {
  const uint32_t m0 = __builtin_amdgcn_readfirstlane(lds_address(lds));
  asm volatile("s_mov_b32 m0, %0\n\ts_nop 0\n\tbuffer_load_dwordx4 %1, %2, 0 offen lds" ::"s"(m0), "v"(off), "s"(rs)
               : "memory");
}
// The same with the LDS destination as a wave-uniform 32-bit LDS address.
__device__ __forceinline__ void dma16_at(const u32x4& rs, uint32_t lds, uint32_t off) {
  asm volatile("s_mov_b32 m0, %0\n\ts_nop 0\n\tbuffer_load_dwordx4 %1, %2, 0 offen lds" ::"s"(lds), "v"(off), "s"(rs)
               : "memory");
}
// The raw buffer descriptor rs moved off bytes forward: the base advances
// (48-bit address) and the size shrinks by as much (off must not exceed it).
// A tile loop puts the tile's offset here (scalar arithmetic, once per tile)
// instead of into every lane's offset, and the range check still returns
// zeros past the end.
__device__ __forceinline__ u32x4 advance_rsrc(const u32x4& rs, uint32_t off) {
  const uint64_t b = (((uint64_t)(rs[1] & 0xFFFFu) << 32) | rs[0]) + off;
  return u32x4{(uint32_t)b, ((uint32_t)(b >> 32) & 0xFFFFu) | (rs[1] & 0xFFFF0000u), rs[2] - off, rs[3]};
}

}  // namespace attn
