// attn_bwd_mxfp8.hip -- block-scaled e4m3 (MXFP8) attention backward for gfx950,
// and the square-block MX quantiser it needs for dO.
//
// "PyTorch FlashAttention-4 adds MXFP8 block-scaled forward and backward for
// Blackwell", section "Quantization along both axes and jagged tensors": the
// backward products reduce along both axes (dP over d, dV and dK over the
// queries, dQ over the keys), so Q, K, V and dO carry one E8M0 scale per
// square 32x32 block, which makes one e4m3 payload valid for a product and
// its transpose; dS is quantised the same way, one scale per 32x32 block of
// (queries, keys), so that dK and dQ consume the same representation. Every
// product runs on v_mfma_scale_f32_32x32x64_f8f6f4 with the scales applied
// inside the MFMA (operand layout as in the forward MXFP8 kernel: lane l holds
// 32 bytes of row l % 32, bytes 0..15 of lanes m and m+32 form K-block 0,
// bytes 16..31 K-block 1; lane half h supplies the scale of K-block h).
//
//   bwd_mx_prep_kernel   D_i = sum_c dO_ic O_ic (dO dequantised, O bf16) and
//                        LSE_i * log2(e) (+inf for rows without keys).
//   bwd_mx_dkdv_kernel   4 waves x 32 keys; the workgroup's K and V rows in
//                        LDS as B operands (in registers they spill next to
//                        the dK and dV accumulators: 30 % slower); 64-query
//                        tiles of Q and dO (e4m3) DMA'd to LDS. Per tile and 32-query half: S = Q K^T and
//                        dP = dO V^T (permuted rows, so each lane holds 16
//                        consecutive queries), P = 2^(S*c - LSE*log2 e),
//                        dS = P * (dP - D). P <= 1 exactly (the true LSE is
//                        known), so P is stored times 2^8 with one fixed scale
//                        byte; dS gets the E8M0 byte of its 32x32 block's
//                        amax (a wave-wide max). Then dV^T += dO^T P and
//                        dK^T += Q^T dS over the 64 queries, A through
//                        ds_read_b64_tr_b8.
//   bwd_mx_dq_kernel     4 waves x 32 queries; K and V stream in 64-key tiles:
//                        S^T = K Q^T, dP^T = V dO^T, dS^T quantised per 32x32
//                        block as above, dQ^T += K^T dS^T (K^T through the
//                        transpose read).
// The two kernels recompute dS for each block from the same inputs; the
// blocks are the same 32x32 squares, so they quantise the same values (up to
// float32 summation order in S and dP).
#include "attn_device.h"
#include "attn_internal.h"
#include "attn_mx_common.h"

namespace attn {
namespace {

constexpr int kD = 128;
constexpr int kRB = kD;              // bytes per row (one byte per element)
constexpr int kCH = kRB / 16;        // 16-byte chunks per row
constexpr int kNW = 4;               // waves per workgroup
constexpr int kThreads = 64 * kNW;
constexpr int kTileRows = 64;        // query tile (dK/dV kernel), key tile (dQ kernel)
constexpr int kTile = kTileRows * kRB;
constexpr int kLoads = kTileRows * kCH / 64 / kNW;
static_assert(kLoads * 64 * kNW == kTileRows * kCH, "tile split");
constexpr int kPScaleByte = 127 - 8; // P is stored times 2^8
constexpr float kLog2e = 1.4426950408889634f;
constexpr uint32_t kUnitScales = 0x7F7F7F7Fu;  // four E8M0 bytes of scale 1

// Chunk swizzle of tiles read both as permuted rows and through the
// transpose read (position c ^ f(r)). LDS serves a 16-byte read 16 lanes at a
// time and an 8-byte read 32 lanes at a time, and each such group must touch
// 64 different banks; f, a map of row bits 1, 2 and 4 found by exhaustive
// search over such maps, does that for both patterns. It ignores row bits 3
// and 5, the steps between the rows of one transpose read and between 32-row
// blocks, so one per-lane offset serves all of them.
__device__ __forceinline__ int swz_mx(int r) { return (r & 6) ^ ((r >> 4) & 1); }

struct MxOffsets {
  uint32_t row[2][2];     // permuted-row read: [64-wide d step][16-byte half]
  uint32_t tr[4];         // transpose read: per 32-wide d block
  uint32_t ld[kLoads];    // DMA: byte offset of this lane's chunk within a tile
  __device__ __forceinline__ void init(int lane, int wave) {
    const int hh = lane >> 5, l32 = lane & 31;
    const int pr = mx_key_of_row(l32);
#pragma unroll
    for (int s = 0; s < 2; ++s)
#pragma unroll
      for (int w = 0; w < 2; ++w) row[s][w] = pr * kRB + 16 * ((4 * s + 2 * w + hh) ^ swz_mx(pr));
    const int L = lane & 15, gidx = (lane >> 4) & 1;
    const int vr = 16 * hh + (L >> 1);
#pragma unroll
    for (int db = 0; db < 4; ++db) tr[db] = vr * kRB + 16 * ((2 * db + gidx) ^ swz_mx(vr)) + 8 * (L & 1);
#pragma unroll
    for (int i = 0; i < kLoads; ++i) {
      const int pos = 64 * (wave + kNW * i) + lane;
      const int r = pos / kCH, p = pos % kCH;
      ld[i] = r * kRB + 16 * (p ^ swz_mx(r));
    }
  }
};

// A operand: rows 32*blk + mx_key_of_row(m) of a tile, d 64s .. 64s+63.
__device__ __forceinline__ i32x8 row_operand(const char* tile, const MxOffsets& o, int blk, int s) {
  const char* p = tile + blk * 32 * kRB;
  const u32x4 lo = *(const u32x4*)(p + o.row[s][0]);
  const u32x4 hi = *(const u32x4*)(p + o.row[s][1]);
  return i32x8{(int)lo[0], (int)lo[1], (int)lo[2], (int)lo[3], (int)hi[0], (int)hi[1], (int)hi[2], (int)hi[3]};
}

// A operand through the transpose read: element (m, k) = tile[row k][32 db + m]
// for the 64 rows of the tile (lane half h: rows 16h.. of each 32-row block).
__device__ __forceinline__ i32x8 tr_operand(const char* tile, const MxOffsets& o, int db) {
  i32x8 a;
#pragma unroll
  for (int r = 0; r < 4; ++r) {
    const char* p = tile + o.tr[db] + (32 * (r >> 1) + 8 * (r & 1)) * kRB;
    const intx2 v = __builtin_amdgcn_ds_read_tr8_b64_v2i32((lds_intx2*)p);
    a[2 * r] = v[0];
    a[2 * r + 1] = v[1];
  }
  return a;
}

// One row of e4m3 bytes as the B operand (lane half h: d 64s+16h.. and 64s+32+16h..).
__device__ __forceinline__ void load_row_mx(i32x8 (&f)[2], const uint8_t* row, bool ok, int hh) {
#pragma unroll
  for (int s = 0; s < 2; ++s) {
    const u32x4 lo = ok ? *(const u32x4*)(row + 64 * s + 16 * hh) : u32x4{0u, 0u, 0u, 0u};
    const u32x4 hi = ok ? *(const u32x4*)(row + 64 * s + 32 + 16 * hh) : u32x4{0u, 0u, 0u, 0u};
    f[s] = i32x8{(int)lo[0], (int)lo[1], (int)lo[2], (int)lo[3], (int)hi[0], (int)hi[1], (int)hi[2], (int)hi[3]};
  }
}

__device__ __forceinline__ uint32_t scale_word(const uint8_t* base, int blk, int nblk) {
  return blk < nblk ? *(const uint32_t*)(base + (size_t)blk * 4) : kUnitScales;
}

// Largest |x| over the wave's 64 lanes x 16 elements (one 32x32 block): a
// v_maximum3_f32 tree in the lane (|x| as a source modifier), then DPP lane
// swaps within each row of 16 (xor 1, xor 2, the other half of 8, the other
// half of 16) and the row and wave-half swaps of v_permlane16/32_swap.
template <int CTRL>
__device__ __forceinline__ float dpp_mov(float v) {
  return __builtin_bit_cast(float, __builtin_amdgcn_mov_dpp(__builtin_bit_cast(int, v), CTRL, 0xF, 0xF, false));
}
__device__ __forceinline__ float wave_absmax(const floatx16& x) {
  float t[16];
#pragma unroll
  for (int e = 0; e < 16; ++e) t[e] = __builtin_fabsf(x[e]);
  float m = MaxTree3<16>::run(t);
  m = vmax(m, dpp_mov<0xB1>(m));   // quad_perm [1,0,3,2]
  m = vmax(m, dpp_mov<0x4E>(m));   // quad_perm [2,3,0,1]
  m = vmax(m, dpp_mov<0x141>(m));  // row_half_mirror
  m = vmax(m, dpp_mov<0x140>(m));  // row_mirror
  const uint32_t u = __builtin_bit_cast(uint32_t, m);
  const auto r = __builtin_amdgcn_permlane16_swap(u, u, false, false);
  m = vmax(__builtin_bit_cast(float, (uint32_t)r[0]), __builtin_bit_cast(float, (uint32_t)r[1]));
  return pl_max_halves(m);
}

// 16 floats (times f) to e4m3 bytes, 4 per dword, in element order.
__device__ __forceinline__ void to_e4m3(const floatx16& x, float f, int (&out)[4]) {
#pragma unroll
  for (int w = 0; w < 4; ++w) {
    int v = 0;
    v = __builtin_amdgcn_cvt_pk_fp8_f32(x[4 * w] * f, x[4 * w + 1] * f, v, false);
    v = __builtin_amdgcn_cvt_pk_fp8_f32(x[4 * w + 2] * f, x[4 * w + 3] * f, v, true);
    out[w] = v;
  }
}

__device__ __forceinline__ float inv_scale_of(uint32_t byte) { return __builtin_bit_cast(float, (254u - byte) << 23); }

__device__ __forceinline__ void store_row_bf16(__bf16* row, const floatx16 (&acc)[4], float f, int hh) {
#pragma unroll
  for (int db = 0; db < 4; ++db)
#pragma unroll
    for (int g = 0; g < 4; ++g) {
      bf16x4 w;
#pragma unroll
      for (int r = 0; r < 4; ++r) w[r] = (__bf16)(acc[db][4 * g + r] * f);
      *(bf16x4*)(row + 32 * db + 8 * g + 4 * hh) = w;
    }
}

// ---------------------------------------------------------------------------
// Square-block MX quantiser: bf16 [rows, 128] -> e4m3 [rows, 128] + one E8M0
// byte per 32x32 block ([rows/32, 4]). Wave w of a workgroup takes d block w
// of 32 rows; lane l covers row l/2, elements 16*(l%2) .. +16 of the block.
// The byte is the smallest power of two X with amax / X <= 448; values are
// divided by X (exact) and rounded to nearest even by v_cvt_pk_fp8_f32.
// ---------------------------------------------------------------------------
__global__ __attribute__((amdgpu_flat_work_group_size(256, 256)))
void mx_quantize_kernel(const __bf16* __restrict__ x, uint8_t* __restrict__ q, uint8_t* __restrict__ sc) {
  const int lane = threadIdx.x & 63, w = threadIdx.x >> 6;
  const size_t row = (size_t)blockIdx.x * 32 + (lane >> 1);
  const int col = 32 * w + 16 * (lane & 1);
  const __bf16* p = x + row * kD + col;
  const bf16x8 a = __builtin_bit_cast(bf16x8, *(const u32x4*)p);
  const bf16x8 b = __builtin_bit_cast(bf16x8, *(const u32x4*)(p + 8));
  floatx16 v;
#pragma unroll
  for (int e = 0; e < 8; ++e) {
    v[e] = (float)a[e];
    v[8 + e] = (float)b[e];
  }
  const uint32_t byte = e8m0_of(wave_absmax(v));
  int out[4];
  to_e4m3(v, inv_scale_of(byte), out);
  *(u32x4*)(q + row * kD + col) = u32x4{(uint32_t)out[0], (uint32_t)out[1], (uint32_t)out[2], (uint32_t)out[3]};
  if (lane == 0) sc[(size_t)blockIdx.x * 4 + w] = (uint8_t)byte;
}

// ---------------------------------------------------------------------------
// Pre-pass: ws[2i] = LSE_i * log2(e) (+inf where LSE_i = -inf), ws[2i+1] = D_i
// with D_i = sum_c dO_ic O_ic, dO dequantised. 8 lanes per row, 16 elements each.
// ---------------------------------------------------------------------------
__global__ __attribute__((amdgpu_flat_work_group_size(256, 256)))
void bwd_mx_prep_kernel(const __bf16* __restrict__ O, const uint8_t* __restrict__ dO, const uint8_t* __restrict__ dOS,
                        const float* __restrict__ LSE, float* __restrict__ ws, long long rows) {
  const long long r = (long long)blockIdx.x * 32 + threadIdx.x / 8;
  const int part = threadIdx.x % 8;
  float acc = 0.0f;
  if (r < rows) {
    const u32x4 g = *(const u32x4*)(dO + r * kD + 16 * part);
    const bf16x8 o0 = __builtin_bit_cast(bf16x8, *(const u32x4*)(O + r * kD + 16 * part));
    const bf16x8 o1 = __builtin_bit_cast(bf16x8, *(const u32x4*)(O + r * kD + 16 * part + 8));
    const float xs = __builtin_bit_cast(float, (uint32_t)dOS[(r / 32) * 4 + part / 2] << 23);
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const auto lo = __builtin_amdgcn_cvt_pk_f32_fp8((int)g[i], false);
      const auto hi = __builtin_amdgcn_cvt_pk_f32_fp8((int)g[i], true);
      const float ov[4] = {(float)(i < 2 ? o0[4 * i] : o1[4 * i - 8]), (float)(i < 2 ? o0[4 * i + 1] : o1[4 * i - 7]),
                           (float)(i < 2 ? o0[4 * i + 2] : o1[4 * i - 6]), (float)(i < 2 ? o0[4 * i + 3] : o1[4 * i - 5])};
      acc = __builtin_fmaf(lo[0], ov[0], acc);
      acc = __builtin_fmaf(lo[1], ov[1], acc);
      acc = __builtin_fmaf(hi[0], ov[2], acc);
      acc = __builtin_fmaf(hi[1], ov[3], acc);
    }
    acc *= xs;
  }
#pragma unroll
  for (int w = 4; w >= 1; w >>= 1) acc += __shfl_xor(acc, w);
  if (r < rows && part == 0) {
    const float l = LSE[r];
    ws[2 * r] = l == kNegInf ? -kNegInf : l * kLog2e;
    ws[2 * r + 1] = acc;
  }
}

// ---------------------------------------------------------------------------
// dK, dV: workgroup = 4 waves x 32 keys of one head; query tiles of 64 rows.
// ---------------------------------------------------------------------------
template <bool CAUSAL>
__global__ __attribute__((amdgpu_flat_work_group_size(kThreads, kThreads), amdgpu_waves_per_eu(2, 2)))
void bwd_mx_dkdv_kernel(const uint8_t* __restrict__ Q, const uint8_t* __restrict__ K, const uint8_t* __restrict__ V,
                        const uint8_t* __restrict__ dO, const uint8_t* __restrict__ QS, const uint8_t* __restrict__ KS,
                        const uint8_t* __restrict__ VS, const uint8_t* __restrict__ dOS, const float* __restrict__ ws,
                        __bf16* __restrict__ dK, __bf16* __restrict__ dV, int Nq, int Nk, int n_kt, float c,
                        float scale, int bottom_right) {
  __shared__ __attribute__((aligned(1024))) char q0s[kTile];
  __shared__ __attribute__((aligned(1024))) char d0s[kTile];
  __shared__ __attribute__((aligned(1024))) char q1s[kTile];
  __shared__ __attribute__((aligned(1024))) char d1s[kTile];
  __shared__ __attribute__((aligned(16))) float w0s[2 * kTileRows];
  __shared__ __attribute__((aligned(16))) float w1s[2 * kTileRows];
  __shared__ __attribute__((aligned(1024))) char kls[32 * kNW * kRB];  // the workgroup's K rows
  __shared__ __attribute__((aligned(1024))) char vls[32 * kNW * kRB];  // and V rows

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int hh = lane >> 5, l32 = lane & 31;

  int bh, kt;
  if (CAUSAL) {
    causal_tile_of(blockIdx.x, gridDim.x, n_kt, bh, kt);
    kt = n_kt - 1 - kt;  // key blocks that start later see fewer queries
  } else {
    const int logical = xcd_logical_id(blockIdx.x, gridDim.x);
    bh = logical / n_kt;
    kt = logical - bh * n_kt;
  }
  const int k0 = kt * 32 * kNW;
  const int kw0 = k0 + 32 * wave;
  const int key = kw0 + l32;
  const bool key_ok = key < Nk;
  const size_t qbase = (size_t)bh * Nq * kD, kbase = (size_t)bh * Nk * kD;
  const int nqb = Nq / 32, nkb = Nk / 32;
  const uint8_t* qsb = QS + (size_t)bh * nqb * 4;
  const uint8_t* dsb = dOS + (size_t)bh * nqb * 4;
  const int diag = bottom_right ? Nk - Nq : 0;  // key j is hidden from query i when j > i + diag

  MxOffsets to;
  to.init(lane, wave);
  const u32x4 rq = raw_buffer_rsrc(Q + qbase, (uint32_t)(Nq * kRB));
  const u32x4 rdo = raw_buffer_rsrc(dO + qbase, (uint32_t)(Nq * kRB));
  const u32x4 rw = raw_buffer_rsrc(ws + (size_t)bh * Nq * 2, (uint32_t)(Nq * 8));

  // K and V rows of the workgroup's keys stay in LDS (registers would spill
  // next to the dK and dV accumulators); chunk c of row r sits at c ^ f(r),
  // f(r) = (r >> 1) & 7, so the B-operand reads (16 rows, one chunk) hit 16
  // bank groups. Keys past Nk read as zero.
  {
    const u32x4 rk = raw_buffer_rsrc(K + kbase, (uint32_t)(Nk * kRB));
    const u32x4 rv = raw_buffer_rsrc(V + kbase, (uint32_t)(Nk * kRB));
#pragma unroll
    for (int i = 0; i < 32 * kNW * kCH / 64 / kNW; ++i) {
      const int pos = 64 * (wave + kNW * i) + lane;
      const int r = pos / kCH, p = pos % kCH;
      const uint32_t off = (uint32_t)(k0 + r) * kRB + 16 * (p ^ ((r >> 1) & 7));
      dma16(rk, kls + 1024 * (wave + kNW * i), off);
      dma16(rv, vls + 1024 * (wave + kNW * i), off);
    }
  }
  const int krow = 32 * wave + l32;
  auto kv_operand = [&](const char* base, int s) __attribute__((always_inline)) -> i32x8 {
    const char* p = base + krow * kRB;
    const int f = (l32 >> 1) & 7;
    const u32x4 lo = *(const u32x4*)(p + 16 * ((4 * s + hh) ^ f));
    const u32x4 hi = *(const u32x4*)(p + 16 * ((4 * s + 2 + hh) ^ f));
    return i32x8{(int)lo[0], (int)lo[1], (int)lo[2], (int)lo[3], (int)hi[0], (int)hi[1], (int)hi[2], (int)hi[3]};
  };
  const int kb_idx = kw0 / 32;
  const int ksc = (int)(scale_word(KS + (size_t)bh * nkb * 4, kb_idx, nkb) >> (8 * hh));
  const int vsc = (int)(scale_word(VS + (size_t)bh * nkb * 4, kb_idx, nkb) >> (8 * hh));

  floatx16 dk[4], dv[4];
#pragma unroll
  for (int i = 0; i < 4; ++i) dk[i] = dv[i] = floatx16{};

  const int qlo = CAUSAL ? max(0, k0 - diag) : 0;
  const int t0 = qlo / kTileRows;
  const int nt = (Nq + kTileRows - 1) / kTileRows;

  auto load = [&](int t, char* qd, char* dd, float* wd) __attribute__((always_inline)) {
    const uint32_t off = (uint32_t)t * kTile;
#pragma unroll
    for (int i = 0; i < kLoads; ++i) {
      dma16(rq, qd + 1024 * (wave + kNW * i), to.ld[i] + off);
      dma16(rdo, dd + 1024 * (wave + kNW * i), to.ld[i] + off);
    }
    if (wave == 0 && lane < 32) dma16(rw, (const char*)wd, (uint32_t)t * (8 * kTileRows) + 16 * lane);
  };

  auto compute = [&](int t, const char* qs, const char* dos, const float* wsd) __attribute__((always_inline)) {
    const int q0 = t * kTileRows;
    if (CAUSAL && q0 + kTileRows - 1 + diag < kw0) return;  // wave-uniform: no query here sees the wave's keys
    int pq[8], sq[8];
    int dsb_byte[2];
#pragma unroll
    for (int sb = 0; sb < 2; ++sb) {
      const int qb = 2 * t + sb;
      const int qsc = (int)(scale_word(qsb, qb, nqb) >> (8 * hh));
      const int gsc = (int)(scale_word(dsb, qb, nqb) >> (8 * hh));
      floatx16 s = {}, dp = {};
      s = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(row_operand(qs, to, sb, 0), kv_operand(kls, 0), s, 0, 0, 0,
                                                          qsc, 0, ksc);
      s = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(row_operand(qs, to, sb, 1), kv_operand(kls, 1), s, 0, 0, 2,
                                                          qsc, 2, ksc);
      dp = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(row_operand(dos, to, sb, 0), kv_operand(vls, 0), dp, 0, 0,
                                                           0, gsc, 0, vsc);
      dp = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(row_operand(dos, to, sb, 1), kv_operand(vls, 1), dp, 0, 0,
                                                           2, gsc, 2, vsc);
      // element e of lane half h holds query q0 + 32 sb + 16 h + e
      const int qe0 = q0 + 32 * sb + 16 * hh;
      const float4* wp = (const float4*)(wsd + 2 * (32 * sb + 16 * hh));
      if (CAUSAL && qe0 - 16 * hh + diag < kw0 + 31) {  // masked pairs get S = -inf (one wave-uniform branch)
#pragma unroll
        for (int e = 0; e < 16; ++e)
          if (key > qe0 + e + diag) s[e] = kNegInf;
      }
#pragma unroll
      for (int i = 0; i < 8; ++i) {
        const float4 w = wp[i];  // rows 2i, 2i+1 of the lane's 16
#pragma unroll
        for (int j = 0; j < 2; ++j) {
          const int e = 2 * i + j;
          const float p = exp2_hw(__builtin_fmaf(s[e], c, -w[2 * j]));
          s[e] = p;
          dp[e] = p * (dp[e] - w[2 * j + 1]);
        }
      }
      const uint32_t byte = e8m0_of(wave_absmax(dp));
      dsb_byte[sb] = (int)byte;
      int pw[4], dw[4];
      to_e4m3(s, 256.0f, pw);
      to_e4m3(dp, inv_scale_of(byte), dw);
#pragma unroll
      for (int w = 0; w < 4; ++w) {
        pq[4 * sb + w] = pw[w];
        sq[4 * sb + w] = dw[w];
      }
      __builtin_amdgcn_sched_barrier(0);  // one 32-query half at a time (registers)
    }
    const i32x8 pb = {pq[0], pq[1], pq[2], pq[3], pq[4], pq[5], pq[6], pq[7]};
    const i32x8 db = {sq[0], sq[1], sq[2], sq[3], sq[4], sq[5], sq[6], sq[7]};
    const int ds_sc = hh ? dsb_byte[1] : dsb_byte[0];
    const int qsc_t = (int)scale_word(qsb, 2 * t + hh, nqb);
    const int gsc_t = (int)scale_word(dsb, 2 * t + hh, nqb);
#pragma unroll
    for (int d = 0; d < 4; ++d) {
      const i32x8 ga = tr_operand(dos, to, d);
      const i32x8 qa = tr_operand(qs, to, d);
      switch (d) {
        case 0:
          dv[0] = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(ga, pb, dv[0], 0, 0, 0, gsc_t, 0, kPScaleByte);
          dk[0] = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(qa, db, dk[0], 0, 0, 0, qsc_t, 0, ds_sc);
          break;
        case 1:
          dv[1] = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(ga, pb, dv[1], 0, 0, 1, gsc_t, 0, kPScaleByte);
          dk[1] = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(qa, db, dk[1], 0, 0, 1, qsc_t, 0, ds_sc);
          break;
        case 2:
          dv[2] = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(ga, pb, dv[2], 0, 0, 2, gsc_t, 0, kPScaleByte);
          dk[2] = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(qa, db, dk[2], 0, 0, 2, qsc_t, 0, ds_sc);
          break;
        default:
          dv[3] = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(ga, pb, dv[3], 0, 0, 3, gsc_t, 0, kPScaleByte);
          dk[3] = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(qa, db, dk[3], 0, 0, 3, qsc_t, 0, ds_sc);
          break;
      }
    }
  };

  if (t0 < nt) {
    load(t0, q0s, d0s, w0s);
    wait_own_loads();
    __syncthreads();
  }
  for (int t = t0; t < nt; ++t) {
    const bool odd = (t - t0) & 1;
    if (t + 1 < nt) load(t + 1, odd ? q0s : q1s, odd ? d0s : d1s, odd ? w0s : w1s);
    compute(t, odd ? q1s : q0s, odd ? d1s : d0s, odd ? w1s : w0s);
    wait_own_loads();
    __syncthreads();
  }

  if (key_ok) {
    store_row_bf16(dK + kbase + (size_t)key * kD, dk, scale, hh);
    store_row_bf16(dV + kbase + (size_t)key * kD, dv, 1.0f, hh);
  }
}

// ---------------------------------------------------------------------------
// dQ: workgroup = 4 waves x 32 queries of one head; key tiles of 64 keys.
// ---------------------------------------------------------------------------
template <bool CAUSAL>
__global__ __attribute__((amdgpu_flat_work_group_size(kThreads, kThreads), amdgpu_waves_per_eu(2, 2)))
void bwd_mx_dq_kernel(const uint8_t* __restrict__ Q, const uint8_t* __restrict__ K, const uint8_t* __restrict__ V,
                      const uint8_t* __restrict__ dO, const uint8_t* __restrict__ QS, const uint8_t* __restrict__ KS,
                      const uint8_t* __restrict__ VS, const uint8_t* __restrict__ dOS, const float* __restrict__ ws,
                      __bf16* __restrict__ dQ, int Nq, int Nk, int n_qt, float c, float scale, int bottom_right) {
  __shared__ __attribute__((aligned(1024))) char k0s[kTile];
  __shared__ __attribute__((aligned(1024))) char v0s[kTile];
  __shared__ __attribute__((aligned(1024))) char k1s[kTile];
  __shared__ __attribute__((aligned(1024))) char v1s[kTile];

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int hh = lane >> 5, l32 = lane & 31;

  int bh, qt;
  if (CAUSAL) {
    causal_tile_of(blockIdx.x, gridDim.x, n_qt, bh, qt);
  } else {
    const int logical = xcd_logical_id(blockIdx.x, gridDim.x);
    bh = logical / n_qt;
    qt = logical - bh * n_qt;
  }
  const int q0 = qt * 32 * kNW;
  const int qw0 = q0 + 32 * wave;
  const int qi = qw0 + l32;
  const bool row_ok = qi < Nq;
  const size_t qbase = (size_t)bh * Nq * kD, kbase = (size_t)bh * Nk * kD;
  const int nqb = Nq / 32, nkb = Nk / 32;
  const uint8_t* ksb = KS + (size_t)bh * nkb * 4;
  const uint8_t* vsb = VS + (size_t)bh * nkb * 4;
  const int diag = bottom_right ? Nk - Nq : 0;

  MxOffsets to;
  to.init(lane, wave);
  const u32x4 rk = raw_buffer_rsrc(K + kbase, (uint32_t)(Nk * kRB));
  const u32x4 rv = raw_buffer_rsrc(V + kbase, (uint32_t)(Nk * kRB));

  i32x8 qf[2], gf[2];
  load_row_mx(qf, Q + qbase + (size_t)(row_ok ? qi : 0) * kD, row_ok, hh);
  load_row_mx(gf, dO + qbase + (size_t)(row_ok ? qi : 0) * kD, row_ok, hh);
  const int qsc = (int)(scale_word(QS + (size_t)bh * nqb * 4, qw0 / 32, nqb) >> (8 * hh));
  const int gsc = (int)(scale_word(dOS + (size_t)bh * nqb * 4, qw0 / 32, nqb) >> (8 * hh));
  float l2 = -kNegInf, dd = 0.0f;  // rows past Nq: P = 0
  if (row_ok) {
    const float2 w = *(const float2*)(ws + ((size_t)bh * Nq + qi) * 2);
    l2 = w[0];
    dd = w[1];
  }

  floatx16 dq[4];
#pragma unroll
  for (int i = 0; i < 4; ++i) dq[i] = floatx16{};

  const int kend = CAUSAL ? min(Nk, q0 + 32 * kNW + diag) : Nk;
  const int T = kend > 0 ? (kend + kTileRows - 1) / kTileRows : 0;

  auto load = [&](int t, char* kd, char* vd) __attribute__((always_inline)) {
    const uint32_t off = (uint32_t)t * kTile;
#pragma unroll
    for (int i = 0; i < kLoads; ++i) {
      dma16(rk, kd + 1024 * (wave + kNW * i), to.ld[i] + off);
      dma16(rv, vd + 1024 * (wave + kNW * i), to.ld[i] + off);
    }
  };

  auto compute = [&](int t, const char* ks, const char* vs) __attribute__((always_inline)) {
    const int kk0 = t * kTileRows;
    if (CAUSAL && kk0 > qw0 + 31 + diag) return;  // wave-uniform: every key of the tile is hidden
    int sq[8];
    int ds_byte[2];
#pragma unroll
    for (int kb = 0; kb < 2; ++kb) {
      const int kblk = 2 * t + kb;
      const int ksc = (int)(scale_word(ksb, kblk, nkb) >> (8 * hh));
      const int vsc = (int)(scale_word(vsb, kblk, nkb) >> (8 * hh));
      floatx16 s = {}, dp = {};
      s = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(row_operand(ks, to, kb, 0), qf[0], s, 0, 0, 0, ksc, 0, qsc);
      s = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(row_operand(ks, to, kb, 1), qf[1], s, 0, 0, 2, ksc, 2, qsc);
      dp = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(row_operand(vs, to, kb, 0), gf[0], dp, 0, 0, 0, vsc, 0, gsc);
      dp = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(row_operand(vs, to, kb, 1), gf[1], dp, 0, 0, 2, vsc, 2, gsc);
      // element e of lane half h holds key kk0 + 32 kb + 16 h + e
      const int ke0 = kk0 + 32 * kb + 16 * hh;
      if ((CAUSAL && kk0 + 32 * kb + 31 > qw0 + diag) || (kk0 + 32 * kb + 32 > Nk)) {  // masked: S = -inf
#pragma unroll
        for (int e = 0; e < 16; ++e)
          if (ke0 + e >= Nk || (CAUSAL && ke0 + e > qi + diag)) s[e] = kNegInf;
      }
#pragma unroll
      for (int e = 0; e < 16; ++e) {
        const float p = exp2_hw(__builtin_fmaf(s[e], c, -l2));
        dp[e] = p * (dp[e] - dd);
      }
      const uint32_t byte = e8m0_of(wave_absmax(dp));
      ds_byte[kb] = (int)byte;
      int dw[4];
      to_e4m3(dp, inv_scale_of(byte), dw);
#pragma unroll
      for (int w = 0; w < 4; ++w) sq[4 * kb + w] = dw[w];
      __builtin_amdgcn_sched_barrier(0);  // one 32-key block at a time (registers)
    }
    const i32x8 db = {sq[0], sq[1], sq[2], sq[3], sq[4], sq[5], sq[6], sq[7]};
    const int ds_sc = hh ? ds_byte[1] : ds_byte[0];
    const int ksc_t = (int)scale_word(ksb, 2 * t + hh, nkb);
#pragma unroll
    for (int d = 0; d < 4; ++d) {
      const i32x8 ka = tr_operand(ks, to, d);
      switch (d) {
        case 0: dq[0] = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(ka, db, dq[0], 0, 0, 0, ksc_t, 0, ds_sc); break;
        case 1: dq[1] = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(ka, db, dq[1], 0, 0, 1, ksc_t, 0, ds_sc); break;
        case 2: dq[2] = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(ka, db, dq[2], 0, 0, 2, ksc_t, 0, ds_sc); break;
        default: dq[3] = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(ka, db, dq[3], 0, 0, 3, ksc_t, 0, ds_sc); break;
      }
    }
  };

  if (T > 0) {
    load(0, k0s, v0s);
    wait_own_loads();
    __syncthreads();
  }
  for (int t = 0; t < T; ++t) {
    const bool odd = t & 1;
    if (t + 1 < T) load(t + 1, odd ? k0s : k1s, odd ? v0s : v1s);
    compute(t, odd ? k1s : k0s, odd ? v1s : v0s);
    wait_own_loads();
    __syncthreads();
  }

  if (row_ok) store_row_bf16(dQ + qbase + (size_t)qi * kD, dq, scale, hh);
}

template <bool CAUSAL>
hipError_t launch_bwd_mx_c(const BwdArgs& a, hipStream_t stream) {
  const long long rows = (long long)a.B * a.H * a.Nq;
  hipError_t e = hipSuccess;
  if (rows > 0) {
    hipLaunchKernelGGL(bwd_mx_prep_kernel, dim3((unsigned)((rows + 31) / 32)), dim3(256), 0, stream,
                       (const __bf16*)a.o, (const uint8_t*)a.d_o, a.do_scale, a.lse, a.ws, rows);
    if ((e = hipGetLastError()) != hipSuccess) return e;
  }
  const int n_kt = (a.Nk + 32 * kNW - 1) / (32 * kNW);
  if (n_kt > 0) {
    hipLaunchKernelGGL((bwd_mx_dkdv_kernel<CAUSAL>), dim3((unsigned)((long long)a.B * a.H * n_kt)), dim3(kThreads), 0,
                       stream, (const uint8_t*)a.q, (const uint8_t*)a.k, (const uint8_t*)a.v, (const uint8_t*)a.d_o,
                       a.q_scale, a.k_scale, a.v_scale, a.do_scale, (const float*)a.ws, (__bf16*)a.d_k,
                       (__bf16*)a.d_v, a.Nq, a.Nk, n_kt, a.scale_log2, a.scale, a.bottom_right);
    if ((e = hipGetLastError()) != hipSuccess) return e;
  }
  const int n_qt = (a.Nq + 32 * kNW - 1) / (32 * kNW);
  if (n_qt > 0) {
    hipLaunchKernelGGL((bwd_mx_dq_kernel<CAUSAL>), dim3((unsigned)((long long)a.B * a.H * n_qt)), dim3(kThreads), 0,
                       stream, (const uint8_t*)a.q, (const uint8_t*)a.k, (const uint8_t*)a.v, (const uint8_t*)a.d_o,
                       a.q_scale, a.k_scale, a.v_scale, a.do_scale, (const float*)a.ws, (__bf16*)a.d_q, a.Nq, a.Nk,
                       n_qt, a.scale_log2, a.scale, a.bottom_right);
    e = hipGetLastError();
  }
  return e;
}

}  // namespace

hipError_t launch_bwd_mxfp8(const BwdArgs& a, hipStream_t stream) {
  if (a.d != kD) return hipErrorInvalidValue;
  return a.causal ? launch_bwd_mx_c<true>(a, stream) : launch_bwd_mx_c<false>(a, stream);
}

hipError_t launch_mx_quantize(const void* x, uint8_t* q, uint8_t* scale, long long rows, hipStream_t stream) {
  if (rows <= 0) return hipSuccess;
  hipLaunchKernelGGL(mx_quantize_kernel, dim3((unsigned)(rows / 32)), dim3(256), 0, stream, (const __bf16*)x, q, scale);
  return hipGetLastError();
}

}  // namespace attn
