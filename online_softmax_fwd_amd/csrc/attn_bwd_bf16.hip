// attn_bwd_bf16.hip -- bf16 attention backward for gfx950 (MI355X).
//
// Gradients of O = softmax(S) V, S = scale * Q K^T, given dO and the forward
// pass's O and LSE. The forward kernel returns the per-row log-sum-exp so that
// P can be rebuilt as exp(S - LSE) without a second softmax ("Lecture 2 --
// Online Softmax and Numerical Correctness", section "Use it in the real
// stack"), and the backward pass is five products, S, dP = dO V^T, dV = P^T dO,
// dK = dS^T Q and dQ = dS K, with dK and dV accumulated over all queries
// ("PyTorch FlashAttention-4 adds MXFP8 block-scaled forward and backward for
// Blackwell", section "TMEM allocation and scale factor placement"). Here:
//
//   bwd_prep_kernel   D_i = sum_c dO_ic O_ic (float32) and LSE_i * log2(e),
//                     interleaved per row in the workspace (+inf for a row
//                     that saw no key, so that its P is 0).
//   bwd_dkdv_kernel   one workgroup per 32*NW keys of a head; each wave owns
//                     32 keys, holds their K and V rows as MFMA operands and
//                     dK^T, dV^T accumulators, and streams the queries in
//                     64-row tiles (Q, dO and the prep values DMA'd to LDS,
//                     double-buffered). Per 32 queries:
//                       S    = Q K^T        A = Q rows (LDS, permuted), B = K
//                       dP   = dO V^T       A = dO rows (LDS, permuted), B = V
//                       P    = 2^(S*c - LSE*log2 e),  dS = P * (dP - D)
//                       dV^T += dO^T P      A = dO^T (LDS transpose read), B = P
//                       dK^T += Q^T dS      A = Q^T (LDS transpose read), B = dS
//                     The permuted rows put queries 8h..8h+7 and 16+8h..+7 in
//                     lane half h, the B-operand layout of the two updates, so
//                     P and dS go from accumulators to operands in registers.
//   bwd_dq_kernel     one workgroup per 32*NW queries; streams K and V in
//                     64-key tiles like the forward kernel:
//                       S^T  = K Q^T,  dP^T = V dO^T,  dS^T = P^T * (dP^T - D)
//                       dQ^T += K^T dS^T    A = K^T (LDS transpose read)
//   bwd_dq_pp_kernel  the same products on the forward's ping-pong schedule
//                     (d = 128, 256 queries per workgroup, two groups of 4
//                     waves alternating MFMA and vector phases); it serves
//                     launches with at least one workgroup per CU, the
//                     streaming kernel the smaller ones and d = 64.
//
// dQ has its own kernel (recomputing S and dP: seven products instead of
// five) rather than atomic float adds from every key block into a float32
// buffer: no atomics, no extra buffer of Nq x d floats, and a result that is
// the same bit for bit on every run.
//
// The Q/dO tiles (dK/dV kernel) and the K tile (dQ kernel) are read both as
// permuted rows and through ds_read_b64_tr_b16, so their 16-byte chunks use a
// swizzle that spreads both access patterns evenly over the 64 LDS banks.
#include "attn_bf16_common.h"
#include "attn_device.h"
#include "attn_internal.h"

namespace attn {
namespace {

constexpr float kLog2e = 1.4426950408889634f;

template <int D>
struct BwdCfg {
  static constexpr int RB = 2 * D;      // bytes per row
  static constexpr int CH = D / 8;      // 16-byte chunks per row
  static constexpr int NW = 4;          // waves per workgroup
  static constexpr int THREADS = 64 * NW;
  static constexpr int BM = 64;         // query rows per tile (dK/dV kernel)
  static constexpr int BN = 64;         // keys per tile (dQ kernel)
  static constexpr int TILE = 64 * RB;  // bytes per tile (both kernels)
  static constexpr int LOADS = 64 * CH / 64 / NW;  // wave-loads per wave per tensor per tile
  static constexpr int WAVES_PER_SIMD = D == 64 ? 3 : 2;
  static_assert(LOADS * 64 * NW == 64 * CH, "tile split");
};

// Chunk swizzle of the tiles read both ways (position c ^ f(r)): a map of
// row bits 0, 1 and 3 chosen (by exhaustive search over such maps) so that a
// permuted-row read (16 rows, one chunk per 16 lanes) and a transpose read (8
// rows x 4 chunks) each touch every one of the 64 banks the minimum number of
// times. It ignores row bits 2, 4 and 5, so one per-lane offset serves both
// halves (rows r and r+4) of a transpose read and every 16-row step of a tile.
template <int D>
__device__ __forceinline__ int swz_dual(int r) {
  if (D == 128) return ((r & 3) << 1) | (r & 8);
  return (r & 2) | ((r & 8) >> 1);
}

// f(integral_constant<int, I>) for I = B .. E-1, in order
template <int B, int E, class F>
__device__ __forceinline__ void bwd_static_for(F&& f) {
  if constexpr (B < E) {
    f(std::integral_constant<int, B>{});
    bwd_static_for<B + 1, E>(f);
  }
}

// Per-lane LDS offsets (within a 32-row block of a tile) of the two read
// patterns, and the global offsets of this lane's DMA chunks.
template <int D>
struct TileOffsets {
  uint32_t row[D / 16];   // permuted-row read, one per 16-wide d step
  uint32_t tr[D / 32];    // transpose read, one per 32-wide d block
  uint32_t ld[BwdCfg<D>::LOADS];
  __device__ __forceinline__ void init(int lane, int wave, int rsb) {
    using C = BwdCfg<D>;
    const int hh = lane >> 5, l32 = lane & 31;
    const int pr = key_of_row(l32);
#pragma unroll
    for (int s = 0; s < D / 16; ++s) row[s] = pr * C::RB + 16 * ((2 * s + hh) ^ swz_dual<D>(pr));
    const int L = lane & 15, gidx = (lane >> 4) & 1;
    const int vr = 8 * hh + (L >> 2);
#pragma unroll
    for (int db = 0; db < D / 32; ++db) {
      const int cch = 4 * db + 2 * gidx + ((L & 3) >> 1);
      tr[db] = vr * C::RB + 16 * (cch ^ swz_dual<D>(vr)) + 8 * (L & 1);
    }
#pragma unroll
    for (int i = 0; i < C::LOADS; ++i) {
      const int pos = 64 * (wave + C::NW * i) + lane;
      const int r = pos / C::CH, p = pos % C::CH;
      ld[i] = r * rsb + 16 * (p ^ swz_dual<D>(r));
    }
  }
};

// A operand (32 x 16 of bf16) for rows 32*blk.. of an LDS tile through the
// transpose read: element (m, k) = tile[16*cc + k][32*db + m].
template <int D>
__device__ __forceinline__ bf16x8 tr_operand(const char* tile, uint32_t tr_off, int row0) {
  constexpr int RB = BwdCfg<D>::RB;
  const char* p = tile + tr_off + row0 * RB;
  const shortx4 lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_shortx4*)(p));
  const shortx4 hi = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_shortx4*)(p + 4 * RB));
  return __builtin_bit_cast(bf16x8, u32x4{__builtin_bit_cast(u32x2, lo)[0], __builtin_bit_cast(u32x2, lo)[1],
                                          __builtin_bit_cast(u32x2, hi)[0], __builtin_bit_cast(u32x2, hi)[1]});
}

// One DMA round of a 64-row tile of one tensor (every wave issues LOADS).
template <int D>
__device__ __forceinline__ void dma_tile(const u32x4& rs, char* dst, const TileOffsets<D>& to, int wave,
                                         uint32_t tile_off) {
  using C = BwdCfg<D>;
#pragma unroll
  for (int i = 0; i < C::LOADS; ++i) dma16(rs, dst + 1024 * (wave + C::NW * i), to.ld[i] + tile_off);
}

// Registers of one row (lane l32 of the wave's 32 rows) as the B operand of
// a 32x32x16 MFMA: lane half h holds elements 16 s + 8 h .. +8 for s < D/16.
template <int D>
__device__ __forceinline__ void load_row_operand(bf16x8 (&f)[D / 16], const __bf16* row, bool ok, int hh) {
#pragma unroll
  for (int s = 0; s < D / 16; ++s) {
    const u32x4 w = ok ? *(const u32x4*)(row + 16 * s + 8 * hh) : u32x4{0u, 0u, 0u, 0u};
    f[s] = __builtin_bit_cast(bf16x8, w);
  }
}

// Store the accumulators X^T (m = feature, n = row l32) of one row, times f,
// as bf16: element e of block db is feature 32 db + 8 (e/4) + 4 h + e%4.
template <int D>
__device__ __forceinline__ void store_row(__bf16* row, const floatx16 (&acc)[D / 32], float f, int hh) {
#pragma unroll
  for (int db = 0; db < D / 32; ++db)
#pragma unroll
    for (int g = 0; g < 4; ++g) {
      bf16x4 w;
#pragma unroll
      for (int r = 0; r < 4; ++r) w[r] = (__bf16)(acc[db][4 * g + r] * f);
      *(bf16x4*)(row + 32 * db + 8 * g + 4 * hh) = w;
    }
}

// ---------------------------------------------------------------------------
// Pre-pass: ws[2i] = LSE_i * log2(e) (+inf where LSE_i = -inf), ws[2i+1] = D_i.
// D/8 lanes per row, 16 bytes of O and dO each, reduced across the lanes.
// ---------------------------------------------------------------------------
template <int D>
__global__ __attribute__((amdgpu_flat_work_group_size(256, 256)))
void bwd_prep_kernel(const __bf16* __restrict__ O, const __bf16* __restrict__ dO, const float* __restrict__ LSE,
                     float* __restrict__ ws, long long rows) {
  constexpr int LPR = D / 8, RPB = 256 / LPR;
  const long long r = (long long)blockIdx.x * RPB + threadIdx.x / LPR;
  const int part = threadIdx.x % LPR;
  float acc = 0.0f;
  if (r < rows) {
    const bf16x8 o = __builtin_bit_cast(bf16x8, *(const u32x4*)(O + r * D + 8 * part));
    const bf16x8 g = __builtin_bit_cast(bf16x8, *(const u32x4*)(dO + r * D + 8 * part));
#pragma unroll
    for (int e = 0; e < 8; ++e) acc = __builtin_fmaf((float)o[e], (float)g[e], acc);
  }
#pragma unroll
  for (int w = LPR / 2; w >= 1; w >>= 1) acc += __shfl_xor(acc, w);
  if (r < rows && part == 0) {
    const float l = LSE[r];
    ws[2 * r] = l == kNegInf ? -kNegInf : l * kLog2e;
    ws[2 * r + 1] = acc;
  }
}

// ---------------------------------------------------------------------------
// dK, dV: workgroup = 4 waves x 32 keys of one head; query tiles of 64 rows.
// ---------------------------------------------------------------------------
template <int D, bool CAUSAL>
__global__ __attribute__((amdgpu_flat_work_group_size(BwdCfg<D>::THREADS, BwdCfg<D>::THREADS),
                          amdgpu_waves_per_eu(BwdCfg<D>::WAVES_PER_SIMD, BwdCfg<D>::WAVES_PER_SIMD)))
void bwd_dkdv_kernel(const __bf16* __restrict__ Q, const __bf16* __restrict__ K, const __bf16* __restrict__ V,
                     const __bf16* __restrict__ dO, const float* __restrict__ ws, __bf16* __restrict__ dK,
                     __bf16* __restrict__ dV, int Nq, int Nk, int n_kt, float c, float scale, int bottom_right) {
  using C = BwdCfg<D>;
  constexpr int RB = C::RB;
  __shared__ __attribute__((aligned(1024))) char q0s[C::TILE];
  __shared__ __attribute__((aligned(1024))) char d0s[C::TILE];
  __shared__ __attribute__((aligned(1024))) char q1s[C::TILE];
  __shared__ __attribute__((aligned(1024))) char d1s[C::TILE];
  __shared__ __attribute__((aligned(16))) float w0s[2 * C::BM];  // (LSE*log2 e, D) of the tile's rows
  __shared__ __attribute__((aligned(16))) float w1s[2 * C::BM];

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int hh = lane >> 5, l32 = lane & 31;

  // key tiles of a head need less work the later they start (causal): hand
  // them out longest first, per XCD, like the forward kernel's query tiles
  int bh, kt;
  if (CAUSAL) {
    causal_tile_of(blockIdx.x, gridDim.x, n_kt, bh, kt);
    kt = n_kt - 1 - kt;
  } else {
    const int logical = xcd_logical_id(blockIdx.x, gridDim.x);
    bh = logical / n_kt;
    kt = logical - bh * n_kt;
  }
  const int k0 = kt * 32 * C::NW;
  const int kw0 = k0 + 32 * wave;
  const int key = kw0 + l32;
  const size_t qbase = (size_t)bh * Nq * D, kbase = (size_t)bh * Nk * D;
  const int diag = bottom_right ? Nk - Nq : 0;  // key j is hidden from query i when j > i + diag

  TileOffsets<D> to;
  to.init(lane, wave, RB);
  const u32x4 rq = raw_buffer_rsrc(Q + qbase, (uint32_t)(Nq * RB));
  const u32x4 rdo = raw_buffer_rsrc(dO + qbase, (uint32_t)(Nq * RB));
  const u32x4 rw = raw_buffer_rsrc(ws + (size_t)bh * Nq * 2, (uint32_t)(Nq * 8));

  bf16x8 kf[D / 16], vf[D / 16];
  load_row_operand<D>(kf, K + kbase + (size_t)(key < Nk ? key : 0) * D, key < Nk, hh);
  load_row_operand<D>(vf, V + kbase + (size_t)(key < Nk ? key : 0) * D, key < Nk, hh);

  floatx16 dk[D / 32], dv[D / 32];
#pragma unroll
  for (int i = 0; i < D / 32; ++i) dk[i] = dv[i] = floatx16{};

  // query tiles that can see a key of this workgroup
  const int qlo = CAUSAL ? max(0, k0 - diag) : 0;
  const int t0 = qlo / C::BM;
  const int nt = (Nq + C::BM - 1) / C::BM;

  auto load = [&](int t, char* qd, char* dd, float* wd) __attribute__((always_inline)) {
    const uint32_t off = (uint32_t)t * C::TILE;
    dma_tile<D>(rq, qd, to, wave, off);
    dma_tile<D>(rdo, dd, to, wave, off);
    if (wave == 0 && lane < 32) dma16(rw, (const char*)wd, (uint32_t)t * (8 * C::BM) + 16 * lane);
  };

  auto compute = [&](int t, const char* qs, const char* dos, const float* wsd) __attribute__((always_inline)) {
#pragma unroll 1
    for (int sb = 0; sb < 2; ++sb) {
      const int q0 = t * C::BM + 32 * sb;
      if (CAUSAL && q0 + 31 + diag < kw0) continue;  // wave-uniform: no query here sees the wave's keys
      floatx16 s = {}, dp = {};
#pragma unroll
      for (int st = 0; st < D / 16; ++st) {
        const bf16x8 a = *(const bf16x8*)(qs + sb * 32 * RB + to.row[st]);
        s = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, kf[st], s, 0, 0, 0);
      }
#pragma unroll
      for (int st = 0; st < D / 16; ++st) {
        const bf16x8 a = *(const bf16x8*)(dos + sb * 32 * RB + to.row[st]);
        dp = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, vf[st], dp, 0, 0, 0);
      }
      __builtin_amdgcn_sched_barrier(0);  // keep the update's operand reads below the softmax (registers)
      // element e holds query q0 + 16 (e/8) + 8 h + e%8: two runs of 8 rows,
      // each with its 8 (LSE*log2 e, D) pairs read just before use
      if (CAUSAL && q0 + diag < kw0 + 31) {  // masked pairs get S = -inf (one wave-uniform branch)
#pragma unroll
        for (int e = 0; e < 16; ++e)
          if (key > q0 + 16 * (e >> 3) + 8 * hh + (e & 7) + diag) s[e] = kNegInf;
      }
      bf16x8 pb[2], db[2];
#pragma unroll
      for (int run = 0; run < 2; ++run) {
        const float4* wp = (const float4*)(wsd + 2 * (32 * sb + 16 * run + 8 * hh));
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          const float4 w = wp[i];  // rows 2i and 2i+1 of the run
#pragma unroll
          for (int j = 0; j < 2; ++j) {
            const int e = 8 * run + 2 * i + j;
            const float p = exp2_hw(__builtin_fmaf(s[e], c, -w[2 * j]));
            pb[run][2 * i + j] = (__bf16)p;
            db[run][2 * i + j] = (__bf16)(p * (dp[e] - w[2 * j + 1]));
          }
        }
      }
      __builtin_amdgcn_sched_barrier(0);
#pragma unroll
      for (int d = 0; d < D / 32; ++d)
#pragma unroll
        for (int cc = 0; cc < 2; ++cc) {
          const bf16x8 a = tr_operand<D>(dos, to.tr[d], 32 * sb + 16 * cc);
          dv[d] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, pb[cc], dv[d], 0, 0, 0);
          const bf16x8 b = tr_operand<D>(qs, to.tr[d], 32 * sb + 16 * cc);
          dk[d] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(b, db[cc], dk[d], 0, 0, 0);
        }
    }
  };

  // double-buffered: tile t+1 is in flight while tile t is computed; one loop
  // body with the buffer chosen per tile (two inlined copies, one per buffer,
  // spill the K and V operands)
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

  if (key < Nk) {
    store_row<D>(dK + kbase + (size_t)key * D, dk, scale, hh);
    store_row<D>(dV + kbase + (size_t)key * D, dv, 1.0f, hh);
  }
}

// ---------------------------------------------------------------------------
// dQ: workgroup = 4 waves x 32 queries of one head; key tiles of 64 keys.
// ---------------------------------------------------------------------------
template <int D, bool CAUSAL>
__global__ __attribute__((amdgpu_flat_work_group_size(BwdCfg<D>::THREADS, BwdCfg<D>::THREADS),
                          amdgpu_waves_per_eu(BwdCfg<D>::WAVES_PER_SIMD, BwdCfg<D>::WAVES_PER_SIMD)))
void bwd_dq_kernel(const __bf16* __restrict__ Q, const __bf16* __restrict__ K, const __bf16* __restrict__ V,
                   const __bf16* __restrict__ dO, const float* __restrict__ ws, __bf16* __restrict__ dQ, int Nq,
                   int Nk, int n_qt, float c, float scale, int bottom_right) {
  using C = BwdCfg<D>;
  constexpr int RB = C::RB;
  __shared__ __attribute__((aligned(1024))) char k0s[C::TILE];
  __shared__ __attribute__((aligned(1024))) char v0s[C::TILE];
  __shared__ __attribute__((aligned(1024))) char k1s[C::TILE];
  __shared__ __attribute__((aligned(1024))) char v1s[C::TILE];

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
  const int q0 = qt * 32 * C::NW;
  const int qw0 = q0 + 32 * wave;
  const int qi = qw0 + l32;
  const bool row_ok = qi < Nq;
  const size_t qbase = (size_t)bh * Nq * D, kbase = (size_t)bh * Nk * D;
  const int diag = bottom_right ? Nk - Nq : 0;

  TileOffsets<D> to;
  to.init(lane, wave, RB);
  const u32x4 rk = raw_buffer_rsrc(K + kbase, (uint32_t)(Nk * RB));
  const u32x4 rv = raw_buffer_rsrc(V + kbase, (uint32_t)(Nk * RB));

  bf16x8 qf[D / 16], gf[D / 16];
  load_row_operand<D>(qf, Q + qbase + (size_t)(row_ok ? qi : 0) * D, row_ok, hh);
  load_row_operand<D>(gf, dO + qbase + (size_t)(row_ok ? qi : 0) * D, row_ok, hh);
  float l2 = -kNegInf, dd = 0.0f;  // rows past Nq: P = 0
  if (row_ok) {
    const float2 w = *(const float2*)(ws + ((size_t)bh * Nq + qi) * 2);
    l2 = w[0];
    dd = w[1];
  }

  floatx16 dq[D / 32];
#pragma unroll
  for (int i = 0; i < D / 32; ++i) dq[i] = floatx16{};

  const int kend = CAUSAL ? min(Nk, q0 + 32 * C::NW + diag) : Nk;
  const int T = kend > 0 ? (kend + C::BN - 1) / C::BN : 0;

  auto load = [&](int t, char* kd, char* vd) __attribute__((always_inline)) {
    const uint32_t off = (uint32_t)t * C::TILE;
    dma_tile<D>(rk, kd, to, wave, off);
    dma_tile<D>(rv, vd, to, wave, off);
  };

  auto compute = [&](int t, const char* ks, const char* vs) __attribute__((always_inline)) {
#pragma unroll 1
    for (int kb = 0; kb < 2; ++kb) {
      const int kk0 = t * C::BN + 32 * kb;
      if (CAUSAL && kk0 > qw0 + 31 + diag) continue;  // wave-uniform: every key here is hidden
      floatx16 s = {}, dp = {};
#pragma unroll
      for (int st = 0; st < D / 16; ++st) {
        const bf16x8 a = *(const bf16x8*)(ks + kb * 32 * RB + to.row[st]);
        s = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, qf[st], s, 0, 0, 0);
      }
#pragma unroll
      for (int st = 0; st < D / 16; ++st) {
        const bf16x8 a = *(const bf16x8*)(vs + kb * 32 * RB + to.row[st]);
        dp = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, gf[st], dp, 0, 0, 0);
      }
      __builtin_amdgcn_sched_barrier(0);
      // masked keys get S = -inf, in a block of its own behind one
      // wave-uniform branch (per element, the compiler turns the test into
      // selects that run on every block)
      if ((CAUSAL && kk0 + 31 > qw0 + diag) || (kk0 + 32 > Nk)) {
#pragma unroll
        for (int e = 0; e < 16; ++e) {
          const int kj = kk0 + 16 * (e >> 3) + 8 * hh + (e & 7);
          if (kj >= Nk || (CAUSAL && kj > qi + diag)) s[e] = kNegInf;
        }
      }
      bf16x8 db[2];
#pragma unroll
      for (int e = 0; e < 16; ++e) {
        const float p = exp2_hw(__builtin_fmaf(s[e], c, -l2));
        db[e >> 3][e & 7] = (__bf16)(p * (dp[e] - dd));
      }
      __builtin_amdgcn_sched_barrier(0);
#pragma unroll
      for (int d = 0; d < D / 32; ++d)
#pragma unroll
        for (int cc = 0; cc < 2; ++cc) {
          const bf16x8 a = tr_operand<D>(ks, to.tr[d], 32 * kb + 16 * cc);
          dq[d] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, db[cc], dq[d], 0, 0, 0);
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

  if (row_ok) store_row<D>(dQ + qbase + (size_t)qi * D, dq, scale, hh);
}

// ---------------------------------------------------------------------------
// dQ on the forward's ping-pong schedule (d = 128): 8 waves x 32 query rows,
// two groups of 4 (waves i and i+4 share a SIMD), 64-key tiles. Per tile j a
// wave runs an MFMA phase -- dQ^T += K_{j-1}^T dS_{j-1}^T (16 MFMAs, K^T
// through the transpose read), then S_j^T = K_j Q^T and dP_j^T = V_j dO^T
// interleaved (32 MFMAs) -- and a VALU phase: mask, P = 2^(S c - LSE log2 e),
// dS = P (dP - D), dS to bf16. Group 1 runs one phase behind group 0 with a
// workgroup barrier between phases, so on every SIMD one wave feeds the
// matrix core while the other runs the vector work. K is read in two
// consecutive MFMA phases (S, then dQ), so K and V sit in rings of three
// tiles; DMA batch b (K_{b+1}, V_{b+1}) is issued at half-phase 2b into the
// slots of tile b-2, which every wave finished reading in MFMA phase b-1, and
// waited for at the end of half-phase 2b+1, just before MFMA phase b+1.
// ---------------------------------------------------------------------------
template <int D, bool CAUSAL>
__global__ __attribute__((amdgpu_flat_work_group_size(512, 512), amdgpu_waves_per_eu(2, 2)))
void bwd_dq_pp_kernel(const __bf16* __restrict__ Q, const __bf16* __restrict__ K, const __bf16* __restrict__ V,
                      const __bf16* __restrict__ dO, const float* __restrict__ ws, __bf16* __restrict__ dQ, int Nq,
                      int Nk, int n_qt, float c, float scale, int bottom_right) {
  static_assert(D == 128, "the ping-pong dQ kernel is written for d = 128");
  constexpr int RB = 2 * D, CH = D / 8, NW = 8, BN = 64, KB = BN / 32, TILE = BN * RB, S = 3;
  constexpr int LOADS = BN * CH / 64 / NW;  // wave-loads per wave per tensor per tile
  constexpr int NDB = D / 32, NST = D / 16;
  constexpr int NDQ = NDB * KB * 2, NSP = 2 * KB * NST, RING = 6;
  __shared__ __attribute__((aligned(1024))) char kring[S * TILE];
  __shared__ __attribute__((aligned(1024))) char vring[S * TILE];

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int group = wave >> 2;
  const int hh = lane >> 5, l32 = lane & 31;

  int bh, qt;
  if (CAUSAL) {
    causal_tile_of(blockIdx.x, gridDim.x, n_qt, bh, qt);
  } else {
    const int logical = xcd_logical_id(blockIdx.x, gridDim.x);
    bh = logical / n_qt;
    qt = logical - bh * n_qt;
  }
  const int q0 = qt * 32 * NW;
  const int qw0 = q0 + 32 * wave;
  const int qi = qw0 + l32;
  const bool row_ok = qi < Nq;
  const size_t qbase = (size_t)bh * Nq * D, kbase = (size_t)bh * Nk * D;
  const int diag = bottom_right ? Nk - Nq : 0;

  // Per-lane LDS offsets with the ring bases in the register part (opaque to
  // the compiler, so slot + in-tile offsets fit the 16-bit immediate): K and V
  // rows for S and dP (permuted rows, one per 16-wide d step), K^T for dQ.
  uint32_t kr = lds_address(kring), vbase = lds_address(vring);
  asm volatile("" : "+s"(kr));
  asm volatile("" : "+s"(vbase));
  uint32_t rowk[NST], rowv[NST], trk[NDB], ld[LOADS];
  {
    const int pr = key_of_row(l32);
#pragma unroll
    for (int st = 0; st < NST; ++st) {
      const uint32_t o = pr * RB + 16 * ((2 * st + hh) ^ swz_dual<D>(pr));
      rowk[st] = kr + o;
      rowv[st] = vbase + o;
    }
    const int L = lane & 15, gidx = (lane >> 4) & 1;
    const int vr = 8 * hh + (L >> 2);
#pragma unroll
    for (int db = 0; db < NDB; ++db) {
      const int cch = 4 * db + 2 * gidx + ((L & 3) >> 1);
      trk[db] = kr + vr * RB + 16 * (cch ^ swz_dual<D>(vr)) + 8 * (L & 1);
    }
#pragma unroll
    for (int i = 0; i < LOADS; ++i) {
      const int pos = 64 * (wave + NW * i) + lane;
      const int r = pos / CH, p = pos % CH;
      ld[i] = r * RB + 16 * (p ^ swz_dual<D>(r));
    }
  }
  const u32x4 rk = raw_buffer_rsrc(K + kbase, (uint32_t)(Nk * RB));
  const u32x4 rv = raw_buffer_rsrc(V + kbase, (uint32_t)(Nk * RB));

  bf16x8 qf[NST], gf[NST];
  load_row_operand<D>(qf, Q + qbase + (size_t)(row_ok ? qi : 0) * D, row_ok, hh);
  load_row_operand<D>(gf, dO + qbase + (size_t)(row_ok ? qi : 0) * D, row_ok, hh);
  float l2 = -kNegInf, dd = 0.0f;  // rows past Nq: P = 0
  if (row_ok) {
    const float2 w = *(const float2*)(ws + ((size_t)bh * Nq + qi) * 2);
    l2 = w[0];
    dd = w[1];
  }

  floatx16 dq[NDB];
#pragma unroll
  for (int i = 0; i < NDB; ++i) dq[i] = floatx16{};
  const int kend = CAUSAL ? min(Nk, q0 + 32 * NW + diag) : Nk;
  const int T = kend > 0 ? (kend + BN - 1) / BN : 0;
  if (T == 0) {  // no row of this workgroup sees a key: dQ = 0
    if (row_ok) store_row<D>(dQ + qbase + (size_t)qi * D, dq, scale, hh);
    return;
  }

  floatx16 s[KB], dp[KB];  // S^T and dP^T of the current tile
  bf16x8 db[KB][2];        // dS^T of the previous tile, the dQ MFMAs' B operand

  auto slot_off = [&](int i) __attribute__((always_inline)) -> uint32_t { return ((i % S + S) % S) * TILE; };
  // DMA batch b: this wave's share of K_{b+1} and V_{b+1}
  auto load_tiles = [&](int b) __attribute__((always_inline)) {
    if (b + 1 < T) {
      const uint32_t so = slot_off(b + 1), go = (uint32_t)(b + 1) * TILE;
#pragma unroll
      for (int i = 0; i < LOADS; ++i) {
        dma16(rk, kring + so + 1024 * (wave + NW * i), ld[i] + go);
        dma16(rv, vring + so + 1024 * (wave + NW * i), ld[i] + go);
      }
    }
  };

  // MFMA phase: dQ of tile j-1 (K^T from kprev), then S^T and dP^T of tile j
  // (K and V rows from kcur / vcur), operands read RING MFMAs ahead
  auto mfma_phase = [&](auto do_dq, auto do_sp, uint32_t kprev, uint32_t kcur, uint32_t vcur)
      __attribute__((always_inline)) {
    constexpr int N0 = decltype(do_dq)::value ? NDQ : 0;
    constexpr int N = N0 + (decltype(do_sp)::value ? NSP : 0);
    auto read = [&](int i) __attribute__((always_inline)) -> bf16x8 {
      if (i < N0) {
        const int d = i % NDB, k = i / NDB, kb = k >> 1, cc = k & 1;
        const uint32_t p = trk[d] + kprev + (32 * kb + 16 * cc) * RB;
        const shortx4 lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_shortx4*)(uintptr_t)(p));
        const shortx4 hi = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_shortx4*)(uintptr_t)(p + 4 * RB));
        return __builtin_bit_cast(bf16x8, u32x4{__builtin_bit_cast(u32x2, lo)[0], __builtin_bit_cast(u32x2, lo)[1],
                                                __builtin_bit_cast(u32x2, hi)[0], __builtin_bit_cast(u32x2, hi)[1]});
      }
      const int q = i - N0, dpk = q & 1, kb = (q >> 1) & 1, st = q >> 2;
      const uint32_t p = (dpk ? rowv[st] + vcur : rowk[st] + kcur) + kb * 32 * RB;
      return *(const lds_bf16x8*)(uintptr_t)(p);
    };
    bf16x8 ring[RING];
#pragma unroll
    for (int i = 0; i < RING && i < N; ++i) ring[i] = read(i);
    __builtin_amdgcn_sched_barrier(0);
#pragma unroll
    for (int i = 0; i < N; ++i) {
      const bf16x8 a = ring[i % RING];
      if (i + RING < N) ring[i % RING] = read(i + RING);
      if (i < N0) {
        const int d = i % NDB, k = i / NDB, kb = k >> 1, cc = k & 1;
        dq[d] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, db[kb][cc], dq[d], 0, 0, 0);
      } else {
        const int q = i - N0, dpk = q & 1, kb = (q >> 1) & 1, st = q >> 2;
        if (dpk)
          dp[kb] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, gf[st], st == 0 ? floatx16{} : dp[kb], 0, 0, 0);
        else
          s[kb] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, qf[st], st == 0 ? floatx16{} : s[kb], 0, 0, 0);
      }
      __builtin_amdgcn_sched_barrier(0);
    }
  };

  // VALU phase j: masked keys get S = -inf (one wave-uniform branch per 32-key
  // block), P, dS, and dS^T as bf16 for the next MFMA phase
  auto valu_phase = [&](int j) __attribute__((always_inline)) {
#pragma unroll
    for (int kb = 0; kb < KB; ++kb) {
      const int kk0 = j * BN + 32 * kb;
      if ((CAUSAL && kk0 + 31 > qw0 + diag) || (kk0 + 32 > Nk)) {
#pragma unroll
        for (int e = 0; e < 16; ++e) {
          const int kj = kk0 + 16 * (e >> 3) + 8 * hh + (e & 7);
          if (kj >= Nk || (CAUSAL && kj > qi + diag)) s[kb][e] = kNegInf;
        }
      }
#pragma unroll
      for (int e = 0; e < 16; ++e) {
        const float p = exp2_hw(__builtin_fmaf(s[kb][e], c, -l2));
        db[kb][e >> 3][e & 7] = (__bf16)(p * (dp[kb][e] - dd));
      }
    }
    // dS must be complete here, in the VALU phase (the compiler would sink it
    // into the next MFMA phase, past the barrier)
#pragma unroll
    for (int kb = 0; kb < KB; ++kb)
#pragma unroll
      for (int cc = 0; cc < 2; ++cc) asm volatile("" : "+v"(db[kb][cc]));
  };

  // One step j = [MFMA phase j] barrier [VALU phase j] barrier; group 1 runs
  // it one barrier later. Batch j goes out at half-phase 2j (group 0 at the
  // start of its MFMA phase j, group 1 at the start of its VALU phase j-1)
  // and every wave waits for its share at the end of half-phase 2j+1.
  auto step = [&](int j, auto do_dq, auto do_sp, auto slot) __attribute__((always_inline)) {
    constexpr int r = decltype(slot)::value;  // j % S
    if (group == 0) load_tiles(j);
    mfma_phase(do_dq, do_sp, slot_off(r - 1), slot_off(r), slot_off(r));
    if (group == 1) wait_own_loads();
    block_sync();
    if (group == 1) load_tiles(j + 1);
    if constexpr (decltype(do_sp)::value) valu_phase(j);
    if (group == 0) wait_own_loads();
    block_sync();
  };
  using Y = std::true_type;
  using N = std::false_type;

  // prologue: K_0 and V_0 by every wave; group 1's share of batch 0 (K_1, V_1)
  // goes out with group 0's, at half-phase 0
#pragma unroll
  for (int i = 0; i < LOADS; ++i) {
    dma16(rk, kring + 1024 * (wave + NW * i), ld[i]);
    dma16(rv, vring + 1024 * (wave + NW * i), ld[i]);
  }
  wait_own_loads();
  block_sync();
  if (group == 1) {
    load_tiles(0);
    block_sync();
  }
  step(0, N{}, Y{}, std::integral_constant<int, 0>{});
  int j = 1;
  for (; j + S - 1 < T; j += S)
    bwd_static_for<0, S>([&](auto R) __attribute__((always_inline)) {
      step(j + R, Y{}, Y{}, std::integral_constant<int, (decltype(R)::value + 1) % S>{});
    });
  // the remaining steps j .. T-1 (fewer than S; j = 1 mod S), then step T: dQ of the last tile
  bwd_static_for<0, S - 1>([&](auto R) __attribute__((always_inline)) {
    if (j + R < T) step(j + R, Y{}, Y{}, std::integral_constant<int, (decltype(R)::value + 1) % S>{});
  });
  bwd_static_for<0, S>([&](auto R) __attribute__((always_inline)) {
    if (T % S == R) step(T, Y{}, N{}, R);
  });
  if (group == 0) block_sync();

  if (row_ok) store_row<D>(dQ + qbase + (size_t)qi * D, dq, scale, hh);
}

template <int D, bool CAUSAL>
hipError_t launch_bwd_d(const BwdArgs& a, hipStream_t stream) {
  using C = BwdCfg<D>;
  const long long rows = (long long)a.B * a.H * a.Nq;
  constexpr int RPB = 256 / (D / 8);
  hipError_t e = hipSuccess;
  if (rows > 0) {  // no queries: dK = dV = 0 and dQ is empty
    hipLaunchKernelGGL((bwd_prep_kernel<D>), dim3((unsigned)((rows + RPB - 1) / RPB)), dim3(256), 0, stream,
                       (const __bf16*)a.o, (const __bf16*)a.d_o, a.lse, a.ws, rows);
    if ((e = hipGetLastError()) != hipSuccess) return e;
  }
  const int n_kt = (a.Nk + 32 * C::NW - 1) / (32 * C::NW);
  if (n_kt > 0) {
    hipLaunchKernelGGL((bwd_dkdv_kernel<D, CAUSAL>), dim3((unsigned)((long long)a.B * a.H * n_kt)),
                       dim3(C::THREADS), 0, stream, (const __bf16*)a.q, (const __bf16*)a.k, (const __bf16*)a.v,
                       (const __bf16*)a.d_o, (const float*)a.ws, (__bf16*)a.d_k, (__bf16*)a.d_v, a.Nq, a.Nk, n_kt,
                       a.scale_log2, a.scale, a.bottom_right);
    if ((e = hipGetLastError()) != hipSuccess) return e;
  }
  // The ping-pong dQ kernel takes 256 query rows per workgroup and fills a CU
  // with one. Below one workgroup per CU the streaming kernel, with twice as
  // many 128-row workgroups, finishes first (whole backward, B2 H8 N1024
  // causal: 125 against 117 TFLOP/s; B1 H4 N2048: 130 against 127).
  constexpr long long kDqPingPongMinTiles = 256;
  if constexpr (D == 128) {
    const int n_qt = (a.Nq + 255) / 256;
    if (n_qt > 0 && (long long)a.B * a.H * n_qt >= kDqPingPongMinTiles) {
      hipLaunchKernelGGL((bwd_dq_pp_kernel<D, CAUSAL>), dim3((unsigned)((long long)a.B * a.H * n_qt)), dim3(512), 0,
                         stream, (const __bf16*)a.q, (const __bf16*)a.k, (const __bf16*)a.v, (const __bf16*)a.d_o,
                         (const float*)a.ws, (__bf16*)a.d_q, a.Nq, a.Nk, n_qt, a.scale_log2, a.scale,
                         a.bottom_right);
      return hipGetLastError();
    }
  }
  const int n_qt = (a.Nq + 32 * C::NW - 1) / (32 * C::NW);
  if (n_qt > 0) {
    hipLaunchKernelGGL((bwd_dq_kernel<D, CAUSAL>), dim3((unsigned)((long long)a.B * a.H * n_qt)), dim3(C::THREADS),
                       0, stream, (const __bf16*)a.q, (const __bf16*)a.k, (const __bf16*)a.v, (const __bf16*)a.d_o,
                       (const float*)a.ws, (__bf16*)a.d_q, a.Nq, a.Nk, n_qt, a.scale_log2, a.scale,
                       a.bottom_right);
    e = hipGetLastError();
  }
  return e;
}

}  // namespace

hipError_t launch_bwd_bf16(const BwdArgs& a, hipStream_t stream) {
  if (a.d == 128) return a.causal ? launch_bwd_d<128, true>(a, stream) : launch_bwd_d<128, false>(a, stream);
  if (a.d == 64) return a.causal ? launch_bwd_d<64, true>(a, stream) : launch_bwd_d<64, false>(a, stream);
  return hipErrorInvalidValue;
}

}  // namespace attn
