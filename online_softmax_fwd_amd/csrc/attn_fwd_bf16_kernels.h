// attn_fwd_bf16_kernels.h -- pieces of the bf16 forward shared by its
// translation units: tile configuration, LDS swizzles, the lane row sum, and
// the streaming kernel, which serves both whole-row launches and launches
// that split each row's keys into chunks handled by separate workgroups.
#pragma once
#include <type_traits>

#include "attn_bf16_common.h"
#include "attn_device.h"
#include "attn_internal.h"

namespace attn {
namespace {

template <int D_, int BN_, int NW_>
struct Cfg {
  static constexpr int D = D_, BN = BN_, NW = NW_;
  static constexpr int THREADS = 64 * NW;
  static constexpr int BM = 32 * NW;          // query rows per workgroup
  static constexpr int RB = 2 * D;            // bytes per K/V row
  static constexpr int CH = D / 8;            // 16-byte chunks per row
  static constexpr int TILE = BN * RB;        // bytes per K or V tile
  static constexpr int KB = BN / 32;          // 32-key MFMA blocks per tile
  static constexpr int LOADS = BN * CH / 64 / NW;  // wave-loads per wave per tensor per tile
  static_assert(LOADS >= 1 && LOADS * 64 * NW == BN * CH, "tile does not split evenly over the waves");
  static_assert(D == 64 || D == 128 || D == 192 || D == 256, "head dim");
};

// Swizzles (16-byte chunk position of logical chunk c in row r is c ^ f(r)).
// K reads touch one chunk of 16 rows per 16-lane group: f_K makes those 16
// rows land on 16 different bank groups. V transpose reads touch 4 chunks of
// 8 rows per instruction: f_V spreads them so each bank is hit exactly twice
// (512 bytes, the minimum of two passes). Rows of 256 or 512 bytes start on
// bank 0 (d = 128, 256); rows of 128 or 384 bytes alternate between bank 0 and
// bank 32 (d = 64, 192), so there odd and even rows share XOR values. At
// d = 192 (24 chunks) every XOR stays below 8, which keeps a chunk in its row.
template <int D>
__device__ __forceinline__ int swz_k(int r) { return (D == 128 || D == 256) ? (r & 15) : ((r >> 1) & 7); }
template <int D>
__device__ __forceinline__ int swz_v(int r) { return (D == 128 || D == 256) ? 4 * (r & 3) : 4 * ((r >> 1) & 1); }

// Sum of a lane's scores as a balanced tree instead of a serial chain, so the
// softmax stage is not latency-bound (the max tree is tree_max).
template <int KB>
__device__ __forceinline__ float tree_sum(const floatx16 (&x)[KB]) {
  float t[8 * KB];
#pragma unroll
  for (int kb = 0; kb < KB; ++kb)
#pragma unroll
    for (int e = 0; e < 8; ++e) t[8 * kb + e] = x[kb][e] + x[kb][e + 8];
#pragma unroll
  for (int w = 4 * KB; w >= 1; w >>= 1)
#pragma unroll
    for (int e = 0; e < w; ++e) t[e] = t[e] + t[e + w];
  return t[0];
}

// f(integral_constant<int, I>) for I = B .. E-1, in order
template <int B, int E, class F>
__device__ __forceinline__ void static_for(F&& f) {
  if constexpr (B < E) {
    f(std::integral_constant<int, B>{});
    static_for<B + 1, E>(f);
  }
}

// ---------------------------------------------------------------------------
// Streaming kernel: d = 64 and 256, and small causal d = 128 and 192 launches. Each wave owns 32 query rows
// and runs the S^T MFMAs, the softmax and the PV MFMAs of a key tile in
// order, with no cross-wave phases; K and V tiles stream through two LDS
// buffers shared by the workgroup. Several workgroups share a CU, so each
// SIMD interleaves three or four independent streams. Measured against the
// ping-pong schedule of fwd_bf16_kernel: at d = 64, where the softmax weighs
// twice as much per MFMA, 968 vs 883 TFLOP/s non-causal and 898 vs 781
// causal (B=2, H=32, N=8192); at d = 128 the ping-pong kernel is faster
// (1137 vs about 1050 non-causal, 1017 vs 987 causal at B=4, H=16, N=4096).
// The per-tile steps and their sources are those of fwd_bf16_kernel.
// ---------------------------------------------------------------------------
// d = 64: 8 waves x 64-key tiles, two workgroups per CU (~120 VGPRs).
// d = 128: 4 waves x 32-key tiles, three workgroups per CU (~157 VGPRs, 32 KB
// of LDS each); used for causal launches too small to give every CU a
// 256-row workgroup of the ping-pong kernel.
// d = 192, 256: 4 waves x 32-key tiles, two workgroups per CU (the O
// accumulators alone take d/2 VGPRs, Q another d/4; 48 / 64 KB of LDS each);
// d = 192 only for small causal launches.
template <int D_, int BN_, int NW_, int WPS_>
struct StreamCfgT : Cfg<D_, BN_, NW_> {
  static constexpr int WAVES_PER_SIMD = WPS_;  // occupancy the register budget is set for
  static constexpr int STAGES = 2;             // K/V tiles of each in the LDS ring
};
template <int D>
using StreamCfg = StreamCfgT<D, D == 64 ? 64 : 32, D == 64 ? 8 : 4, D == 64 ? 4 : D == 128 ? 3 : 2>;

// Key chunks of a split launch ("Lecture 2 -- Online Softmax and Numerical
// Correctness", section "Combining two blocks exactly": the softmax state of
// two key ranges merges exactly). Query tile qt of a head needs the keys
// below kend(qt) (all Nk, or up to its causal diagonal); they are cut into
// n_chunks(qt) chunks of `chunk` keys (at least one, so that a tile with no
// key still writes its rows). A head's units are its (tile, chunk) pairs in
// tile order; unit u of head bh owns workspace slot bh * units + u.
struct SplitPlan {
  int chunk;   // keys per chunk, a multiple of the key tile
  int units;   // (tile, chunk) units per head
  int BM;      // query rows per tile
  int Nq, Nk, diag;
  bool causal;
  __host__ __device__ int kend(int qt) const {
    const int k = (qt + 1) * BM + diag;
    return causal ? (k < Nk ? k : Nk) : Nk;
  }
  __host__ __device__ int n_chunks(int qt) const {
    const int k = kend(qt);
    return k > 0 ? (k + chunk - 1) / chunk : 1;
  }
  // tile and chunk of unit u, and the head's first unit of that tile
  __host__ __device__ void unit(int u, int& qt, int& ch, int& u0) const {
    const int n_qt = (Nq + BM - 1) / BM;
    qt = 0;
    u0 = 0;
    for (;;) {
      const int n = n_chunks(qt);
      if (u < u0 + n || qt == n_qt - 1) break;
      u0 += n;
      ++qt;
    }
    ch = u - u0;
  }
};

// SPLIT: each workgroup runs one key chunk of one query tile (a unit of the
// SplitPlan). A tile cut into one chunk writes O and LSE as usual; otherwise
// the workgroup writes its chunk's normalised float32 O and its LSE in log2
// units (m * c + log2 l, -inf for a row that saw no key of the chunk) to slot
// bh * units + u of the workspace, and the merge kernel combines the chunks
// of a row. A slot holds BM * D floats of O in the accumulators' own lane
// order, so that each store of a wave is one contiguous 1 KiB block: float4
// number ((wave * D/8 + 4 * db + g) * 64 + lane) holds row 32 * wave +
// lane % 32, columns 32 * db + 8 * g + 4 * (lane / 32) .. +3. The LSE of all
// slots follows the O of all slots: ws[n_slots * BM * D + slot * BM + row].
// Rows past Nq within a wave that has rows below Nq are stored too (never read).
template <class C, bool CAUSAL, int EMU16, bool PACKED, bool SPLIT = false>
__global__ __attribute__((amdgpu_flat_work_group_size(C::THREADS, C::THREADS),
                          amdgpu_waves_per_eu(C::WAVES_PER_SIMD, C::WAVES_PER_SIMD)))
void fwd_bf16_stream_kernel(const __bf16* __restrict__ Q, const __bf16* __restrict__ K,
                            const __bf16* __restrict__ V, __bf16* __restrict__ O, float* __restrict__ LSE,
                            unsigned long long* __restrict__ stats, int H, int Nq_dense, int Nk_dense, int n_qt,
                            float c, float tau, int bottom_right, const int* __restrict__ cu_q,
                            const int* __restrict__ cu_k, int total_q, int total_k, SplitPlan plan,
                            float* __restrict__ ws) {
  constexpr int D = C::D, BN = C::BN, NW = C::NW, S = C::STAGES;
  constexpr int KB = C::KB;  // 32-key blocks per tile
  static_assert(!(SPLIT && PACKED), "key splitting is for dense batches");
  __shared__ __attribute__((aligned(1024))) char kring[S * C::TILE];
  __shared__ __attribute__((aligned(1024))) char vring[S * C::TILE];

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int hh = lane >> 5, l32 = lane & 31;

  int bh, qt;
  int unit = 0, chunk = 0, unit0 = 0, n_ch = 1;  // SPLIT: this workgroup's unit and chunk
  if (SPLIT) {
    // each XCD takes a contiguous range of units, so the tiles that read one
    // chunk of a head's K and V share that XCD's L2
    const int logical = xcd_logical_id(blockIdx.x, gridDim.x);
    bh = logical / plan.units;
    unit = logical - bh * plan.units;
    plan.unit(unit, qt, chunk, unit0);
    n_ch = plan.n_chunks(qt);
  } else if (CAUSAL) {
    causal_tile_of(blockIdx.x, gridDim.x, n_qt, bh, qt);
  } else {
    const int logical = xcd_logical_id(blockIdx.x, gridDim.x);
    bh = logical / n_qt;
    qt = logical - bh * n_qt;
  }
  const int q0 = qt * C::BM;
  const int qw0 = q0 + wave * 32;
  const int qi = qw0 + l32;
  const Slice sl = slice_of(bh, H, D, Nq_dense, Nk_dense, PACKED ? cu_q : nullptr, cu_k, total_q, total_k);
  const int Nq = sl.Nq, Nk = sl.Nk;
  if (PACKED && q0 >= Nq) return;  // a query tile past this sequence's end
  const size_t qbase = sl.qbase, kbase = sl.kbase;
  const int rs = PACKED ? sl.rs : D;
  const int rsb = rs * 2;
  const uint32_t tile_bytes = (uint32_t)BN * rsb;
  const int diag = bottom_right ? Nk - Nq : 0;  // causal: key j hidden from query i when j > i + diag

  // The swizzles XOR only the low 3 (d = 64, 192) or 4 (d = 128, 256) chunk
  // bits, so the read offsets repeat every KP 16-wide d steps and every VP
  // 32-wide d blocks, shifted by a whole number of 128 / 256 bytes: only the
  // first period lives in registers, the shift is an instruction immediate.
  constexpr int KP = (D == 128 || D == 256) ? 8 : 4, VP = KP / 2;
  constexpr int NKO = D / 16 < KP ? D / 16 : KP, NVO = D / 32 < VP ? D / 32 : VP;
  uint32_t koff[NKO], voff[NVO], kld[C::LOADS], vld[C::LOADS];
  {
    const int krow = key_of_row(l32);
#pragma unroll
    for (int s = 0; s < NKO; ++s) koff[s] = krow * C::RB + 16 * ((2 * s + hh) ^ swz_k<D>(krow));
    const int L = lane & 15, gidx = (lane >> 4) & 1;
    const int vr = 8 * hh + (L >> 2);
#pragma unroll
    for (int db = 0; db < NVO; ++db) {
      const int cch = 4 * db + 2 * gidx + ((L & 3) >> 1);
      voff[db] = vr * C::RB + 16 * (cch ^ swz_v<D>(vr)) + 8 * (L & 1);
    }
#pragma unroll
    for (int i = 0; i < C::LOADS; ++i) {
      const int pos = 64 * (wave + NW * i) + lane;
      const int r = pos / C::CH, p = pos % C::CH;
      kld[i] = r * rsb + 16 * (p ^ swz_k<D>(r));
      vld[i] = r * rsb + 16 * (p ^ swz_v<D>(r));
    }
  }
  const int nrec = Nk * rsb;
  const u32x4 rk = raw_buffer_rsrc(K + kbase, (uint32_t)nrec);
  const u32x4 rv = raw_buffer_rsrc(V + kbase, (uint32_t)nrec);

  bf16x8 qf[D / 16];
  {
    const bool ok = qi < Nq;
    const __bf16* qp = Q + qbase + (size_t)(ok ? qi : 0) * rs + 8 * hh;
#pragma unroll
    for (int s = 0; s < D / 16; ++s) {
      const u32x4 w = ok ? *(const u32x4*)(qp + 16 * s) : u32x4{0u, 0u, 0u, 0u};
      qf[s] = __builtin_bit_cast(bf16x8, w);
    }
  }

  const int kend = CAUSAL ? min(Nk, q0 + C::BM + diag) : Nk;
  // key tiles t0 .. t1-1 (SPLIT: those of this workgroup's chunk; the chunk
  // size is a multiple of BN)
  int t0 = 0, t1 = kend > 0 ? (kend + BN - 1) / BN : 0;
  if (SPLIT && kend > 0) {
    const int kb = chunk * plan.chunk;
    t0 = kb / BN;
    t1 = (min(kend, kb + plan.chunk) + BN - 1) / BN;
  }

  floatx16 o[D / 32];
#pragma unroll
  for (int i = 0; i < D / 32; ++i) o[i] = floatx16{};
  float m_run = kNegInf, l_run = 0.0f;
  const float p_max = exp2_hw(tau);  // largest P the lagging max lets a row keep
  unsigned long long cnt[4] = {0, 0, 0, 0};

  auto load_tile = [&](int t, char* kd, char* vd) __attribute__((always_inline)) {
    const u32x4 rkt = advance_rsrc(rk, (uint32_t)t * tile_bytes), rvt = advance_rsrc(rv, (uint32_t)t * tile_bytes);
    const uint32_t kl = __builtin_amdgcn_readfirstlane(lds_address(kd)), vl = __builtin_amdgcn_readfirstlane(lds_address(vd));
#pragma unroll
    for (int i = 0; i < C::LOADS; ++i) {
      const uint32_t slot = 1024 * (wave + NW * i);
      dma16_at(rkt, kl + slot, kld[i]);
      dma16_at(rvt, vl + slot, vld[i]);
    }
  };

  // O^T += V^T P^T for the tile whose P (bf16) is in pb
  auto pv = [&](const bf16x8 (&pb)[KB][2], const char* vs) __attribute__((always_inline)) {
#pragma unroll
    for (int db = 0; db < D / 32; ++db)
#pragma unroll
      for (int kb = 0; kb < KB; ++kb)
#pragma unroll
        for (int cc = 0; cc < 2; ++cc) {
          const char* vp = vs + voff[db % VP] + (db / VP) * 64 * VP + (kb * 32 + 16 * cc) * C::RB;
          const shortx4 lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_shortx4*)(vp));
          const shortx4 hi = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_shortx4*)(vp + 4 * C::RB));
          const bf16x8 a = __builtin_bit_cast(
              bf16x8, u32x4{__builtin_bit_cast(u32x2, lo)[0], __builtin_bit_cast(u32x2, lo)[1],
                            __builtin_bit_cast(u32x2, hi)[0], __builtin_bit_cast(u32x2, hi)[1]});
          o[db] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, pb[kb][cc], o[db], 0, 0, 0);
        }
  };

  // S^T of tile t from the K tile at ks, masked where the tile crosses the
  // causal diagonal or the end of the keys
  auto scores = [&](int t, const char* ks, floatx16 (&s)[KB]) __attribute__((always_inline)) {
    const int k0 = t * BN;
#pragma unroll
    for (int kb = 0; kb < KB; ++kb) {
#pragma unroll
      for (int st = 0; st < D / 16; ++st) {
        const bf16x8 a = *(const bf16x8*)(ks + kb * 32 * C::RB + koff[st % KP] + (st / KP) * 32 * KP);
        s[kb] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, qf[st], st == 0 ? floatx16{} : s[kb], 0, 0, 0);
      }
    }
    if ((CAUSAL && k0 + BN - 1 > qw0 + diag) || (k0 + BN > Nk)) {
      const int lim = (CAUSAL ? min(Nk - 1, qi + diag) : Nk - 1) - (k0 + 8 * hh);
#pragma unroll
      for (int kb = 0; kb < KB; ++kb)
#pragma unroll
        for (int e = 0; e < 16; ++e) {
          // key k0 + 8h + off is hidden when off > lim (past the last key or
          // the causal diagonal): one compare with a constant per element
          const int off = kb * 32 + 16 * (e >> 3) + (e & 7);
          if (off > lim) s[kb][e] = kNegInf;
        }
    }
  };

  auto compute = [&](int t, const char* ks, const char* vs) __attribute__((always_inline)) {
    const int k0 = t * BN;
    if (CAUSAL && k0 > qw0 + 31 + diag) return;  // wave-uniform: every key of the tile is masked
    floatx16 s[KB];
    scores(t, ks, s);
    bf16x8 pb[KB][2];
    // The common case first, without the row maximum (as in the ping-pong
    // kernel): P from the stale maximum, in place of the scores; if every
    // lane's partial row sum is at most 2^tau, no score exceeded its row's
    // maximum by more than tau and the lagging-max rule keeps it (factor 1).
    // Otherwise -- a row's first tile, a grown maximum -- the scores are
    // computed again from the K tile, which stays in LDS until the end of
    // this step, and the general path below runs on them. Counting launches
    // always take the general path, and so do the software-exp2 instances:
    // with the stale maximum an exponent may exceed 127, where the software
    // exp2 wraps around instead of saturating (the hardware one gives +inf or
    // NaN, which the check rejects). Only at d = 128 and 192: at d = 64 and
    // 256 the second path pushes the kernel past its register budget
    // (spills; measured 13 % and 15 % slower).
    if (EMU16 == 0 && (D == 128 || D == 192) && !stats) {
      const float mc = m_run * c;
#pragma unroll
      for (int kb = 0; kb < KB; ++kb)
#pragma unroll
        for (int e = 0; e < 16; ++e) s[kb][e] = exp2_sel<EMU16>(__builtin_fmaf(s[kb][e], c, -mc), e);
      const float ps = tree_sum<KB>(s);
      __builtin_amdgcn_sched_barrier(0);
      if (!__builtin_amdgcn_ballot_w64(!(ps <= p_max))) {
        l_run = l_run + ps;
#pragma unroll
        for (int kb = 0; kb < KB; ++kb)
#pragma unroll
          for (int cc = 0; cc < 2; ++cc)
#pragma unroll
            for (int e = 0; e < 8; ++e) pb[kb][cc][e] = (__bf16)s[kb][8 * cc + e];
        pv(pb, vs);
        return;
      }
      __builtin_amdgcn_sched_barrier(0);
      scores(t, ks, s);
    }
    const float mx = pl_max_halves(tree_max<KB>(s));
    const float m_new = vmax(m_run, mx);
    const float acc = (m_run - m_new) * c;
    const bool seen = mx > kNegInf;
    const bool commit = seen && !(acc >= -tau);
    const float alpha = commit ? exp2_hw(acc) : 1.0f;
    if (stats) {
      const bool step = seen && (m_run > kNegInf) && hh == 0 && qi < Nq;
      const unsigned long long bs = __builtin_amdgcn_ballot_w64(step);
      const unsigned long long br = __builtin_amdgcn_ballot_w64(step && commit);
      cnt[0] += __builtin_popcountll(bs);
      cnt[1] += __builtin_popcountll(br);
      cnt[2] += bs != 0;
      cnt[3] += br != 0;
    }
    m_run = commit ? m_new : m_run;
    if (__builtin_amdgcn_ballot_w64(commit)) {
#pragma unroll
      for (int db = 0; db < D / 32; ++db) o[db] *= alpha;
    }
    const float mc = (m_run > kNegInf) ? m_run * c : 0.0f;
#pragma unroll
    for (int kb = 0; kb < KB; ++kb)
#pragma unroll
      for (int e = 0; e < 16; ++e) s[kb][e] = exp2_sel<EMU16>(__builtin_fmaf(s[kb][e], c, -mc), e);
    l_run = __builtin_fmaf(l_run, alpha, tree_sum<KB>(s));
#pragma unroll
    for (int kb = 0; kb < KB; ++kb)
#pragma unroll
      for (int cc = 0; cc < 2; ++cc)
#pragma unroll
        for (int e = 0; e < 8; ++e) pb[kb][cc][e] = (__bf16)s[kb][8 * cc + e];
    pv(pb, vs);
  };

  // double-buffered: tile t+1 is in flight while tile t is computed; each
  // wave waits for its own DMA before the barrier that publishes the tile
  char* const k0s = kring;
  char* const v0s = vring;
  char* const k1s = kring + C::TILE;
  char* const v1s = vring + C::TILE;
  if (t0 < t1) {
    load_tile(t0, k0s, v0s);
    wait_own_loads();
    __syncthreads();
  }
  for (int t = t0; t < t1; t += 2) {
    if (t + 1 < t1) load_tile(t + 1, k1s, v1s);
    compute(t, k0s, v0s);
    wait_own_loads();
    __syncthreads();
    if (t + 1 >= t1) break;
    if (t + 2 < t1) load_tile(t + 2, k0s, v0s);
    compute(t + 1, k1s, v1s);
    wait_own_loads();
    __syncthreads();
  }

  const float l_tot = pl_sum_halves(l_run);
  const float inv = l_tot > 0.0f ? 1.0f / l_tot : 0.0f;  // a row that saw no key: O = 0, LSE = -inf
  if (SPLIT && n_ch > 1) {
    // this chunk's share: normalised O in float32 and its LSE in log2 units
    // (a wave whose rows all lie past Nq has nothing to store)
    if (qw0 >= Nq) return;
    const size_t slot = (size_t)bh * plan.units + unit;
    const size_t n_slots = (size_t)gridDim.x;
    floatx4* op = (floatx4*)ws + (slot * NW + wave) * (D / 8) * 64 + lane;
#pragma unroll
    for (int db = 0; db < D / 32; ++db)
#pragma unroll
      for (int g = 0; g < 4; ++g)
        op[(4 * db + g) * 64] =
            floatx4{o[db][4 * g] * inv, o[db][4 * g + 1] * inv, o[db][4 * g + 2] * inv, o[db][4 * g + 3] * inv};
    if (hh == 0)
      ws[n_slots * C::BM * D + slot * C::BM + 32 * wave + l32] =
          l_tot > 0.0f ? m_run * c + __builtin_log2f(l_tot) : kNegInf;
    return;
  }
  if (qi < Nq) {
    __bf16* op = O + qbase + (size_t)qi * rs + 4 * hh;
#pragma unroll
    for (int db = 0; db < D / 32; ++db)
#pragma unroll
      for (int g = 0; g < 4; ++g) {
        bf16x4 w;
#pragma unroll
        for (int r = 0; r < 4; ++r) w[r] = (__bf16)(o[db][4 * g + r] * inv);
        *(bf16x4*)(op + 32 * db + 8 * g) = w;
      }
    if (hh == 0) LSE[sl.lse + qi] = (m_run * c + __builtin_log2f(l_tot)) * 0.693147180559945309f;
  }
  if (stats && lane == 0) {
#pragma unroll
    for (int i = 0; i < 4; ++i) atomicAdd(stats + i, cnt[i]);
  }
}

}  // namespace
}  // namespace attn
