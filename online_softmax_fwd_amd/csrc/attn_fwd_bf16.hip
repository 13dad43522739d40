// attn_fwd_bf16.hip -- bf16 attention forward for gfx950 (MI355X).
//
// A workgroup of 8 waves owns 256 query rows of one (batch, head) (128 or 64
// in small launches, with key parities: see below); each wave owns 32 rows.
// K and V stream through LDS in 64-key tiles, two buffers per
// tensor; per row the wave keeps a running max m (raw score units), a
// denominator l and a 32 x d float accumulator, so S and P never reach
// memory. Per tile and wave:
//
//   S^T = K_tile Q^T      v_mfma_f32_32x32x16_bf16; A = K rows (LDS), B = Q
//                         (registers). The 32x32 output puts one query per
//                         lane (lane % 32) and 16 keys per lane, so the row
//                         max and row sum are in-lane plus one exchange between
//                         the two 32-lane halves.
//   mask                  only on tiles that cross the causal diagonal or the
//                         end of the keys ("Lecture 2 -- Online Softmax and
//                         Numerical Correctness", section "Causal masking just
//                         changes which blocks contribute"); tiles above the
//                         workgroup's diagonal are never loaded.
//   lagging max           "FlashAttention-4's Softmax Tricks", section
//                         "Conditional rescaling, and when it's exact": keep the
//                         stale max while (m_old - m_new) * scale_log2 >= -tau,
//                         else commit and rescale O and l by that power of two;
//                         the O rescale is a wave-uniform branch.
//   P = 2^(S*c - m*c)     one FMA then exp2 (the exp2 fold of "Flash Attention 4
//                         -- the algorithm and the two-MMA problem", section "The
//                         exp2 trick"): hardware, software, or a fixed mix
//   l = alpha*l + sum P   from the float32 P
//   O^T += V^T P^T        v_mfma_f32_32x32x16_bf16; A = V^T read from the
//                         row-major V tile with ds_read_b64_tr_b16, B = P in
//                         bf16 taken straight from the S^T registers (the K rows
//                         feeding S^T are permuted so each lane half holds 8
//                         consecutive keys per 16-key step, which is the PV
//                         operand layout).
// The epilogue divides by l once per row and writes LSE = ln2 * (m*c + log2 l).
//
// Memory path. K and V tiles go from HBM to LDS with buffer_load_dwordx4 ...
// lds (no VGPR staging, no address registers beyond one offset per load): a
// wave-load writes 64 lanes x 16 B contiguously, and each lane picks the global
// 16-byte chunk that belongs at its LDS slot. The buffer range check returns
// zeros past the last key, which makes ragged tails free. Within a row the
// 16-byte chunks are XOR-swizzled per tile so that
//   - the K reads of one instruction (32 rows x one chunk) and
//   - the V transpose reads (8 rows x 4 chunks)
// each spread evenly over the 64 LDS banks.
//
// Schedule: see "Ping-pong schedule" below.
#include "attn_fwd_bf16_kernels.h"

namespace attn {
namespace {


// ---------------------------------------------------------------------------
// The MFMA phase as one software-pipelined sequence: the PV MFMAs of the
// previous tile, then the S^T MFMAs of the current tile. Operands come from
// LDS through a ring RING MFMAs deep (the LDS round trip is several MFMA
// durations long), and consecutive MFMAs rotate over independent accumulators
// (the 4 (d=128) or 2 (d=64) blocks of O^T, then the 2 blocks of S^T). The
// previous tile's P arrives as bf16 (pb, converted by the softmax stage).
// sched_barrier pins the issue order so the reads stay ahead.
// ---------------------------------------------------------------------------
template <int D, int KB, int RB, bool DO_PV, bool DO_QK>
__device__ __forceinline__ void mfma_sequence(floatx16 (&o)[D / 32], floatx16 (&s)[KB], const bf16x8 (&pb)[KB][2],
                                              const bf16x8 (&qf)[D / 16], uint32_t ksrc, uint32_t vsrc,
                                              const uint32_t (&koff)[D / 16], const uint32_t (&voff)[D / 32]) {
  constexpr int NDB = D / 32;
  constexpr int NPV = DO_PV ? NDB * KB * 2 : 0;
  constexpr int NQK = DO_QK ? KB * (D / 16) : 0;
  constexpr int N = NPV + NQK;
  constexpr int RING = 6;
  auto read = [&](int i) __attribute__((always_inline)) -> bf16x8 {
    if (i < NPV) {
      const int db = i % NDB, k = i / NDB, kb = k >> 1, cc = k & 1;
      const uint32_t vp = voff[db] + vsrc + (kb * 32 + 16 * cc) * RB;
      const shortx4 lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_shortx4*)(uintptr_t)(vp));
      const shortx4 hi = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_shortx4*)(uintptr_t)(vp + 4 * RB));
      return __builtin_bit_cast(bf16x8, u32x4{__builtin_bit_cast(u32x2, lo)[0], __builtin_bit_cast(u32x2, lo)[1],
                                              __builtin_bit_cast(u32x2, hi)[0], __builtin_bit_cast(u32x2, hi)[1]});
    }
    const int q = i - NPV, kb = q % KB, st = q / KB;
    return *(const lds_bf16x8*)(uintptr_t)(koff[st] + ksrc + kb * 32 * RB);
  };
  bf16x8 ring[RING];
#pragma unroll
  for (int i = 0; i < RING && i < N; ++i) ring[i] = read(i);

  __builtin_amdgcn_sched_barrier(0);

  auto mma = [&](int i, const bf16x8& a) __attribute__((always_inline)) {
    if (i < NPV) {
      const int db = i % NDB, k = i / NDB, kb = k >> 1, cc = k & 1;
      o[db] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, pb[kb][cc], o[db], 0, 0, 0);
    } else {
      const int q = i - NPV, kb = q % KB, st = q / KB;
      s[kb] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, qf[st], st == 0 ? floatx16{} : s[kb], 0, 0, 0);
    }
  };
#pragma unroll
  for (int i = 0; i < N; ++i) {
    const bf16x8 a = ring[i % RING];
    if (i + RING < N) ring[i % RING] = read(i + RING);
    mma(i, a);
    __builtin_amdgcn_sched_barrier(0);
  }
}

// Depth of the ping-pong kernel's K/V ring in LDS (tiles of each): a tile's
// DMA is issued 2S - 2 half-phases before its first reader. Depth 3 (96 KiB
// of LDS) measured no faster than 2 at d = 128: the loads already arrive in
// time.
constexpr int kPingPongStages = 2;
#ifndef PP_PERSIST
#define PP_PERSIST 1
#endif
constexpr bool kPingPongPersist = PP_PERSIST;
constexpr int kPingPongPersistWgs = 256;  // one per CU (8 XCDs x 32)

// ---------------------------------------------------------------------------
// Ping-pong schedule. The 8 waves form two groups of 4 (one wave of each
// group per SIMD). Each wave runs, per K/V tile j,
//     MFMA phase M(j): O^T += V_{j-1}^T P_{j-1}^T   and   S_j^T = K_j Q^T
//     VALU phase V(j): mask, row max, lagging-max rescale, P_j = exp2, row sum
// and group 1 runs one phase behind group 0, with a workgroup barrier between
// phases: while one wave of a SIMD issues MFMAs the other issues the softmax
// VALU work, so the matrix core and the vector ALU overlap. Tile j's K and
// V_{j-1} are read in the two half-phases 2j and 2j+1; the DMA for K_{j+1} and
// V_j is issued at the start of half-phase 2j into the other buffer of each
// pair and waited for at the end of half-phase 2j+1.
//
// Key parities (KPAR = 2 or 4, small launches at d = 128): the workgroup
// owns 256 / KPAR rows; waves w, w + 8/KPAR, ... hold the same 32 rows and
// take consecutive 32-key parts of every tile of 32 * KPAR keys (one tile
// holds 64 or 128 keys), each with its own m, l and O; the parities of a row
// block split over the two groups, so the phases still alternate on every
// SIMD. At the end the states merge exactly through LDS ("Lecture 2 --
// Online Softmax and Numerical Correctness", section "Combining two blocks
// exactly").
// ---------------------------------------------------------------------------
// Persistent grid: 8 * NS workgroups, NS on each XCD (workgroup wg runs on
// XCD wg % 8), each looping over query tiles until its share is done. XCD x
// owns an eighth of the tiles (the batch-heads count is a multiple of 8):
// non-causal, the contiguous logical range [x * per, (x + 1) * per) of
// (head, tile) pairs, taken NS at a time, so that each round holds whole
// heads whose K and V the XCD's L2 shares; causal, the heads bh = x (mod 8)
// G = NS / n_qt at a time when that divides evenly (round k: the tiles of G
// heads, one per workgroup, longest first in even rounds and shortest first
// in odd ones, so every workgroup's sum is the same: 34 key tiles each for
// 16 tiles of 8 heads on 32 workgroups), else longest tile first over all
// the XCD's heads, dealt in alternating directions. Tile k of workgroup wg,
// or false past its share.
__device__ __forceinline__ bool persistent_tile(int wg, int n_wg, int k, int n_qt, int n_tiles, bool causal,
                                                int& bh, int& qt) {
  const int x = wg & 7, s = wg >> 3, ns = n_wg >> 3;
  const int per = n_tiles >> 3;
  if (causal && ns % n_qt == 0 && (per / n_qt) % (ns / n_qt) == 0) {
    // G = NS / n_qt heads at a time (round k: heads kG .. kG + G - 1 of the
    // XCD, one tile per workgroup), so that few heads' K and V are in flight
    // in the XCD's L2; the tiles' lengths alternate direction between rounds
    // (round k even: longest first), which evens out each workgroup's sum
    const int G = ns / n_qt, hpx = per / n_qt;
    if (k >= hpx / G) return false;
    const int r = s / G;
    qt = (k & 1) ? r : n_qt - 1 - r;
    bh = (k * G + s % G) * 8 + x;
    return true;
  }
  const int p = k * ns + ((causal && (k & 1)) ? ns - 1 - s : s);
  if (p >= per) return false;
  if (causal) {
    const int hpx = per / n_qt;  // heads per XCD
    qt = n_qt - 1 - p / hpx;
    bh = (p % hpx) * 8 + x;
  } else {
    const int logical = x * per + p;
    bh = logical / n_qt;
    qt = logical - bh * n_qt;
  }
  return true;
}

template <int D, bool CAUSAL, int EMU16, bool PACKED, bool PERSIST, int KPAR = 1>
__global__ __attribute__((amdgpu_flat_work_group_size(512, 512), amdgpu_waves_per_eu(2, 2)))
void fwd_bf16_kernel(const __bf16* __restrict__ Q, const __bf16* __restrict__ K, const __bf16* __restrict__ V,
                     __bf16* __restrict__ O, float* __restrict__ LSE, unsigned long long* __restrict__ stats,
                     int H, int Nq_dense, int Nk_dense, int n_qt, float c, float tau, int bottom_right,
                     const int* __restrict__ cu_q, const int* __restrict__ cu_k, int total_q, int total_k,
                     int n_tiles) {
  static_assert(!(PERSIST && PACKED), "persistent launches are dense");
  static_assert(KPAR == 1 || (D == 128 && !PERSIST && (KPAR == 2 || KPAR == 4)), "key parities");
  // KPAR key parities: waves w, w + RW, ... own the same 32 rows and take
  // consecutive 32-key parts of every key tile, each with its own softmax
  // state, merged exactly at the end (one parity: 64-key tiles, 256 rows)
  constexpr int RW = 8 / KPAR;                    // 32-row blocks per workgroup
  constexpr int BM = 32 * RW;                     // query rows per workgroup
  constexpr int KB = KPAR == 1 ? 2 : 1;           // 32-key blocks per wave per tile
  using C = Cfg<D, 32 * KB * KPAR, 8>;
  constexpr int BN = C::BN;
  constexpr int S = kPingPongStages;
  __shared__ __attribute__((aligned(1024))) char kring[S * C::TILE];
  __shared__ __attribute__((aligned(1024))) char vring[S * C::TILE];
  __shared__ float xml[KPAR > 1 ? 2 * 8 * 64 : 1];  // key parities: every wave's m and l at the end

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int group = wave >> 2;
  const int hh = lane >> 5, l32 = lane & 31;
  const int rw = wave % RW, par = wave / RW;  // row block, key parity
  // a counting launch, as a scalar: tested per tile, a pointer compare kept
  // as a lane mask cost two vector instructions a step
  const int counting = __builtin_amdgcn_readfirstlane(stats != nullptr ? 1 : 0);
  const int kw = par * KB * 32;               // first key of this wave's part of a tile

  bf16x8 qf[D / 16];  // Q as the B operand: lane (h, n) holds Q[n][16s + 8h .. +8]

  // One query tile: everything below runs per tile (returns end the tile, and
  // are taken by the whole workgroup, so the barrier counts stay matched).
  // pre: the previous tile already loaded this tile's Q and its first K tile;
  // nbh >= 0: this tile loads those of tile (nbh, nqt) after its last LDS
  // read, so that they arrive during its epilogue. Returns whether it did.
  auto run_tile = [&](const int bh, const int qt, const bool pre, const int nbh, const int nqt)
                      __attribute__((always_inline)) -> bool {
  const int q0 = qt * BM;
  const int qw0 = q0 + rw * 32;
  const int qi = qw0 + l32;
  // PACKED: a sequence of a packed batch (rows H*D apart); else dense [B,H,N,D]
  // with the row pitch a compile-time constant
  const Slice sl = slice_of(bh, H, D, Nq_dense, Nk_dense, PACKED ? cu_q : nullptr, cu_k, total_q, total_k);
  const int Nq = sl.Nq, Nk = sl.Nk;
  if (PACKED && q0 >= Nq) return false;  // a query tile past this sequence's end
  const size_t qbase = sl.qbase, kbase = sl.kbase;
  const int rs = PACKED ? sl.rs : D;  // elements between rows in memory
  const int rsb = rs * 2;             // bytes between K/V rows
  // causal: key j is hidden from query i when j > i + diag (top-left: diag = 0)
  const int diag = bottom_right ? Nk - Nq : 0;

  // ---- per-lane constants --------------------------------------------------
  // LDS addresses of the K/V reads carry the ring's base in the register part
  // (opaque to the compiler, so it does not split it off again), leaving
  // slot + in-tile offsets below 64 KiB for the instruction's immediate field:
  // the rings span more than a 16-bit offset reaches.
  uint32_t kr = lds_address(kring), vbase = lds_address(vring);
  asm volatile("" : "+s"(kr));
  asm volatile("" : "+s"(vbase));
  uint32_t koff[D / 16], voff[D / 32], kld[C::LOADS], vld[C::LOADS];
  {
    const int krow = key_of_row(l32);
#pragma unroll
    for (int s = 0; s < D / 16; ++s) koff[s] = kr + (kw + krow) * C::RB + 16 * ((2 * s + hh) ^ swz_k<D>(krow));
    const int L = lane & 15, gidx = (lane >> 4) & 1;
    const int vr = 8 * hh + (L >> 2);
#pragma unroll
    for (int db = 0; db < D / 32; ++db) {
      const int cch = 4 * db + 2 * gidx + ((L & 3) >> 1);
      voff[db] = vbase + (kw + vr) * C::RB + 16 * (cch ^ swz_v<D>(vr)) + 8 * (L & 1);
    }
#pragma unroll
    for (int i = 0; i < C::LOADS; ++i) {
      const int pos = 64 * (wave + 8 * i) + lane;
      const int r = pos / C::CH, p = pos % C::CH;
      kld[i] = r * rsb + 16 * (p ^ swz_k<D>(r));
      vld[i] = r * rsb + 16 * (p ^ swz_v<D>(r));
    }
  }
  const int nrec = Nk * rsb;
  const uint32_t tile_bytes = (uint32_t)BN * rsb;
  const u32x4 rk = raw_buffer_rsrc(K + kbase, (uint32_t)nrec);
  const u32x4 rv = raw_buffer_rsrc(V + kbase, (uint32_t)nrec);

  // ---- Q as the B operand: lane (h, n) holds Q[n][16s + 8h .. +8] -----------
  if (!pre) {
    const bool ok = qi < Nq;
    const __bf16* qp = Q + qbase + (size_t)(ok ? qi : 0) * rs + 8 * hh;
#pragma unroll
    for (int s = 0; s < D / 16; ++s) {
      const u32x4 w = ok ? *(const u32x4*)(qp + 16 * s) : u32x4{0u, 0u, 0u, 0u};
      qf[s] = __builtin_bit_cast(bf16x8, w);
    }
  }

  // causal: key j is hidden from query i when j > i + diag (diag = 0 aligns the
  // mask top-left, Nk - Nq bottom-right)
  const int kend = CAUSAL ? min(Nk, q0 + BM + diag) : Nk;
  const int T = (kend + BN - 1) / BN;
  if (T <= 0) {  // no row of this workgroup sees a key (bottom-right, Nq > Nk)
    if (par == 0 && qi < Nq) {
      __bf16* op = O + qbase + (size_t)qi * rs + 4 * hh;
#pragma unroll
      for (int db = 0; db < D / 32; ++db)
#pragma unroll
        for (int g = 0; g < 4; ++g) *(bf16x4*)(op + 32 * db + 8 * g) = bf16x4{};
      if (hh == 0) LSE[sl.lse + qi] = kNegInf;
    }
    return false;
  }

  floatx16 o[D / 32];
#pragma unroll
  for (int i = 0; i < D / 32; ++i) o[i] = floatx16{};
  floatx16 s[KB];        // S^T of the current tile, then its float32 P
  bf16x8 pb[KB][2];      // that P as bf16, the next MFMA phase's PV B operand
  float alpha_p = 1.0f;  // rescale factor of the tile whose P is in s
  const float p_max = exp2_hw(tau);  // largest P the lagging max lets a row keep
  float m_run = kNegInf;  // running max, raw score units
  float l_run = 0.0f;     // running denominator over this lane's half of the keys
  unsigned long long cnt[4] = {0, 0, 0, 0};

  // DMA batch b: this wave's share of K_{b+S-1} (into ring slot ks) and
  // V_{b+S-2} (into slot vs), the tiles that MFMA phase b+S-1 reads. The
  // tile's byte offset goes into a copy of the buffer descriptor (base
  // advanced, size shortened: scalar arithmetic, and the range check still
  // zero-fills past the last key) rather than into every lane's offset, and
  // M0 is the ring's LDS base plus a constant.
  auto load_tiles = [&](int b, uint32_t ks, uint32_t vs) __attribute__((always_inline)) {
    const int tk = b + S - 1, tv = b + S - 2;
    if (tk < T) {
      const u32x4 r = advance_rsrc(rk, (uint32_t)tk * tile_bytes);
#pragma unroll
      for (int i = 0; i < C::LOADS; ++i) dma16_at(r, kr + ks + 1024 * (wave + 8 * i), kld[i]);
    }
    if (tv < T) {
      const u32x4 r = advance_rsrc(rv, (uint32_t)tv * tile_bytes);
#pragma unroll
      for (int i = 0; i < C::LOADS; ++i) dma16_at(r, vbase + vs + 1024 * (wave + 8 * i), vld[i]);
    }
  };
  // Wait until batch j - S + 2 (issued S - 2 batches before the newest, j)
  // has landed: vmcnt counts this wave's outstanding DMAs in issue order, so
  // the wait leaves the newer batches j - S + 3 .. j in flight.
  auto wait_batch = [&](int j) __attribute__((always_inline)) {
    int newer = 0;  // DMAs per wave in batches j - S + 3 .. j (wave-uniform)
#pragma unroll
    for (int b = j - S + 3; b <= j; ++b) newer += C::LOADS * ((b + S - 1 < T) + (b + S - 2 < T));
    static_for<0, 2 * (S - 2) * C::LOADS + 1>([&](auto n) __attribute__((always_inline)) {
      if (newer == decltype(n)::value) asm volatile("s_waitcnt vmcnt(%0)" ::"n"(decltype(n)::value) : "memory");
    });
  };

  // MFMA phase: PV of tile j-1 from vsrc (DO_PV) and S^T of tile j from ksrc
  // (DO_QK). The MFMA phase sets the pace of the schedule (more MFMA work per
  // tile costs more than less softmax work saves), so a wave raises its issue
  // priority while in it: when the matrix core frees up, the SIMD issues the
  // next MFMA before the other wave's vector instructions.
  auto mfma_phase = [&](auto do_pv, auto do_qk, uint32_t ksrc, uint32_t vsrc) __attribute__((always_inline)) {
    __builtin_amdgcn_sched_barrier(0);
    __builtin_amdgcn_s_setprio(1);
    __builtin_amdgcn_sched_barrier(0);
    mfma_sequence<D, KB, C::RB, decltype(do_pv)::value, decltype(do_qk)::value>(o, s, pb, qf, ksrc, vsrc,
                                                                                  koff, voff);
    __builtin_amdgcn_sched_barrier(0);
    __builtin_amdgcn_s_setprio(0);
    __builtin_amdgcn_sched_barrier(0);
  };

  // VALU phase j: softmax of tile j
  auto valu_phase = [&](int j) __attribute__((always_inline)) {
    const int k0 = j * BN + kw;  // first key of this wave's part of tile j
    if ((CAUSAL && k0 + KB * 32 - 1 > qw0 + diag) || (k0 + KB * 32 > Nk)) {
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
    if constexpr (D == 128) {
      // The common case without the row maximum: P from the stale maximum.
      // Each P of a lane is at most that lane's partial row sum, so if every
      // lane's sum is at most 2^tau, no score of this tile exceeds its row's
      // maximum by more than tau and the rule keeps the stale maximum
      // (factor 1) -- the decision the general path below takes, on the same
      // P and the same sum, without its maximum trees. A row's first tile
      // (m = -inf gives an infinite or NaN sum), a row whose maximum grew by
      // more than tau, and counting launches take the general path on the
      // kept scores. At d = 192 the kernel has no registers for the second
      // copy of the scores. Only with the hardware exp2: with the stale
      // maximum an exponent may exceed 127, where the software exp2 wraps
      // around instead of saturating to +inf or NaN as v_exp_f32 does.
      if (EMU16 == 0 && j > 0 && !counting) {
        const float mc = m_run * c;
        floatx16 p[KB];
#pragma unroll
        for (int kb = 0; kb < KB; ++kb)
#pragma unroll
          for (int e = 0; e < 16; ++e) p[kb][e] = exp2_sel<EMU16>(__builtin_fmaf(s[kb][e], c, -mc), e);
        const float ps = tree_sum<KB>(p);
        __builtin_amdgcn_sched_barrier(0);
        if (!__builtin_amdgcn_ballot_w64(!(ps <= p_max))) {
          alpha_p = 1.0f;
          l_run = l_run + ps;
#pragma unroll
          for (int kb = 0; kb < KB; ++kb)
#pragma unroll
            for (int cc = 0; cc < 2; ++cc)
#pragma unroll
              for (int e = 0; e < 8; ++e) pb[kb][cc][e] = (__bf16)p[kb][8 * cc + e];
#pragma unroll
          for (int kb = 0; kb < KB; ++kb)
#pragma unroll
            for (int cc = 0; cc < 2; ++cc) asm volatile("" : "+v"(pb[kb][cc]));
          asm volatile("" : "+v"(l_run));
          return;
        }
        __builtin_amdgcn_sched_barrier(0);
      }
    }
    const float mx = pl_max_halves(tree_max<KB>(s));

    const float m_new = vmax(m_run, mx);
    const float acc = (m_run - m_new) * c;  // -inf on a row's first block
    const bool seen = mx > kNegInf;
    const bool commit = seen && !(acc >= -tau);
    alpha_p = commit ? exp2_hw(acc) : 1.0f;
    if (counting) {
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
      for (int db = 0; db < D / 32; ++db) o[db] *= alpha_p;
    }
    // P = 2^(S*c - m*c) as float32 in s, its row sum folded into l, and P as
    // bf16 in pb (converted here rather than at the start of the MFMA phase,
    // which is the critical one; this also carries 16 registers of P across
    // the barrier instead of 32)
    const float mc = (m_run > kNegInf) ? m_run * c : 0.0f;
#pragma unroll
    for (int kb = 0; kb < KB; ++kb)
#pragma unroll
      for (int e = 0; e < 16; ++e) s[kb][e] = exp2_sel<EMU16>(__builtin_fmaf(s[kb][e], c, -mc), e);
    l_run = __builtin_fmaf(l_run, alpha_p, tree_sum<KB>(s));
#pragma unroll
    for (int kb = 0; kb < KB; ++kb)
#pragma unroll
      for (int cc = 0; cc < 2; ++cc)
#pragma unroll
        for (int e = 0; e < 8; ++e) pb[kb][cc][e] = (__bf16)s[kb][8 * cc + e];
    // P and l must be complete here, in the VALU phase. Without these empty
    // asms the compiler sinks the exponentials and the conversion into the
    // next MFMA phase, past the barrier, and the row sum into the VALU phase
    // after it, which keeps the float32 P of one tile alive next to the S^T of
    // the next (32 more registers, copied at the loop's back edge).
#pragma unroll
    for (int kb = 0; kb < KB; ++kb)
#pragma unroll
      for (int cc = 0; cc < 2; ++cc) asm volatile("" : "+v"(pb[kb][cc]));
    asm volatile("" : "+v"(l_run));
  };

  // One step j = [MFMA phase j] barrier [VALU phase j] barrier, identical for
  // both groups; group 1 runs it one barrier later. K_t and V_t sit in ring
  // slot t % S. DMA batch b (K_{b+S-1}, V_{b+S-2}) is issued at half-phase 2b
  // (group 0 at the start of its MFMA phase b, group 1 at the start of its
  // VALU phase b-1; batch 0 by every wave in the prologue), into the slots of
  // K_{b-1} and V_{b-2}, which every wave
  // finished reading in MFMA phase b-1, and waited for at the end of
  // half-phase 2b + 2S - 3, just before MFMA phase b+S-1 reads it. The slots
  // are compile-time constants (the loop is unrolled S times), so every LDS
  // access has a known target. Step 0 has no PV and step T no S^T or softmax;
  // every other step runs the full MFMA phase for every wave, also on tiles
  // that the causal mask empties for some of its rows (the softmax turns those
  // into P = 0), which keeps the loop free of data-dependent branches.
  auto slot_off = [&](int i) __attribute__((always_inline)) -> uint32_t { return ((i % S + S) % S) * C::TILE; };
  auto step = [&](int j, auto do_pv, auto do_qk, auto slot) __attribute__((always_inline)) {
    constexpr int r = decltype(slot)::value;  // j % S
    if (group == 0 && j > 0) load_tiles(j, slot_off(r - 1), slot_off(r - 2));  // batch 0: in the prologue
    mfma_phase(do_pv, do_qk, slot_off(r), slot_off(r - 1));
    if (group == 1) wait_batch(j);
    block_sync();
    if (group == 1) load_tiles(j + 1, slot_off(r), slot_off(r - 1));
    if constexpr (decltype(do_qk)::value) valu_phase(j);
    if (group == 0) wait_batch(j);
    block_sync();
  };
  using Y = std::true_type;
  using N = std::false_type;
  using I0 = std::integral_constant<int, 0>;

  // prologue: K_0 and DMA batch 0 (K_1, V_0) by every wave, in flight
  // together with Q (all already in flight when the previous tile prefetched
  // them), so that the first PV does not wait for V_0
  static_assert(S == 2, "the prologue and the prefetch load two stages' first tiles");
  if (!pre) {
#pragma unroll
    for (int i = 0; i < C::LOADS; ++i)
      if (T > 0) dma16_at(rk, kr + 1024 * (wave + 8 * i), kld[i]);
    load_tiles(0, slot_off(S - 1), slot_off(S - 2));
  }
  wait_own_loads();
  block_sync();
  if (group == 1) block_sync();  // group 1 runs one phase behind
  // Causal: group 0 holds the workgroup's first 128 rows, which see no key of
  // its last tiles (up to two of them). Group 0 runs the full steps only up
  // to the last tile one of its rows can see (Tw), PV of that tile in step
  // Tw, and in the steps after it only its share of the tile DMAs and the
  // barriers. The skipped tiles are fully masked for these rows (P = 0), so
  // the result is the same.
  int Tw = T;
  if (CAUSAL && KPAR == 1 && group == 0) Tw = max(1, min(T, (q0 + 127 + diag) / BN + 1));
  step(0, N{}, Y{}, I0{});
  int j = 1;
  for (; j + S - 1 < Tw; j += S)
    static_for<0, S>([&](auto R) __attribute__((always_inline)) {
      step(j + R, Y{}, Y{}, std::integral_constant<int, (decltype(R)::value + 1) % S>{});
    });
  // the remaining steps j .. Tw-1 (fewer than S; j = 1 mod S), then step Tw: PV of the last tile
  static_for<0, S - 1>([&](auto R) __attribute__((always_inline)) {
    if (j + R < Tw) step(j + R, Y{}, Y{}, std::integral_constant<int, (decltype(R)::value + 1) % S>{});
  });
  static_for<0, S>([&](auto R) __attribute__((always_inline)) {
    if (Tw % S == R) step(Tw, Y{}, N{}, R);
  });
  if (CAUSAL) {
    for (int i = Tw + 1; i <= T; ++i) {  // group 0 only: DMA share and barriers of step i
      load_tiles(i, slot_off(i % S - 1), slot_off(i % S - 2));
      block_sync();
      wait_batch(i);
      block_sync();
    }
  }
  if (group == 0) block_sync();

  // Every wave is past its last LDS read of this tile and its last use of Q:
  // the next tile's Q and first K tile can load now, behind the epilogue.
  bool prefetched = false;
  if (nbh >= 0) {
    const Slice sn = slice_of(nbh, H, D, Nq_dense, Nk_dense, nullptr, cu_k, total_q, total_k);
    const int q0n = nqt * BM, qin = q0n + rw * 32 + l32;
    const bool ok = qin < sn.Nq;
    const __bf16* qp = Q + sn.qbase + (size_t)(ok ? qin : 0) * D + 8 * hh;
#pragma unroll
    for (int s = 0; s < D / 16; ++s) {
      const u32x4 w = ok ? *(const u32x4*)(qp + 16 * s) : u32x4{0u, 0u, 0u, 0u};
      qf[s] = __builtin_bit_cast(bf16x8, w);
    }
    // its prologue's tiles: K_0, then batch 0 (K_1, V_0)
    const int kendn = CAUSAL ? min(sn.Nk, q0n + BM + diag) : sn.Nk;
    const int Tn = (kendn + BN - 1) / BN;
    const uint32_t nrecn = (uint32_t)(sn.Nk * rsb);
    const u32x4 rkn = raw_buffer_rsrc(K + sn.kbase, nrecn);
    const u32x4 rvn = raw_buffer_rsrc(V + sn.kbase, nrecn);
    if (Tn > 0) {
#pragma unroll
      for (int i = 0; i < C::LOADS; ++i) dma16_at(rkn, kr + 1024 * (wave + 8 * i), kld[i]);
    }
    if (Tn > 1) {
      const u32x4 r1 = advance_rsrc(rkn, tile_bytes);
#pragma unroll
      for (int i = 0; i < C::LOADS; ++i) dma16_at(r1, kr + C::TILE + 1024 * (wave + 8 * i), kld[i]);
    }
    if (Tn > 0) {
#pragma unroll
      for (int i = 0; i < C::LOADS; ++i) dma16_at(rvn, vbase + 1024 * (wave + 8 * i), vld[i]);
    }
    prefetched = true;
  }

  if constexpr (KPAR > 1) {
    // The parities' states merge by the exact rule ("Combining two blocks
    // exactly"): with M the largest maximum of a row, each state is weighted
    // by 2^((m - M) * c) (0 for a state that saw no key), l and O add. Every
    // wave merges and stores its own slice of the columns (BPP 32-column
    // blocks, parity q the blocks q * BPP ..), so the work spreads over all
    // waves: each writes the blocks it does not keep into the free K/V rings
    // (4 KiB per block, float4 per lane) and its m and l into xml, and after
    // one barrier reads its blocks of the other parities of its rows.
    constexpr int BPP = (D / 32) / KPAR;      // 32-column blocks a parity keeps
    constexpr int NB = D / 32 - BPP;          // blocks a wave hands over
    constexpr int XB = 64 * 16 * 4;           // bytes of one block
    constexpr int RING = S * C::TILE;
    static_assert(8 * NB * XB <= 2 * RING && RING % XB == 0, "the handed-over blocks fit the K and V rings");
    auto xblock = [&](int w, int db) __attribute__((always_inline)) -> floatx4* {
      const int pw = w / RW;  // the parity of wave w
      const int k = db < pw * BPP ? db : db - BPP;
      const int off = (w * NB + k) * XB;
      return (floatx4*)(off < RING ? kring + off : vring + (off - RING)) + lane;
    };
#pragma unroll
    for (int db = 0; db < D / 32; ++db) {
      if (db / BPP == par) continue;
      floatx4* xo = xblock(wave, db);
#pragma unroll
      for (int g = 0; g < 4; ++g) xo[g * 64] = floatx4{o[db][4 * g], o[db][4 * g + 1], o[db][4 * g + 2], o[db][4 * g + 3]};
    }
    xml[wave * 64 + lane] = m_run;
    xml[(8 + wave) * 64 + lane] = l_run;
    __syncthreads();
    float mp[KPAR], lp[KPAR];
#pragma unroll
    for (int p1 = 0; p1 < KPAR; ++p1) {
      mp[p1] = xml[(p1 * RW + rw) * 64 + lane];
      lp[p1] = xml[(8 + p1 * RW + rw) * 64 + lane];
    }
    float mm = mp[0];
#pragma unroll
    for (int p1 = 1; p1 < KPAR; ++p1) mm = vmax(mm, mp[p1]);
    float a[KPAR];
    float lsum = 0.0f;
#pragma unroll
    for (int p1 = 0; p1 < KPAR; ++p1) {
      a[p1] = mp[p1] > kNegInf ? exp2_hw((mp[p1] - mm) * c) : 0.0f;
      lsum = __builtin_fmaf(lp[p1], a[p1], lsum);
    }
    const float l_tot = pl_sum_halves(lsum);
    const float inv = l_tot > 0.0f ? 1.0f / l_tot : 0.0f;  // a row that saw no key: O = 0, LSE = -inf
#pragma unroll
    for (int db = 0; db < D / 32; ++db) {
      if (db / BPP != par) continue;  // wave-uniform; db stays a constant index into o
      floatx16 acc;
#pragma unroll
      for (int e = 0; e < 16; ++e) acc[e] = 0.0f;
#pragma unroll
      for (int p1 = 0; p1 < KPAR; ++p1) {
        if (p1 == par) {
#pragma unroll
          for (int e = 0; e < 16; ++e) acc[e] = __builtin_fmaf(o[db][e], a[p1], acc[e]);
        } else {
          const floatx4* xo = xblock(p1 * RW + rw, db);
#pragma unroll
          for (int g = 0; g < 4; ++g) {
            const floatx4 x = xo[g * 64];
#pragma unroll
            for (int r = 0; r < 4; ++r) acc[4 * g + r] = __builtin_fmaf(x[r], a[p1], acc[4 * g + r]);
          }
        }
      }
      if (qi < Nq) {
        __bf16* op = O + qbase + (size_t)qi * rs + 4 * hh + 32 * db;
#pragma unroll
        for (int g = 0; g < 4; ++g) {
          bf16x4 w;
#pragma unroll
          for (int r = 0; r < 4; ++r) w[r] = (__bf16)(acc[4 * g + r] * inv);
          *(bf16x4*)(op + 8 * g) = w;
        }
      }
    }
    if (par == 0 && qi < Nq && hh == 0) LSE[sl.lse + qi] = (mm * c + __builtin_log2f(l_tot)) * 0.693147180559945309f;
    if (stats && lane == 0) {
#pragma unroll
      for (int i = 0; i < 4; ++i) atomicAdd(stats + i, cnt[i]);
    }
    return prefetched;
  }

  // ---- epilogue: O / l, LSE -------------------------------------------------
  const float l_tot = pl_sum_halves(l_run);
  const float inv = l_tot > 0.0f ? 1.0f / l_tot : 0.0f;  // a row that saw no key: O = 0, LSE = -inf
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
  return prefetched;
  };

  if constexpr (PERSIST) {
    int bh, qt;
    if (!persistent_tile(blockIdx.x, gridDim.x, 0, n_qt, n_tiles, CAUSAL, bh, qt)) return;
    bool pre = false;
    for (int k = 0;; ++k) {
      int nbh = -1, nqt = 0;
      const bool more = persistent_tile(blockIdx.x, gridDim.x, k + 1, n_qt, n_tiles, CAUSAL, nbh, nqt);
      pre = run_tile(bh, qt, pre, more ? nbh : -1, nqt);
      if (!more) break;
      bh = nbh;
      qt = nqt;
    }
  } else {
  int bh, qt;
  if (CAUSAL) {
    causal_tile_of(blockIdx.x, gridDim.x, n_qt, bh, qt);
  } else {
    const int logical = xcd_logical_id(blockIdx.x, gridDim.x);
    bh = logical / n_qt;
    qt = logical - bh * n_qt;
  }
    run_tile(bh, qt, false, -1, 0);
  }
}


template <class Cf, bool CAUSAL, int EMU16, bool PACKED>
hipError_t launch_stream_cfg(const FwdArgs& a, hipStream_t stream) {
  constexpr int BM = Cf::BM;
  const int n_qt = (a.Nq + BM - 1) / BM;
  const long long grid = (long long)a.B * a.H * n_qt;
  hipLaunchKernelGGL((fwd_bf16_stream_kernel<Cf, CAUSAL, EMU16, PACKED>), dim3((unsigned)grid), dim3(Cf::THREADS), 0,
                     stream, (const __bf16*)a.q, (const __bf16*)a.k, (const __bf16*)a.v, (__bf16*)a.o, a.lse, a.stats,
                     a.H, a.Nq, a.Nk, n_qt, a.scale_log2, a.tau, a.bottom_right, a.cu_q, a.cu_k, a.total_q,
                     a.total_k, SplitPlan{}, nullptr);
  return hipGetLastError();
}

// A d = 128 launch with at most one 128-row workgroup per CU leaves the CUs
// it uses with little work each. There the ping-pong kernel takes key
// parities: waves w and w + RW own the same rows and split every key tile, so
// a workgroup covers fewer rows and its chain of tiles is shorter, and the
// two groups still alternate MFMA and softmax phases on every SIMD. With
// 64-row workgroups and four parities when even those number at most one per
// CU (the launch then fills every CU and a wave walks a quarter of a row's
// keys), else 128-row workgroups and two parities. Hardware exp2 only;
// counting launches keep one parity, whose per-row tile sequence is the plain
// recurrence.
constexpr long long kParityMaxWgs = 256;
template <bool CAUSAL, int EMU16, bool PACKED, int KPAR>
hipError_t launch_parity(const FwdArgs& a, hipStream_t stream) {
  constexpr int BM = 256 / KPAR;
  const int n_qt = (a.Nq + BM - 1) / BM;  // a.Nq: the longest sequence for packed batches
  const long long tiles = (long long)a.B * a.H * n_qt;
  hipLaunchKernelGGL((fwd_bf16_kernel<128, CAUSAL, EMU16, PACKED, false, KPAR>), dim3((unsigned)tiles), dim3(512), 0,
                     stream, (const __bf16*)a.q, (const __bf16*)a.k, (const __bf16*)a.v, (__bf16*)a.o, a.lse, a.stats,
                     a.H, a.Nq, a.Nk, n_qt, a.scale_log2, a.tau, a.bottom_right, a.cu_q, a.cu_k, a.total_q, a.total_k,
                     (int)tiles);
  return hipGetLastError();
}
template <int D, bool CAUSAL, int EMU16, bool PACKED>
hipError_t launch_stream(const FwdArgs& a, hipStream_t stream) {
  return launch_stream_cfg<StreamCfg<D>, CAUSAL, EMU16, PACKED>(a, stream);
}

template <int D, bool CAUSAL, int EMU16, bool PACKED>
hipError_t launch_k(const FwdArgs& a, hipStream_t stream) {
  constexpr int BM = Cfg<D, 64, 8>::BM;
  const int n_qt = (a.Nq + BM - 1) / BM;  // a.Nq: the longest sequence for packed batches
  const long long n_bh = (long long)a.B * a.H;
  const long long tiles = n_bh * n_qt;
  // Dense launches of at least two tiles per CU whose heads split evenly over
  // the XCDs run persistent: one workgroup per CU loops over its tiles (each
  // workgroup that ends and the next that starts on its CU cost ~2.9 us of
  // dispatch between them, measured, next to ~100 us of work per tile).
  // (d = 128 only: at d = 192 the loop's live state spills.)
  if constexpr (D == 128 && !PACKED && kPingPongPersist) {
    if (n_bh % 8 == 0 && tiles >= 2 * kPingPongPersistWgs && tiles <= 0x7FFFFFFF) {
      hipLaunchKernelGGL((fwd_bf16_kernel<D, CAUSAL, EMU16, false, true>), dim3(kPingPongPersistWgs), dim3(512), 0,
                         stream, (const __bf16*)a.q, (const __bf16*)a.k, (const __bf16*)a.v, (__bf16*)a.o, a.lse,
                         a.stats, a.H, a.Nq, a.Nk, n_qt, a.scale_log2, a.tau, a.bottom_right, a.cu_q, a.cu_k,
                         a.total_q, a.total_k, (int)tiles);
      return hipGetLastError();
    }
  }
  hipLaunchKernelGGL((fwd_bf16_kernel<D, CAUSAL, EMU16, PACKED, false>), dim3((unsigned)tiles), dim3(512), 0, stream,
                     (const __bf16*)a.q, (const __bf16*)a.k, (const __bf16*)a.v, (__bf16*)a.o, a.lse, a.stats, a.H,
                     a.Nq, a.Nk, n_qt, a.scale_log2, a.tau, a.bottom_right, a.cu_q, a.cu_k, a.total_q, a.total_k,
                     (int)tiles);
  return hipGetLastError();
}

// d = 128 and 192 run the ping-pong kernel, except causal launches with
// fewer than one 256-row workgroup per CU (B * H * ceil(Nq / 256) < 256),
// where the streaming kernel's 128-row workgroups spread the short launch
// wider. Measured (B4 H16 N4096, TFLOP/s, ping-pong vs streaming): d = 128
// 1137 vs ~1050 non-causal, 1017 vs 987 causal; d = 192 1233 vs 1017 and 1078
// vs 952; causal B2 H8 N1024 d128 31.8 vs 31.2 us. Small d = 128 launches
// (hardware exp2, not counting) run the ping-pong kernel's key parities
// instead, causal or not. d = 64 stays on the streaming kernel (faster
// there), d = 256 too (the ping-pong kernel's O and Q operands alone take 192
// of its 256 registers).
constexpr long long kPingPongCausalMinTiles = 256;
template <int D, bool CAUSAL, int EMU16>
hipError_t launch(const FwdArgs& a, hipStream_t stream) {
  if constexpr (D == 128 && EMU16 == 0) {
    if (!a.stats) {
      const long long bh = (long long)a.B * a.H;
      if (bh * ((a.Nq + 63) / 64) <= kParityMaxWgs)
        return a.cu_q ? launch_parity<CAUSAL, EMU16, true, 4>(a, stream)
                      : launch_parity<CAUSAL, EMU16, false, 4>(a, stream);
      if (bh * ((a.Nq + 127) / 128) <= kParityMaxWgs)
        return a.cu_q ? launch_parity<CAUSAL, EMU16, true, 2>(a, stream)
                      : launch_parity<CAUSAL, EMU16, false, 2>(a, stream);
    }
  }
  bool pingpong = D == 128 || D == 192;
  if (CAUSAL && pingpong) pingpong = (long long)a.B * a.H * ((a.Nq + 255) / 256) >= kPingPongCausalMinTiles;
  if constexpr (D == 128 || D == 192) {
    if (pingpong)
      return a.cu_q ? launch_k<D, CAUSAL, EMU16, true>(a, stream) : launch_k<D, CAUSAL, EMU16, false>(a, stream);
  }
  return a.cu_q ? launch_stream<D, CAUSAL, EMU16, true>(a, stream) : launch_stream<D, CAUSAL, EMU16, false>(a, stream);
}

template <int D, bool CAUSAL>
hipError_t launch_mode(const FwdArgs& a, hipStream_t stream) {
  switch (a.emu16) {
    case 0: return launch<D, CAUSAL, 0>(a, stream);
    case 1: return launch<D, CAUSAL, 1>(a, stream);
    case 2: return launch<D, CAUSAL, 2>(a, stream);
    case 3: return launch<D, CAUSAL, 3>(a, stream);
    case 4: return launch<D, CAUSAL, 4>(a, stream);
    case 8: return launch<D, CAUSAL, 8>(a, stream);
    case 16: return launch<D, CAUSAL, 16>(a, stream);
    case kEmuDeg4: return launch<D, CAUSAL, kEmuDeg4>(a, stream);
    case kEmuDeg5: return launch<D, CAUSAL, kEmuDeg5>(a, stream);
    default: return hipErrorInvalidValue;
  }
}

}  // namespace

bool emu16_supported(int emu16) {
  return emu16 == 0 || emu16 == 1 || emu16 == 2 || emu16 == 3 || emu16 == 4 || emu16 == 8 || emu16 == 16 ||
         emu16 == kEmuDeg4 || emu16 == kEmuDeg5;
}

hipError_t launch_fwd_bf16(const FwdArgs& a, hipStream_t stream) {
  if (a.d == 128) return a.causal ? launch_mode<128, true>(a, stream) : launch_mode<128, false>(a, stream);
  if (a.d == 64) return a.causal ? launch_mode<64, true>(a, stream) : launch_mode<64, false>(a, stream);
  if (a.d == 192) return a.causal ? launch_mode<192, true>(a, stream) : launch_mode<192, false>(a, stream);
  if (a.d == 256) return a.causal ? launch_mode<256, true>(a, stream) : launch_mode<256, false>(a, stream);
  return hipErrorInvalidValue;
}

}  // namespace attn
