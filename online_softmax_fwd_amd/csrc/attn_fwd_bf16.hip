// attn_fwd_bf16.hip -- bf16 attention forward for gfx950 (MI355X).
//
// A workgroup of NW waves owns 32*NW query rows of one (batch, head); each
// wave owns 32 rows. K and V stream through LDS in BN-key tiles, two stages
// deep; per row the wave keeps a running max m (raw score units), a
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
//                         changes which blocks contribute"); tiles wholly above
//                         the diagonal are never loaded.
//   lagging max           "FlashAttention-4's Softmax Tricks", section
//                         "Conditional rescaling, and when it's exact": keep the
//                         stale max while (m_old - m_new) * scale_log2 >= -tau,
//                         else commit and rescale O and l by that power of two;
//                         the O rescale is a wave-uniform branch.
//   P = 2^(S*c - m*c)     one FMA then exp2 (the exp2 fold of "Flash Attention 4
//                         -- the algorithm and the two-MMA problem", section "The
//                         exp2 trick"): hardware, software, or a fixed mix
//   l = alpha*l + sum P   from the float32 P, an in-lane partial per half
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
#include "attn_device.h"
#include "attn_internal.h"

namespace attn {
namespace {

typedef short shortx4 __attribute__((ext_vector_type(4)));
typedef __attribute__((address_space(3))) void lds_void;
typedef __attribute__((address_space(3))) shortx4 lds_shortx4;

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
  static_assert(D == 64 || D == 128, "head dim");
};

// Swizzles (16-byte chunk position of logical chunk c in row r is c ^ f(r)).
// K reads touch one chunk of 16 rows per 16-lane group: f_K makes those 16
// rows land on 16 different bank groups. V transpose reads touch 4 chunks of
// 8 rows per instruction: f_V spreads them so each bank is hit exactly twice
// (512 bytes, the minimum of two passes).
template <int D>
__device__ __forceinline__ int swz_k(int r) { return D == 128 ? (r & 15) : ((r >> 1) & 7); }
template <int D>
__device__ __forceinline__ int swz_v(int r) { return D == 128 ? 4 * (r & 3) : 4 * ((r >> 1) & 1); }

// A-operand row m of the S^T MFMA reads key key_of_row(m) of its 32-key
// block. With the 32x32 output layout (lane half h, element j <-> row 8*(j/4)
// + 4*h + j%4), this leaves keys 8h..8h+7 in elements 0..7 and keys
// 16+8h..16+8h+7 in elements 8..15 of each lane.
__device__ __forceinline__ int key_of_row(int m) {
  const int g = m >> 3, h = (m >> 2) & 1, r = m & 3;
  return ((g >> 1) << 4) | (h << 3) | ((g & 1) << 2) | r;
}

template <class C, bool CAUSAL, int EMU16>
struct Body {
  // per-lane constants
  int lane, wave, hh, l32;
  int qi, qw0;
  uint32_t koff[C::D / 16];   // K operand read offsets, one per 16-wide d step
  uint32_t voff[C::D / 32];   // V transpose read offsets, one per 32-wide d block
  uint32_t kld[C::LOADS];     // global byte offsets of this lane's K chunks within a tile
  uint32_t vld[C::LOADS];
  __amdgpu_buffer_rsrc_t rk, rv;

  __device__ __forceinline__ void issue_loads(int t, char* ks, char* vs) {
    const uint32_t soff = (uint32_t)t * C::TILE;
#pragma unroll
    for (int i = 0; i < C::LOADS; ++i) {
      const int j = wave + C::NW * i;
      __builtin_amdgcn_raw_ptr_buffer_load_lds(rk, (lds_void*)(ks + 1024 * j), 16, kld[i], soff, 0, 0);
      __builtin_amdgcn_raw_ptr_buffer_load_lds(rv, (lds_void*)(vs + 1024 * j), 16, vld[i], soff, 0, 0);
    }
  }
};

__device__ __forceinline__ void wait_own_loads() { asm volatile("s_waitcnt vmcnt(0)" ::: "memory"); }

template <int D, int BN, int NW, bool CAUSAL, int EMU16>
__global__ __attribute__((amdgpu_flat_work_group_size(64 * NW, 64 * NW), amdgpu_waves_per_eu(2, 2)))
void fwd_bf16_kernel(const __bf16* __restrict__ Q, const __bf16* __restrict__ K, const __bf16* __restrict__ V,
                     __bf16* __restrict__ O, float* __restrict__ LSE, unsigned long long* __restrict__ stats,
                     int H, int Nq, int Nk, int n_qt, float c, float tau) {
  using C = Cfg<D, BN, NW>;
  __shared__ __attribute__((aligned(1024))) char k0s[C::TILE];
  __shared__ __attribute__((aligned(1024))) char v0s[C::TILE];
  __shared__ __attribute__((aligned(1024))) char k1s[C::TILE];
  __shared__ __attribute__((aligned(1024))) char v1s[C::TILE];

  Body<C, CAUSAL, EMU16> bd;
  const int tid = threadIdx.x;
  bd.lane = tid & 63;
  bd.wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  bd.hh = bd.lane >> 5;
  bd.l32 = bd.lane & 31;
  const int lane = bd.lane, hh = bd.hh, l32 = bd.l32;

  const int logical = xcd_logical_id(blockIdx.x, gridDim.x);
  const int bh = logical / n_qt;
  int qt = logical - bh * n_qt;
  if (CAUSAL) qt = n_qt - 1 - qt;  // longest rows first
  const int q0 = qt * C::BM;
  const int qw0 = q0 + bd.wave * 32;
  const int qi = qw0 + l32;
  const size_t qbase = (size_t)bh * Nq * D;
  const size_t kbase = (size_t)bh * Nk * D;

  // ---- per-lane constants --------------------------------------------------
  {
    const int krow = key_of_row(l32);
#pragma unroll
    for (int s = 0; s < D / 16; ++s)
      bd.koff[s] = krow * C::RB + 16 * ((2 * s + hh) ^ swz_k<D>(krow));
    const int L = lane & 15, gidx = (lane >> 4) & 1;
    const int vr = 8 * hh + (L >> 2);
#pragma unroll
    for (int db = 0; db < D / 32; ++db) {
      const int cch = 4 * db + 2 * gidx + ((L & 3) >> 1);
      bd.voff[db] = vr * C::RB + 16 * (cch ^ swz_v<D>(vr)) + 8 * (L & 1);
    }
#pragma unroll
    for (int i = 0; i < C::LOADS; ++i) {
      const int pos = 64 * (bd.wave + NW * i) + lane;
      const int r = pos / C::CH, p = pos % C::CH;
      bd.kld[i] = r * C::RB + 16 * (p ^ swz_k<D>(r));
      bd.vld[i] = r * C::RB + 16 * (p ^ swz_v<D>(r));
    }
    const int nrec = Nk * C::RB;
    bd.rk = __builtin_amdgcn_make_buffer_rsrc((void*)(K + kbase), (short)0, nrec, 0x00020000);
    bd.rv = __builtin_amdgcn_make_buffer_rsrc((void*)(V + kbase), (short)0, nrec, 0x00020000);
  }

  // ---- Q as the B operand: lane (h, n) holds Q[n][16s + 8h .. +8] -----------
  bf16x8 qf[D / 16];
  {
    const bool ok = qi < Nq;
    const __bf16* qp = Q + qbase + (size_t)(ok ? qi : 0) * D + 8 * hh;
#pragma unroll
    for (int s = 0; s < D / 16; ++s) {
      const u32x4 w = ok ? *(const u32x4*)(qp + 16 * s) : u32x4{0u, 0u, 0u, 0u};
      qf[s] = __builtin_bit_cast(bf16x8, w);
    }
  }

  const int kend = CAUSAL ? min(Nk, q0 + C::BM) : Nk;
  const int n_kt = (kend + BN - 1) / BN;

  floatx16 o[D / 32];
#pragma unroll
  for (int i = 0; i < D / 32; ++i) o[i] = floatx16{};
  float m_run = kNegInf;  // running max, raw score units
  float l_run = 0.0f;     // running denominator over this lane's half of the keys
  unsigned long long cnt[4] = {0, 0, 0, 0};

  auto compute = [&](int t, const char* ks, const char* vs) {
    const int k0 = t * BN;
    if (CAUSAL && k0 > qw0 + 31) return;  // wave-uniform: every key of the tile is masked

    // S^T = K Q^T
    floatx16 s[C::KB];
#pragma unroll
    for (int kb = 0; kb < C::KB; ++kb) {
      s[kb] = floatx16{};
#pragma unroll
      for (int st = 0; st < D / 16; ++st) {
        const bf16x8 a = *(const bf16x8*)(ks + kb * 32 * C::RB + bd.koff[st]);
        s[kb] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, qf[st], s[kb], 0, 0, 0);
      }
    }

    if ((CAUSAL && k0 + BN - 1 > qw0) || (k0 + BN > Nk)) {
#pragma unroll
      for (int kb = 0; kb < C::KB; ++kb)
#pragma unroll
        for (int j = 0; j < 16; ++j) {
          const int key = k0 + kb * 32 + 16 * (j >> 3) + 8 * hh + (j & 7);
          if (key >= Nk || (CAUSAL && key > qi)) s[kb][j] = kNegInf;
        }
    }

    float mx = kNegInf;
#pragma unroll
    for (int kb = 0; kb < C::KB; ++kb)
#pragma unroll
      for (int j = 0; j < 16; ++j) mx = __builtin_fmaxf(mx, s[kb][j]);
    mx = max_halves(mx);

    const float m_new = __builtin_fmaxf(m_run, mx);
    const float acc = (m_run - m_new) * c;  // -inf on a row's first block
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
    float rs = 0.0f;
#pragma unroll
    for (int kb = 0; kb < C::KB; ++kb)
#pragma unroll
      for (int j = 0; j < 16; ++j) {
        const float p = exp2_sel<EMU16>(__builtin_fmaf(s[kb][j], c, -mc), j);
        s[kb][j] = p;
        rs += p;
      }
    l_run = l_run * alpha + rs;

    bf16x8 pb[C::KB][2];
#pragma unroll
    for (int kb = 0; kb < C::KB; ++kb)
#pragma unroll
      for (int cc = 0; cc < 2; ++cc)
#pragma unroll
        for (int e = 0; e < 8; ++e) pb[kb][cc][e] = (__bf16)s[kb][8 * cc + e];

    // O^T += V^T P^T
#pragma unroll
    for (int db = 0; db < D / 32; ++db)
#pragma unroll
      for (int kb = 0; kb < C::KB; ++kb)
#pragma unroll
        for (int cc = 0; cc < 2; ++cc) {
          const char* vp = vs + bd.voff[db] + (kb * 32 + 16 * cc) * C::RB;
          const shortx4 lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_shortx4*)(vp));
          const shortx4 hi = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_shortx4*)(vp + 4 * C::RB));
          const bf16x8 a = __builtin_bit_cast(
              bf16x8, u32x4{__builtin_bit_cast(u32x2, lo)[0], __builtin_bit_cast(u32x2, lo)[1],
                            __builtin_bit_cast(u32x2, hi)[0], __builtin_bit_cast(u32x2, hi)[1]});
          o[db] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, pb[kb][cc], o[db], 0, 0, 0);
        }
  };

  bd.issue_loads(0, k0s, v0s);
  wait_own_loads();
  __syncthreads();
  for (int t = 0; t < n_kt; t += 2) {
    if (t + 1 < n_kt) bd.issue_loads(t + 1, k1s, v1s);
    compute(t, k0s, v0s);
    wait_own_loads();
    __syncthreads();
    if (t + 1 >= n_kt) break;
    if (t + 2 < n_kt) bd.issue_loads(t + 2, k0s, v0s);
    compute(t + 1, k1s, v1s);
    wait_own_loads();
    __syncthreads();
  }

  // ---- epilogue: O / l, LSE -------------------------------------------------
  const float l_tot = sum_halves(l_run);
  const float inv = 1.0f / l_tot;
  if (qi < Nq) {
    __bf16* op = O + qbase + (size_t)qi * D + 4 * hh;
#pragma unroll
    for (int db = 0; db < D / 32; ++db)
#pragma unroll
      for (int g = 0; g < 4; ++g) {
        bf16x4 w;
#pragma unroll
        for (int r = 0; r < 4; ++r) w[r] = (__bf16)(o[db][4 * g + r] * inv);
        *(bf16x4*)(op + 32 * db + 8 * g) = w;
      }
    if (hh == 0) LSE[(size_t)bh * Nq + qi] = (m_run * c + __builtin_log2f(l_tot)) * 0.693147180559945309f;
  }
  if (stats && lane == 0) {
#pragma unroll
    for (int i = 0; i < 4; ++i) atomicAdd(stats + i, cnt[i]);
  }
}

// Tile shape per head dim: waves per workgroup and keys per tile.
template <int D> struct Shape;
template <> struct Shape<128> { static constexpr int NW = 4, BN = 64; };
template <> struct Shape<64> { static constexpr int NW = 4, BN = 64; };

template <int D, bool CAUSAL, int EMU16>
hipError_t launch(const FwdArgs& a, hipStream_t stream) {
  constexpr int NW = Shape<D>::NW, BN = Shape<D>::BN;
  constexpr int BM = 32 * NW;
  const int n_qt = (a.Nq + BM - 1) / BM;
  const long long grid = (long long)a.B * a.H * n_qt;
  hipLaunchKernelGGL((fwd_bf16_kernel<D, BN, NW, CAUSAL, EMU16>), dim3((unsigned)grid), dim3(64 * NW), 0, stream,
                     (const __bf16*)a.q, (const __bf16*)a.k, (const __bf16*)a.v, (__bf16*)a.o, a.lse, a.stats, a.H,
                     a.Nq, a.Nk, n_qt, a.scale_log2, a.tau);
  return hipGetLastError();
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
    default: return hipErrorInvalidValue;
  }
}

}  // namespace

bool emu16_supported(int emu16) {
  return emu16 == 0 || emu16 == 1 || emu16 == 2 || emu16 == 3 || emu16 == 4 || emu16 == 8 || emu16 == 16;
}

hipError_t launch_fwd_bf16(const FwdArgs& a, hipStream_t stream) {
  if (a.d == 128) return a.causal ? launch_mode<128, true>(a, stream) : launch_mode<128, false>(a, stream);
  if (a.d == 64) return a.causal ? launch_mode<64, true>(a, stream) : launch_mode<64, false>(a, stream);
  return hipErrorInvalidValue;
}

}  // namespace attn
