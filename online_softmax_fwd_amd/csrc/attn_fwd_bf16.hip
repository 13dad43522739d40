// attn_fwd_bf16.hip -- bf16 attention forward for gfx950 (MI355X).
//
// One workgroup = 4 waves = 128 query rows of one (batch, head); each wave
// owns 32 rows. The kernel streams K and V in 64-key tiles through LDS and
// keeps per row a running max m (raw score units), a denominator l and a
// 32 x d float accumulator, so S and P never reach memory. Per tile and wave:
//
//   S^T = K_tile Q^T      v_mfma_f32_32x32x16_bf16, A = K rows from LDS, B = Q
//                         from registers. The output puts one query per lane
//                         (lane % 32) and 16 keys per lane, so the row max and
//                         row sum are in-lane plus one exchange between the two
//                         32-lane halves.
//   mask                  only on tiles that straddle the causal diagonal or
//                         the end of the keys (the causal rule of "Lecture 2 --
//                         Online Softmax and Numerical Correctness", section
//                         "Causal masking just changes which blocks
//                         contribute"; tiles above the diagonal are skipped)
//   lagging max           "FlashAttention-4's Softmax Tricks", section
//                         "Conditional rescaling, and when it's exact": keep
//                         the stale max while (m_old - m_new) * scale_log2 >=
//                         -tau; otherwise commit it and rescale O and l by
//                         2^((m_old - m_new) * scale_log2). The O rescale is a
//                         wave-uniform branch taken if any row commits.
//   P = 2^(S*c - m*c)     one FMA then exp2 (the exp2 fold of "Flash
//                         Attention 4 -- the algorithm and the two-MMA
//                         problem", section "The exp2 trick"), hardware,
//                         software or a fixed per-lane mix of the two
//   l = alpha*l + sum P   from the float32 P, in-lane partial per half
//   O^T += V^T P^T        v_mfma_f32_32x32x16_bf16, A = V^T from LDS (V is
//                         transposed on its way into LDS), B = P in bf16 taken
//                         straight from the S^T registers: the S^T output
//                         layout already is the B-operand layout, because the
//                         K rows feeding S^T are permuted so that each lane
//                         half holds 8 consecutive keys per 16-key step.
//
// The epilogue divides by l once per row (deferred normalisation, same
// lesson, section "Deferred normalization") and writes LSE = ln2 * (m*c +
// log2 l) ("Lecture 2", section "The classical safe softmax").
//
// K/V tiles are double-buffered: the global loads of tile t+1 are issued
// before the math of tile t and written to the other LDS buffer after it.
#include "attn_device.h"
#include "attn_internal.h"

namespace attn {
namespace {

constexpr int kWaves = 4;
constexpr int kThreads = 64 * kWaves;
constexpr int kQW = 32;             // query rows per wave
constexpr int kBM = kQW * kWaves;   // query rows per workgroup
constexpr int kBN = 64;             // keys per tile
constexpr int kKB = kBN / 32;       // 32-key MFMA blocks per tile

template <int D>
struct Geo {
  static constexpr int kStride = D + 8;      // K tile row, bf16 (16 B pad: 16 rows hit 16 bank groups)
  static constexpr int vStride = kBN + 8;    // V^T tile row, bf16 (same reason)
  static constexpr int kElems = kBN * kStride;
  static constexpr int vElems = D * vStride;
  static constexpr int bufElems = kElems + vElems;
  static constexpr int kChunks = kBN * D / 8 / kThreads;  // 16-byte K chunks per thread
  static constexpr int vRows = kBN * D / 8 / kThreads;    // V rows per thread (8 columns each)
  static constexpr int vGroups = kBN / vRows;             // row groups per tile
  static_assert(kChunks >= 1 && vRows >= 2, "tile does not split over the workgroup");
};

// A-operand row m of the S^T MFMA reads key key_of_row(m) of its 32-key block.
// With the 32x32 output layout (lane half h, element j <-> row 8*(j/4) + 4*h +
// j%4), this puts keys 8h..8h+7 in elements 0..7 and keys 16+8h..16+8h+7 in
// elements 8..15 of every lane, which is how the PV MFMA wants P.
__device__ __forceinline__ int key_of_row(int m) {
  const int g = m >> 3, h = (m >> 2) & 1, r = m & 3;
  return ((g >> 1) << 4) | (h << 3) | ((g & 1) << 2) | r;
}

__device__ __forceinline__ u32x4 zero4() { return u32x4{0u, 0u, 0u, 0u}; }

template <int D, bool CAUSAL, int EMU16>
__global__ __attribute__((amdgpu_flat_work_group_size(kThreads, kThreads), amdgpu_waves_per_eu(2, 2)))
void fwd_bf16_kernel(const __bf16* __restrict__ Q, const __bf16* __restrict__ K,
                     const __bf16* __restrict__ V, __bf16* __restrict__ O, float* __restrict__ LSE,
                     unsigned long long* __restrict__ stats, int H, int Nq, int Nk, int n_qt,
                     float c, float tau) {
  using G = Geo<D>;
  __shared__ __attribute__((aligned(16))) __bf16 smem[2 * G::bufElems];

  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int hh = lane >> 5, l32 = lane & 31;
  const int logical = xcd_logical_id(blockIdx.x, gridDim.x);
  const int bh = logical / n_qt;
  int qt = logical - bh * n_qt;
  if (CAUSAL) qt = n_qt - 1 - qt;  // longest rows first
  const int q0 = qt * kBM;
  const int qw0 = q0 + wave * kQW;
  const int qi = qw0 + l32;
  const size_t qbase = (size_t)bh * Nq * D;
  const size_t kbase = (size_t)bh * Nk * D;

  // ---- Q as the B operand: lane (h, n) holds Q[n][16s + 8h .. +8] -----------
  bf16x8 qf[D / 16];
  {
    const bool ok = qi < Nq;
    const __bf16* qp = Q + qbase + (size_t)(ok ? qi : 0) * D + 8 * hh;
#pragma unroll
    for (int s = 0; s < D / 16; ++s) {
      const u32x4 w = ok ? *(const u32x4*)(qp + 16 * s) : zero4();
      qf[s] = __builtin_bit_cast(bf16x8, w);
    }
  }

  const int kend = CAUSAL ? min(Nk, q0 + kBM) : Nk;
  const int n_kt = (kend + kBN - 1) / kBN;

  // ---- global -> register staging of one K/V tile ---------------------------
  u32x4 kreg[G::kChunks];
  u32x4 vreg[G::vRows];
  // V: lane -> (row group gv, 8-column chunk cv) with gv fastest, so the
  // transposed LDS writes of one wave spread over all banks
  const int gv = lane % G::vGroups;
  const int cv = wave * (64 / G::vGroups) + lane / G::vGroups;

  auto load_tile = [&](int t) {
    const int k0 = t * kBN;
    const bool full = k0 + kBN <= Nk;
#pragma unroll
    for (int i = 0; i < G::kChunks; ++i) {
      const int ch = tid + i * kThreads;
      const int row = ch / (D / 8), col = ch % (D / 8);
      kreg[i] = (full || k0 + row < Nk) ? *(const u32x4*)(K + kbase + (size_t)(k0 + row) * D + col * 8)
                                        : zero4();
    }
#pragma unroll
    for (int r = 0; r < G::vRows; ++r) {
      const int row = gv * G::vRows + r;
      vreg[r] = (full || k0 + row < Nk) ? *(const u32x4*)(V + kbase + (size_t)(k0 + row) * D + cv * 8)
                                        : zero4();
    }
  };

  auto store_tile = [&](int buf) {
    __bf16* ks = smem + buf * G::bufElems;
    __bf16* vs = ks + G::kElems;
#pragma unroll
    for (int i = 0; i < G::kChunks; ++i) {
      const int ch = tid + i * kThreads;
      const int row = ch / (D / 8), col = ch % (D / 8);
      *(u32x4*)(ks + row * G::kStride + col * 8) = kreg[i];
    }
    // V^T[cv*8 + e][gv*vRows + r] = V[gv*vRows + r][cv*8 + e]
#pragma unroll
    for (int e = 0; e < 8; ++e) {
      uint32_t h16[G::vRows];
#pragma unroll
      for (int r = 0; r < G::vRows; ++r) h16[r] = (vreg[r][e >> 1] >> (16 * (e & 1))) & 0xFFFFu;
      __bf16* dst = vs + (cv * 8 + e) * G::vStride + gv * G::vRows;
      if constexpr (G::vRows == 4) {
        *(u32x2*)dst = u32x2{h16[0] | (h16[1] << 16), h16[2] | (h16[3] << 16)};
      } else {
        *(uint32_t*)dst = h16[0] | (h16[1] << 16);
      }
    }
  };

  floatx16 o[D / 32];
#pragma unroll
  for (int i = 0; i < D / 32; ++i) o[i] = floatx16{};
  float m_run = kNegInf;  // running max, raw score units
  float l_run = 0.0f;     // running denominator, this lane's half of the keys
  unsigned long long cnt[4] = {0, 0, 0, 0};

  const int krow = key_of_row(l32);

  load_tile(0);
  store_tile(0);
  __syncthreads();

  for (int t = 0; t < n_kt; ++t) {
    const int buf = t & 1;
    if (t + 1 < n_kt) load_tile(t + 1);
    const int k0 = t * kBN;
    const bool active = !CAUSAL || k0 <= qw0 + kQW - 1;  // wave-uniform
    if (active) {
      const __bf16* ks = smem + buf * G::bufElems;
      const __bf16* vs = ks + G::kElems;

      // S^T = K Q^T
      floatx16 s[kKB];
#pragma unroll
      for (int kb = 0; kb < kKB; ++kb) {
        s[kb] = floatx16{};
        const __bf16* kp = ks + (kb * 32 + krow) * G::kStride + 8 * hh;
#pragma unroll
        for (int st = 0; st < D / 16; ++st) {
          const bf16x8 a = *(const bf16x8*)(kp + 16 * st);
          s[kb] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, qf[st], s[kb], 0, 0, 0);
        }
      }

      // mask keys past the end and, under causal, keys after the query
      const bool need_mask = (CAUSAL && k0 + kBN - 1 > qw0) || (k0 + kBN > Nk);
      if (need_mask) {
#pragma unroll
        for (int kb = 0; kb < kKB; ++kb)
#pragma unroll
          for (int j = 0; j < 16; ++j) {
            const int key = k0 + kb * 32 + 16 * (j >> 3) + 8 * hh + (j & 7);
            if (key >= Nk || (CAUSAL && key > qi)) s[kb][j] = kNegInf;
          }
      }

      // row max over the tile
      float mx = kNegInf;
#pragma unroll
      for (int kb = 0; kb < kKB; ++kb)
#pragma unroll
        for (int j = 0; j < 16; ++j) mx = __builtin_fmaxf(mx, s[kb][j]);
      mx = max_halves(mx);

      // lagging max: commit only when the max grew by more than tau (log2 units)
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

      // P = 2^(S*c - m*c), row sum from the float32 P
      const float mc = (m_run > kNegInf) ? m_run * c : 0.0f;
      float rs = 0.0f;
#pragma unroll
      for (int kb = 0; kb < kKB; ++kb)
#pragma unroll
        for (int j = 0; j < 16; ++j) {
          const float p = exp2_sel<EMU16>(__builtin_fmaf(s[kb][j], c, -mc), j);
          s[kb][j] = p;
          rs += p;
        }
      l_run = l_run * alpha + rs;

      // P in bf16, already in B-operand layout
      bf16x8 pb[kKB][2];
#pragma unroll
      for (int kb = 0; kb < kKB; ++kb)
#pragma unroll
        for (int cc = 0; cc < 2; ++cc)
#pragma unroll
          for (int e = 0; e < 8; ++e) pb[kb][cc][e] = (__bf16)s[kb][8 * cc + e];

      // O^T += V^T P^T
#pragma unroll
      for (int db = 0; db < D / 32; ++db) {
        const __bf16* vp = vs + (32 * db + l32) * G::vStride + 8 * hh;
#pragma unroll
        for (int kb = 0; kb < kKB; ++kb)
#pragma unroll
          for (int cc = 0; cc < 2; ++cc) {
            const bf16x8 a = *(const bf16x8*)(vp + kb * 32 + 16 * cc);
            o[db] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, pb[kb][cc], o[db], 0, 0, 0);
          }
      }
    }
    if (t + 1 < n_kt) store_tile(buf ^ 1);
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

template <int D, bool CAUSAL, int EMU16>
hipError_t launch(const FwdArgs& a, hipStream_t stream) {
  const int n_qt = (a.Nq + kBM - 1) / kBM;
  const long long grid = (long long)a.B * a.H * n_qt;
  hipLaunchKernelGGL((fwd_bf16_kernel<D, CAUSAL, EMU16>), dim3((unsigned)grid), dim3(kThreads), 0, stream,
                     (const __bf16*)a.q, (const __bf16*)a.k, (const __bf16*)a.v, (__bf16*)a.o, a.lse,
                     a.stats, a.H, a.Nq, a.Nk, n_qt, a.scale_log2, a.tau);
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
