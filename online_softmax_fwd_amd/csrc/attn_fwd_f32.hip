// attn_fwd_f32.hip -- float32 attention forward for gfx950.
//
// Same tiling and softmax stage as the bf16 kernel (4 waves x 32 query rows,
// 64-key tiles double-buffered through LDS, S^T with one query per lane, the
// lagging-max rule, deferred normalisation); the contractions use
// v_mfma_f32_32x32x2_f32, which takes one float per lane per k-step, so V
// needs no transpose: the PV A operand is one float of a V row per lane.
//
// K-step assignment: in S^T = K Q^T lane half h covers head dimensions
// h*D/2 .. h*D/2 + D/2 - 1 (so a lane reads four consecutive k-steps of K
// with one 16-byte LDS load); in O^T += V^T P^T k-step j of a 32-key block is
// the key the lane's S^T element j holds.
#include "attn_device.h"
#include "attn_internal.h"

namespace attn {
namespace {

constexpr int kWaves = 4;
constexpr int kThreads = 64 * kWaves;
constexpr int kQW = 32;
constexpr int kBM = kQW * kWaves;
constexpr int kBN = 64;
constexpr int kKB = kBN / 32;

template <int D>
struct GeoF {
  static constexpr int stride = D + 4;  // floats; 16 consecutive rows hit 16 bank groups
  static constexpr int tileElems = kBN * stride;
  static constexpr int bufElems = 2 * tileElems;  // K then V
  static constexpr int chunks = kBN * D / 4 / kThreads;  // 16-byte chunks per thread per tensor
};

__device__ __forceinline__ int key_of_row_f(int m) {
  const int g = m >> 3, h = (m >> 2) & 1, r = m & 3;
  return ((g >> 1) << 4) | (h << 3) | ((g & 1) << 2) | r;
}

template <int D, bool CAUSAL, int EMU16, bool PACKED>
__global__ __attribute__((amdgpu_flat_work_group_size(kThreads, kThreads)))
void fwd_f32_kernel(const float* __restrict__ Q, const float* __restrict__ K, const float* __restrict__ V,
                    float* __restrict__ O, float* __restrict__ LSE, unsigned long long* __restrict__ stats,
                    int H, int Nq_dense, int Nk_dense, int n_qt, float c, float tau, int bottom_right,
                    const int* __restrict__ cu_q, const int* __restrict__ cu_k, int total_q, int total_k) {
  using G = GeoF<D>;
  __shared__ __attribute__((aligned(16))) float smem[2 * G::bufElems];

  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int hh = lane >> 5, l32 = lane & 31;
  int bh, qt;
  if (CAUSAL) {
    causal_tile_of(blockIdx.x, gridDim.x, n_qt, bh, qt);
  } else {
    const int logical = xcd_logical_id(blockIdx.x, gridDim.x);
    bh = logical / n_qt;
    qt = logical - bh * n_qt;
  }
  const int q0 = qt * kBM;
  const int qw0 = q0 + wave * kQW;
  const int qi = qw0 + l32;
  const Slice sl = slice_of(bh, H, D, Nq_dense, Nk_dense, PACKED ? cu_q : nullptr, cu_k, total_q, total_k);
  const int Nq = sl.Nq, Nk = sl.Nk;
  if (PACKED && q0 >= Nq) return;  // a query tile past this sequence's end
  const size_t qbase = sl.qbase, kbase = sl.kbase;
  const int diag = bottom_right ? Nk - Nq : 0;

  float qf[D / 2];
  {
    const bool ok = qi < Nq;
    const float* qp = Q + qbase + (size_t)(ok ? qi : 0) * sl.rs + (D / 2) * hh;
#pragma unroll
    for (int s = 0; s < D / 2; s += 4) {
      const floatx4 w = ok ? *(const floatx4*)(qp + s) : floatx4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int e = 0; e < 4; ++e) qf[s + e] = w[e];
    }
  }

  // causal: key j is hidden from query i when j > i + diag
  const int kend = CAUSAL ? min(Nk, q0 + kBM + diag) : Nk;
  const int n_kt = (kend + kBN - 1) / kBN;

  floatx4 kreg[G::chunks], vreg[G::chunks];
  auto load_tile = [&](int t) {
    const int k0 = t * kBN;
#pragma unroll
    for (int i = 0; i < G::chunks; ++i) {
      const int ch = tid + i * kThreads;
      const int row = ch / (D / 4), col = ch % (D / 4);
      const bool ok = k0 + row < Nk;
      const size_t off = kbase + (size_t)(k0 + row) * sl.rs + col * 4;
      kreg[i] = ok ? *(const floatx4*)(K + off) : floatx4{0.f, 0.f, 0.f, 0.f};
      vreg[i] = ok ? *(const floatx4*)(V + off) : floatx4{0.f, 0.f, 0.f, 0.f};
    }
  };
  auto store_tile = [&](int buf) {
    float* ks = smem + buf * G::bufElems;
    float* vs = ks + G::tileElems;
#pragma unroll
    for (int i = 0; i < G::chunks; ++i) {
      const int ch = tid + i * kThreads;
      const int row = ch / (D / 4), col = ch % (D / 4);
      *(floatx4*)(ks + row * G::stride + col * 4) = kreg[i];
      *(floatx4*)(vs + row * G::stride + col * 4) = vreg[i];
    }
  };

  floatx16 o[D / 32];
#pragma unroll
  for (int i = 0; i < D / 32; ++i) o[i] = floatx16{};
  float m_run = kNegInf, l_run = 0.0f;
  unsigned long long cnt[4] = {0, 0, 0, 0};
  const int krow = key_of_row_f(l32);

  load_tile(0);
  store_tile(0);
  __syncthreads();

  for (int t = 0; t < n_kt; ++t) {
    const int buf = t & 1;
    if (t + 1 < n_kt) load_tile(t + 1);
    const int k0 = t * kBN;
    const bool active = !CAUSAL || k0 <= qw0 + kQW - 1 + diag;
    if (active) {
      const float* ks = smem + buf * G::bufElems;
      const float* vs = ks + G::tileElems;
      floatx16 s[kKB];
#pragma unroll
      for (int kb = 0; kb < kKB; ++kb) {
        s[kb] = floatx16{};
        const float* kp = ks + (kb * 32 + krow) * G::stride + (D / 2) * hh;
#pragma unroll
        for (int st = 0; st < D / 2; st += 4) {
          const floatx4 a = *(const floatx4*)(kp + st);
#pragma unroll
          for (int e = 0; e < 4; ++e)
            s[kb] = __builtin_amdgcn_mfma_f32_32x32x2f32(a[e], qf[st + e], s[kb], 0, 0, 0);
        }
      }
      const bool need_mask = (CAUSAL && k0 + kBN - 1 > qw0 + diag) || (k0 + kBN > Nk);
      if (need_mask) {
#pragma unroll
        for (int kb = 0; kb < kKB; ++kb)
#pragma unroll
          for (int j = 0; j < 16; ++j) {
            const int key = k0 + kb * 32 + 16 * (j >> 3) + 8 * hh + (j & 7);
            if (key >= Nk || (CAUSAL && key > qi + diag)) s[kb][j] = kNegInf;
          }
      }
      float mx = kNegInf;
#pragma unroll
      for (int kb = 0; kb < kKB; ++kb)
#pragma unroll
        for (int j = 0; j < 16; ++j) mx = __builtin_fmaxf(mx, s[kb][j]);
      mx = max_halves(mx);
      const float m_new = __builtin_fmaxf(m_run, mx);
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
#pragma unroll
      for (int db = 0; db < D / 32; ++db)
#pragma unroll
        for (int kb = 0; kb < kKB; ++kb)
#pragma unroll
          for (int j = 0; j < 16; ++j) {
            const int key = kb * 32 + 16 * (j >> 3) + 8 * hh + (j & 7);
            const float a = vs[key * G::stride + 32 * db + l32];
            o[db] = __builtin_amdgcn_mfma_f32_32x32x2f32(a, s[kb][j], o[db], 0, 0, 0);
          }
    }
    if (t + 1 < n_kt) store_tile(buf ^ 1);
    __syncthreads();
  }

  const float l_tot = sum_halves(l_run);
  const float inv = l_tot > 0.0f ? 1.0f / l_tot : 0.0f;  // a row that saw no key: O = 0, LSE = -inf
  if (qi < Nq) {
    float* op = O + qbase + (size_t)qi * sl.rs + 4 * hh;
#pragma unroll
    for (int db = 0; db < D / 32; ++db)
#pragma unroll
      for (int g = 0; g < 4; ++g) {
        floatx4 w;
#pragma unroll
        for (int r = 0; r < 4; ++r) w[r] = o[db][4 * g + r] * inv;
        *(floatx4*)(op + 32 * db + 8 * g) = w;
      }
    if (hh == 0) LSE[sl.lse + qi] = (m_run * c + __builtin_log2f(l_tot)) * 0.693147180559945309f;
  }
  if (stats && lane == 0) {
#pragma unroll
    for (int i = 0; i < 4; ++i) atomicAdd(stats + i, cnt[i]);
  }
}

template <int D, bool CAUSAL, int EMU16, bool PACKED>
hipError_t launch_k(const FwdArgs& a, hipStream_t stream) {
  const int n_qt = (a.Nq + kBM - 1) / kBM;
  const long long grid = (long long)a.B * a.H * n_qt;
  hipLaunchKernelGGL((fwd_f32_kernel<D, CAUSAL, EMU16, PACKED>), dim3((unsigned)grid), dim3(kThreads), 0, stream,
                     (const float*)a.q, (const float*)a.k, (const float*)a.v, (float*)a.o, a.lse, a.stats,
                     a.H, a.Nq, a.Nk, n_qt, a.scale_log2, a.tau, a.bottom_right, a.cu_q, a.cu_k, a.total_q, a.total_k);
  return hipGetLastError();
}

template <int D, bool CAUSAL, int EMU16>
hipError_t launch(const FwdArgs& a, hipStream_t stream) {
  return a.cu_q ? launch_k<D, CAUSAL, EMU16, true>(a, stream) : launch_k<D, CAUSAL, EMU16, false>(a, stream);
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

hipError_t launch_fwd_f32(const FwdArgs& a, hipStream_t stream) {
  if (a.d == 128) return a.causal ? launch_mode<128, true>(a, stream) : launch_mode<128, false>(a, stream);
  if (a.d == 64) return a.causal ? launch_mode<64, true>(a, stream) : launch_mode<64, false>(a, stream);
  return hipErrorInvalidValue;
}

}  // namespace attn
