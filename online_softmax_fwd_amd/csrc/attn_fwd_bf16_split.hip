// attn_fwd_bf16_split.hip -- bf16 attention forward with each row's keys cut
// into chunks that separate workgroups run, then merged exactly.
//
// A launch with few query tiles leaves most of the 256 compute units idle,
// and each busy one runs its tile's whole key range as one chain of
// dependent steps (for B=2 H=8 N=1024 causal: 128 tiles of 128 rows, the
// longest walking all 1024 keys). Cutting the keys of a tile into chunks
// gives one workgroup per (tile, chunk): the chip fills, and the longest chain
// is one chunk. Each chunk's workgroup runs the streaming kernel over its key
// range and leaves its softmax state as a normalised float32 O_k and its
// log-sum-exp L_k (log2 units). A second kernel merges the chunks of a row
// exactly ("Lecture 2 -- Online Softmax and Numerical Correctness", section
// "Combining two blocks exactly": the states of two key ranges combine into
// the state of their union):
//     L = max_k L_k,   w_k = 2^(L_k - L),   O = sum_k w_k O_k / sum_k w_k,
//     LSE = ln 2 * (L + log2 sum_k w_k).
// Tiles whose keys fit one chunk write O and LSE directly and take no part in
// the merge.
#include <mutex>

#include "attn.h"
#include "attn_fwd_bf16_kernels.h"

namespace attn {
namespace {

// Tiles of the split kernel: the streaming kernel's own configuration. A
// four-deep K/V ring was measured as well (per-workgroup timestamps on the
// B=2 H=8 N=1024 causal workload): it does not shorten a workgroup's chain
// of tiles (each 32-key tile is about 0.8 us of one wave's own MFMA and
// softmax work, not DMA waiting) and its 64 KB of LDS fits two workgroups per
// CU instead of three, so 576 workgroups needed a second round.
template <int D>
using SplitCfg = StreamCfg<D>;
// CS threads per float4 of a slot (the split kernel's lane order): float4 f
// of a tile's slots holds row 32 * (f / 64 / (D/8)) + (f % 64) % 32 and four
// columns of it; 256 threads per workgroup, BM * D * CS / 1024 workgroups per
// query tile: workgroup b handles piece b % pieces of tile qt of head bh,
// b / pieces = bh * n_qt + qt. With CS > 1 (rows cut into more chunks than
// one thread folds in one round of loads, e.g. a decoding step) the CS
// adjacent lanes of a float4 fold every CS-th chunk each, and their states
// combine by the same rule across lanes, so the loads of a row's chunks are
// in flight together instead of one group after another.
template <int D, int CS>
__global__ __launch_bounds__(256) void fwd_split_merge_kernel(const float* __restrict__ ws, __bf16* __restrict__ O,
                                                              float* __restrict__ LSE, SplitPlan plan, int n_slots,
                                                              int n_qt, int pieces) {
  const int b = blockIdx.x;
  const int piece = b % pieces;
  const int bq = b / pieces;
  const int qt = bq % n_qt, bh = bq / n_qt;
  const int n = plan.n_chunks(qt);
  if (n <= 1) return;  // written by the split kernel itself
  const int f = piece * (256 / CS) + threadIdx.x / CS;
  const int c0 = threadIdx.x % CS;  // this lane's chunks: c0, c0 + CS, ...
  const int lane = f & 63, i = (f >> 6) % (D / 8), wave = (f >> 6) / (D / 8);
  const int r = 32 * wave + (lane & 31);
  const int row = qt * plan.BM + r;
  if (row >= plan.Nq) return;
  const int col = 32 * (i >> 2) + 8 * (i & 3) + 4 * (lane >> 5);
  int u0 = 0;
  for (int q = 0; q < qt; ++q) u0 += plan.n_chunks(q);
  const size_t slot0 = (size_t)bh * plan.units + u0;
  const size_t slot_f4 = (size_t)plan.BM * D / 4;   // float4s per slot
  const float* lse2 = ws + (size_t)n_slots * plan.BM * D + slot0 * plan.BM + r;
  const floatx4* src = (const floatx4*)ws + slot0 * slot_f4 + f;
  __bf16* op = O + ((size_t)bh * plan.Nq + row) * D + col;
  const bool lse_writer = i == 0 && lane < 32 && c0 == 0;
  // One pass with a running maximum (the same combine, applied a group of G
  // chunks at a time); group g+1 is loaded before group g is folded in, so
  // the loads of two groups are in flight at once.
  constexpr int G = 8;
  float t[2][G];
  floatx4 x[2][G];
  // group position k0 + j is this lane's chunk c0 + CS * (k0 + j)
  const int nl = (n - c0 + CS - 1) / CS;  // chunks of this lane (0 if c0 >= n)
  auto load = [&](int k0, int b) __attribute__((always_inline)) {
#pragma unroll
    for (int j = 0; j < G; ++j) {
      const bool ok = k0 + j < nl;
      const size_t k = (size_t)c0 + (size_t)CS * (ok ? k0 + j : 0);
      t[b][j] = ok ? lse2[k * plan.BM] : kNegInf;
      x[b][j] = ok ? src[k * slot_f4] : floatx4{0.0f, 0.0f, 0.0f, 0.0f};
    }
  };
  float L = kNegInf, wsum = 0.0f;
  floatx4 acc = floatx4{0.0f, 0.0f, 0.0f, 0.0f};
  auto fold = [&](int b) __attribute__((always_inline)) {
    float gm = t[b][0];
#pragma unroll
    for (int j = 1; j < G; ++j) gm = fmaxf(gm, t[b][j]);
    if (gm > L) {  // a larger maximum: rescale what has been summed so far
      const float a = L > kNegInf ? exp2_hw(L - gm) : 0.0f;
      wsum *= a;
#pragma unroll
      for (int e = 0; e < 4; ++e) acc[e] *= a;
      L = gm;
    }
    if (L > kNegInf) {
#pragma unroll
      for (int j = 0; j < G; ++j) {
        const float w = exp2_hw(t[b][j] - L);   // 0 for chunks past n and rows without keys (t = -inf)
        wsum += w;
#pragma unroll
        for (int e = 0; e < 4; ++e) acc[e] = __builtin_fmaf(w, x[b][j][e], acc[e]);
      }
    }
  };
  load(0, 0);
  for (int k0 = 0; k0 < nl; k0 += 2 * G) {
    if (k0 + G < nl) load(k0 + G, 1);
    fold(0);
    if (k0 + G >= nl) break;
    if (k0 + 2 * G < nl) load(k0 + 2 * G, 0);
    fold(1);
  }
  // the CS lanes of this float4 (adjacent, all past or all before the row
  // check above) combine their states pairwise
#pragma unroll
  for (int off = 1; off < CS; off <<= 1) {
    const float Lo = __shfl_xor(L, off, 64);
    const float wo = __shfl_xor(wsum, off, 64);
    floatx4 ao;
#pragma unroll
    for (int e = 0; e < 4; ++e) ao[e] = __shfl_xor(acc[e], off, 64);
    const float Lm = fmaxf(L, Lo);
    const float sa = L > kNegInf ? exp2_hw(L - Lm) : 0.0f;
    const float sb = Lo > kNegInf ? exp2_hw(Lo - Lm) : 0.0f;
    wsum = wsum * sa + wo * sb;
#pragma unroll
    for (int e = 0; e < 4; ++e) acc[e] = acc[e] * sa + ao[e] * sb;
    L = Lm;
  }
  if (c0 != 0) return;
  if (!(L > kNegInf)) {  // the row saw no key in any chunk
    *(bf16x4*)op = bf16x4{};
    if (lse_writer) LSE[(size_t)bh * plan.Nq + row] = kNegInf;
    return;
  }
  const float inv = 1.0f / wsum;
  *(bf16x4*)op = bf16x4{(__bf16)(acc[0] * inv), (__bf16)(acc[1] * inv), (__bf16)(acc[2] * inv),
                        (__bf16)(acc[3] * inv)};
  if (lse_writer) LSE[(size_t)bh * plan.Nq + row] = (L + __builtin_log2f(wsum)) * 0.693147180559945309f;
}

template <int D>
SplitPlan make_plan(const FwdArgs& a, int chunk) {
  SplitPlan p;
  p.chunk = chunk;
  p.BM = SplitCfg<D>::BM;
  p.Nq = a.Nq;
  p.Nk = a.Nk;
  p.diag = a.bottom_right ? a.Nk - a.Nq : 0;
  p.causal = a.causal != 0;
  const int n_qt = (a.Nq + p.BM - 1) / p.BM;
  long long units = 0;
  for (int qt = 0; qt < n_qt; ++qt) units += p.n_chunks(qt);
  p.units = units > 0x7FFFFFFF ? 0x7FFFFFFF : (int)units;
  return p;
}

// The library's chunk. Splitting pays where the whole launch leaves most of
// the chip idle: measured (kernel traces and per-workgroup timestamps),
// B=1 H=8 Nq=1 Nk=32768 runs in 42 us split against 644 us whole (8
// workgroups), while launches of about half a chip gain nothing -- B=2 H=8
// N=1024 causal (128 workgroups): the split kernel's span falls from 29.5 to
// 12.4 us, but writing its float32 partials back from L2 at the kernel's end
// and reading them in the merge take as long again; B=1 H=16 N=2048 (128
// ping-pong workgroups): 64-71 us split against 54 us whole. So a launch is
// split when it would have fewer workgroups than a quarter of the CUs (or,
// on the key-parity kernel, at most half the CUs with rows of 32 or more
// steps), into chunks of at least 128 keys sized for two workgroups per CU
// (measured faster than three for the long rows where splitting pays: fewer
// chunks to merge per row); no split either when the rows are too short to
// cut.
constexpr int kCUs = 256;
template <int D>
int auto_chunk(const FwdArgs& a) {
  using C = SplitCfg<D>;
  const SplitPlan probe = make_plan<D>(a, 1 << 30);
  const int n_qt = (a.Nq + C::BM - 1) / C::BM;
  // workgroups of the whole launch (the dispatch of launch_fwd_bf16): at
  // d = 128 with the hardware exp2, launches of at most 256 tiles of 128 rows
  // run the ping-pong kernel's key parities (64-row tiles if there are at
  // most 256 of those); otherwise its 256-row tiles, or the streaming
  // kernel's tiles
  long long keys = 0;
  int kmax = 0;
  for (int qt = 0; qt < n_qt; ++qt) {
    const int k = probe.kend(qt);
    if (k > 0) keys += k;
    kmax = k > kmax ? k : kmax;
  }
  const long long bh = (long long)a.B * a.H;
  const long long pp_tiles = bh * ((a.Nq + 255) / 256);
  if (D == 128 && a.emu16 == 0 && bh * ((a.Nq + 127) / 128) <= 256) {
    // key parities: 4 x 32 keys per step with 64-row tiles, else 2 x 32.
    // Measured (B = 1, 128 workgroups, non-causal, whole vs split): H4 N2048
    // (16 steps) 25.7 vs 32.0 us, H2 N4096 (32) 45.2 vs 41.0, H1 N8192 (64)
    // 86.9 vs 60.1; the split also wins with fewer than 64 workgroups.
    const bool four = bh * ((a.Nq + 63) / 64) <= 256;
    const long long wgs = four ? bh * ((a.Nq + 63) / 64) : bh * ((a.Nq + 127) / 128);
    const int steps = (kmax + (four ? 127 : 63)) / (four ? 128 : 64);
    if (!(wgs < kCUs / 4 || (wgs <= kCUs / 2 && steps >= 32))) return 0;
  } else {
    const bool pingpong = (D == 128 || D == 192) && (!a.causal || pp_tiles >= 256);
    const long long whole_wgs = pingpong ? pp_tiles : bh * n_qt;
    if (whole_wgs >= kCUs / 4) return 0;
  }
  keys *= (long long)a.B * a.H;
  const long long target = 2LL * kCUs;
  long long chunk = (keys + target - 1) / target;
  chunk = (chunk + 63) / 64 * 64;
  if (chunk < 128) chunk = 128;
  if (chunk >= kmax) return 0;
  return (int)chunk;
}

template <int D, bool CAUSAL, int EMU16>
hipError_t launch_split(const FwdArgs& a, const SplitInfo& s, float* ws, hipStream_t stream) {
  using C = SplitCfg<D>;
  const SplitPlan p = make_plan<D>(a, s.chunk);
  const long long grid = (long long)a.B * a.H * p.units;
  hipLaunchKernelGGL((fwd_bf16_stream_kernel<C, CAUSAL, EMU16, false, true>), dim3((unsigned)grid), dim3(C::THREADS),
                     0, stream, (const __bf16*)a.q, (const __bf16*)a.k, (const __bf16*)a.v, (__bf16*)a.o, a.lse,
                     nullptr, a.H, a.Nq, a.Nk, (a.Nq + C::BM - 1) / C::BM, a.scale_log2, a.tau, a.bottom_right,
                     nullptr, nullptr, 0, 0, p, ws);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  const int n_qt = (a.Nq + C::BM - 1) / C::BM;
  // rows of more chunks than one round of loads (8) take 8 lanes per float4
  if (p.n_chunks(n_qt - 1) > 8) {
    constexpr int CS = 8;
    const int pieces = C::BM * D * CS / 1024;
    const long long mgrid = (long long)a.B * a.H * n_qt * pieces;
    hipLaunchKernelGGL((fwd_split_merge_kernel<D, CS>), dim3((unsigned)mgrid), dim3(256), 0, stream, ws,
                       (__bf16*)a.o, a.lse, p, (int)grid, n_qt, pieces);
  } else {
    const int pieces = C::BM * D / 1024;
    const long long mgrid = (long long)a.B * a.H * n_qt * pieces;
    hipLaunchKernelGGL((fwd_split_merge_kernel<D, 1>), dim3((unsigned)mgrid), dim3(256), 0, stream, ws,
                       (__bf16*)a.o, a.lse, p, (int)grid, n_qt, pieces);
  }
  return hipGetLastError();
}

template <int D, bool CAUSAL>
hipError_t launch_split_mode(const FwdArgs& a, const SplitInfo& s, float* ws, hipStream_t stream) {
  switch (a.emu16) {
    case 0: return launch_split<D, CAUSAL, 0>(a, s, ws, stream);
    case 1: return launch_split<D, CAUSAL, 1>(a, s, ws, stream);
    case 2: return launch_split<D, CAUSAL, 2>(a, s, ws, stream);
    case 3: return launch_split<D, CAUSAL, 3>(a, s, ws, stream);
    case 4: return launch_split<D, CAUSAL, 4>(a, s, ws, stream);
    case 8: return launch_split<D, CAUSAL, 8>(a, s, ws, stream);
    case 16: return launch_split<D, CAUSAL, 16>(a, s, ws, stream);
    case kEmuDeg4: return launch_split<D, CAUSAL, kEmuDeg4>(a, s, ws, stream);
    case kEmuDeg5: return launch_split<D, CAUSAL, kEmuDeg5>(a, s, ws, stream);
    default: return hipErrorInvalidValue;
  }
}

template <int D>
SplitInfo plan_d(const FwdArgs& a, int key_chunk) {
  SplitInfo s;
  const int chunk = key_chunk > 0 ? key_chunk : auto_chunk<D>(a);
  if (chunk <= 0) return s;
  const SplitPlan p = make_plan<D>(a, chunk);
  s.chunk = chunk;
  s.units = p.units;
  s.rows = p.BM;
  // no partials when no tile is cut into more than one chunk
  const int n_qt = (a.Nq + p.BM - 1) / p.BM;
  s.ws_bytes = p.units > n_qt ? (long long)a.B * a.H * p.units * p.BM * (D + 1) * 4 : 0;
  return s;
}

}  // namespace

SplitInfo plan_fwd_split(const FwdArgs& a, int key_chunk) {
  switch (a.d) {
    case 64: return plan_d<64>(a, key_chunk);
    case 128: return plan_d<128>(a, key_chunk);
    case 192: return plan_d<192>(a, key_chunk);
    case 256: return plan_d<256>(a, key_chunk);
    default: return SplitInfo{};
  }
}

hipError_t launch_fwd_bf16_split(const FwdArgs& a, const SplitInfo& s, float* ws, hipStream_t stream) {
  if (s.chunk <= 0 || a.cu_q != nullptr) return hipErrorInvalidValue;
  switch (a.d) {
    case 64: return a.causal ? launch_split_mode<64, true>(a, s, ws, stream) : launch_split_mode<64, false>(a, s, ws, stream);
    case 128: return a.causal ? launch_split_mode<128, true>(a, s, ws, stream) : launch_split_mode<128, false>(a, s, ws, stream);
    case 192: return a.causal ? launch_split_mode<192, true>(a, s, ws, stream) : launch_split_mode<192, false>(a, s, ws, stream);
    case 256: return a.causal ? launch_split_mode<256, true>(a, s, ws, stream) : launch_split_mode<256, false>(a, s, ws, stream);
    default: return hipErrorInvalidValue;
  }
}

}  // namespace attn

// ---------------------------------------------------------------------------
// attn_fwd_split_noalloc: attn_fwd_split with its workspace taken from a
// file-scope device array instead of the caller, for callers that cannot
// allocate device memory (code under graph capture, tight serving loops).
//
// `scratch` is a host-side stand-in for the array: each device holds its own
// copy at its own address, which hipGetSymbolAddress gives with that device
// current. That address is looked up once per device on the first call made
// with the device current, kept, and is what the kernels receive; the array's
// name itself is never passed to a kernel or a copy.
// ---------------------------------------------------------------------------
namespace attn {
namespace {

constexpr long long kScratchBytes = ATTN_NOALLOC_SCRATCH_BYTES;   // per device, held until the process ends
static_assert(kScratchBytes % 256 == 0, "scratch size");
static __device__ __attribute__((aligned(256))) float scratch[kScratchBytes / sizeof(float)];

constexpr int kMaxDevices = 64;
std::mutex g_scratch_mu;
float* g_scratch_ptr[kMaxDevices] = {};

// The scratch address on the device `stream` belongs to, which must be the
// current device (the address is looked up with that device current).
int scratch_for(void* stream, float** out) {
  int dev = -1;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return set_error(ATTN_E_HIP, hipGetErrorString(e));
  if (stream != nullptr) {
    int sdev = -1;
    e = hipStreamGetDevice(static_cast<hipStream_t>(stream), &sdev);
    if (e != hipSuccess) return set_error(ATTN_E_HIP, hipGetErrorString(e));
    if (sdev != dev) return set_error(ATTN_E_HIP, "the stream belongs to another device than the current one");
  }
  if (dev < 0 || dev >= kMaxDevices) return set_error(ATTN_E_HIP, "device index out of range");
  std::lock_guard<std::mutex> lock(g_scratch_mu);
  if (g_scratch_ptr[dev] == nullptr) {
    void* p = nullptr;
    e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    if (e != hipSuccess || p == nullptr)
      return set_error(ATTN_E_HIP, e != hipSuccess ? hipGetErrorString(e) : "no scratch address");
    g_scratch_ptr[dev] = static_cast<float*>(p);
  }
  *out = g_scratch_ptr[dev];
  return ATTN_OK;
}

}  // namespace
}  // namespace attn

extern "C" int attn_fwd_split_noalloc(const void* Q, const void* K, const void* V, void* O, float* LSE, int B, int H,
                                      int Nq, int Nk, int d, int causal, float scale, int exp2_mode, float tau,
                                      int dtype, const uint8_t* q_scale, const uint8_t* k_scale,
                                      const uint8_t* v_scale, int key_chunk, void* stream) {
  attn::FwdArgs a;
  attn::SplitInfo sp;
  bool nothing;
  int rc = attn::prepare_fwd_split(&a, &sp, &nothing, Q, K, V, O, LSE, B, H, Nq, Nk, d, causal, scale, exp2_mode,
                                   tau, dtype, q_scale, k_scale, v_scale, key_chunk, attn::kScratchBytes);
  if (rc != ATTN_OK || nothing) return rc;
  float* ws = nullptr;
  if (sp.ws_bytes > 0) {
    rc = attn::scratch_for(stream, &ws);
    if (rc != ATTN_OK) return rc;
  }
  return attn::run_fwd_split(a, dtype, sp, ws, stream);
}
