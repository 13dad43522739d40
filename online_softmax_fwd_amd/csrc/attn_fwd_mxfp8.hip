// attn_fwd_mxfp8.hip -- block-scaled e4m3 (MXFP8) attention forward for gfx950.
//
// Inputs: Q, K, V as OCP e4m3 bytes [B,H,N,128] with one E8M0 byte per 32x32
// block ([B,H,N/32,4]; V blocked along the sequence with the same square
// blocks) -- "PyTorch FlashAttention-4 adds MXFP8 block-scaled forward and
// backward for Blackwell", section "Quantization along both axes and jagged
// tensors". Output O is bf16, LSE float32.
//
// Both contractions run on v_mfma_scale_f32_32x32x64_f8f6f4, which takes the
// E8M0 scales per lane and applies them inside the MFMA. Its operand layout
// (measured on the GPU): lane l holds 32 bytes of row l % 32; bytes 0..15 of
// lanes m and m+32 form K-block 0 (scaled by lane m's scale byte) and bytes
// 16..31 form K-block 1 (scaled by lane m+32's byte). So every MFMA consumes
// two 32-wide MX blocks, one scale per lane, selected from a packed scale
// dword by op_sel.
//
// Workgroup: 4 waves x 32 query rows; K and V stream through LDS in 64-key
// tiles (two buffers each, filled by buffer_load_dwordx4 ... lds). Per tile:
//   S^T = K Q^T        2 key blocks x 2 MFMAs (d = 128 = 2 x 64)
//   softmax            mask, block maxima of the two 32-key blocks (in-lane
//                      tree + v_permlane32_swap), lagging max ("FlashAttention-4's
//                      Softmax Tricks", "Conditional rescaling"), P = exp2 (hw,
//                      software or mix), l from float32 P
//   P -> e4m3          per 32-key block, as the MXFP8 page's "Softmax conversion
//                      and unroll-KV" section describes: the block amax comes
//                      from the softmax block max already computed (exp is
//                      monotone: amax = 2^a, a = (blockmax - m) * c), the
//                      E8M0 exponent of the smallest power of two X with
//                      amax / X <= 448 as ceil(a - log2 448) (the same rule,
//                      taken in the log domain: no exponential and no bit
//                      decoding), then P / X is converted with v_cvt_pk_fp8_f32.
//   O^T += V^T P^T     4 MFMAs (d blocks), A = V^T via ds_read_b64_tr_b8, B = P
//                      bytes straight from the S^T registers: the K rows
//                      feeding S^T are permuted so lane half h holds keys
//                      16h..16h+15 of each 32-key block, i.e. one half of an MX
//                      block, exactly the PV operand layout.
// Epilogue: O / l (deferred normalisation) and LSE = ln2 * (m*c + log2 l).
#include "attn_device.h"
#include "attn_internal.h"
#include "attn_mx_common.h"

namespace attn {
namespace {

constexpr int kD = 128;
constexpr int kRB = kD;                        // bytes per K/V row (one byte per element)
constexpr int kCH = kRB / 16;                  // 16-byte chunks per row
constexpr int kWaves = 4;
constexpr int kThreads = 64 * kWaves;
constexpr int kBM = 32 * kWaves;               // query rows per workgroup
constexpr int kBN = 64;                        // keys per tile
constexpr int kTile = kBN * kRB;               // bytes per K or V tile
constexpr int kLoads = kBN * kCH / 64 / kWaves;  // wave-loads per wave per tensor per tile
// Tiles whose K/V scale words one LDS refill holds: 2 words per tile and
// tensor, one word per thread.
constexpr int kScaleTiles = 64;
static_assert(4 * kScaleTiles == kThreads, "one scale word per thread per refill");
static_assert(kLoads * 64 * kWaves == kBN * kCH, "tile split");

// Swizzle of the 16-byte chunks (position c ^ f(r)), the same for the K and
// V tiles. LDS serves a 16-byte read 16 lanes at a time and an 8-byte read 32
// lanes at a time, and each group must touch 64 different banks: the K reads
// (one chunk of 16 permuted key rows per 16 lanes) and the V transpose reads
// (rows 16h + 0..7 and +8, +32, +40; 2 chunks) both do with f below, a map of
// row bits 1, 2 and 4 (rows are 128 bytes, two per bank line). Measured
// (SQ_LDS_BANK_CONFLICT / SQ_LDS_IDX_ACTIVE): 0, against 0.33 with the
// previous per-tensor swizzles, and 1-2 % faster.
__device__ __forceinline__ int swz_k(int r) { return (r & 6) ^ ((r >> 4) & 1); }
__device__ __forceinline__ int swz_v(int r) { return (r & 6) ^ ((r >> 4) & 1); }

// P quantisation: kPBlock = one E8M0 scale per 32-key block from the block
// amax (the MXFP8 page's design); kPFixedE4M3 / kPFixedE5M2 = P times the
// fixed 2^max_offset with max_offset = 8 and one constant scale byte, cast to
// E4M3 or E5M2 ("FlashAttention-4's Softmax Tricks", section "Where 'exact'
// breaks: P in FP8"); the boundary only admits tau with
// max_offset + tau < log2(largest finite value), so the cast never saturates.
enum { kPBlock = 0, kPFixedE4M3 = 1, kPFixedE5M2 = 2 };
constexpr int kMaxOffset = 8;

// Exponent k of the P scale X = 2^k of a 32-key block from its largest score
// bm: amax = 2^a with a = bm*c - mc, and the smallest power of two with
// amax / X <= 448 has k = ceil(a - log2 448) (the E8M0 rule, taken in the log
// domain, where the softmax already is: no exponential or bit decoding of
// amax). Clamped to [-126, 127] so that X is a normal float and its byte a
// finite E8M0; a fully masked block (a = -inf) takes -126.
__device__ __forceinline__ float p_scale_exponent(float bm, float c, float mc) {
  constexpr float kLog2Max = 8.80735492205760410f;  // log2(448)
  return __builtin_amdgcn_fmed3f(__builtin_ceilf(__builtin_fmaf(bm, c, -(mc + kLog2Max))), -126.0f, 127.0f);
}

// PACKED: a batch of sequences packed token-major ([total, H, d] data,
// [scale rows, H, d/32] scales at per-sequence scale offsets); lengths need
// not be multiples of 32, so row validity is per lane and the last 32-key
// block of a sequence may be partial (its keys past the end are masked and
// read as zero).
template <bool CAUSAL, int EMU16, int PMODE, bool PACKED>
__global__ __attribute__((amdgpu_flat_work_group_size(kThreads, kThreads), amdgpu_waves_per_eu(3, 3)))
void fwd_mxfp8_kernel(const uint8_t* __restrict__ Q, const uint8_t* __restrict__ K, const uint8_t* __restrict__ V,
                      const uint8_t* __restrict__ QS, const uint8_t* __restrict__ KS, const uint8_t* __restrict__ VS,
                      __bf16* __restrict__ O, float* __restrict__ LSE, unsigned long long* __restrict__ stats, int H,
                      int Nq_dense, int Nk_dense, int n_qt, float c, float tau, int bottom_right,
                      const int* __restrict__ cu_q, const int* __restrict__ cu_k, int total_q, int total_k,
                      const int* __restrict__ soff_q, const int* __restrict__ soff_k, int srows_q, int srows_k) {
  __shared__ __attribute__((aligned(1024))) char kb0[kTile];
  __shared__ __attribute__((aligned(1024))) char kb1[kTile];
  __shared__ __attribute__((aligned(1024))) char vb0[kTile];
  __shared__ __attribute__((aligned(1024))) char vb1[kTile];
  // E8M0 scale words of K and V (one dword = the 4 d-blocks of a 32-key
  // block) for kScaleTiles tiles, staged in LDS (see refill_scales)
  __shared__ uint32_t ksw[2 * kScaleTiles];
  __shared__ uint32_t vsw[2 * kScaleTiles];

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
  const int q0 = qt * kBM;
  const int qw0 = q0 + wave * 32;
  const int qi = qw0 + l32;
  const Slice sl = slice_of(bh, H, kD, Nq_dense, Nk_dense, PACKED ? cu_q : nullptr, cu_k, total_q, total_k);
  const int Nq = sl.Nq, Nk = sl.Nk;
  if (PACKED && q0 >= Nq) return;  // a query tile past this sequence's end
  const ScaleSlice sc =
      scale_slice_of(bh, H, kD, Nq, Nk, PACKED ? soff_q : nullptr, soff_k, srows_q, srows_k);
  const bool wave_rows = qw0 < Nq;  // wave-uniform: the wave has rows to compute
  const bool row_ok = qi < Nq;      // this lane's row (dense sizes are multiples of 32: equal to wave_rows)
  const size_t qbase = sl.qbase, kbase = sl.kbase;
  const int rs = PACKED ? sl.rs : kD;  // elements (= bytes of Q, K, V) between consecutive rows
  const uint32_t tile_bytes = (uint32_t)kBN * rs;

  // ---- per-lane constants --------------------------------------------------
  const int krow = mx_key_of_row(l32);
  uint32_t koff[2][2];  // [d step s][which 16-byte half]
#pragma unroll
  for (int s = 0; s < 2; ++s)
#pragma unroll
    for (int w = 0; w < 2; ++w) koff[s][w] = krow * kRB + 16 * ((4 * s + 2 * w + hh) ^ swz_k(krow));
  uint32_t voff[4];  // per d block: this lane's 8-byte slot of a transpose read, row offset 0
  {
    const int L = lane & 15, gidx = (lane >> 4) & 1;
    const int vr = 16 * hh + (L >> 1);
#pragma unroll
    for (int db = 0; db < 4; ++db) {
      const int cch = 2 * db + gidx;
      voff[db] = vr * kRB + 16 * (cch ^ swz_v(vr)) + 8 * (L & 1);
    }
  }
  uint32_t kld[kLoads], vld[kLoads];
#pragma unroll
  for (int i = 0; i < kLoads; ++i) {
    const int pos = 64 * (wave + kWaves * i) + lane;
    const int r = pos / kCH, p = pos % kCH;
    kld[i] = r * rs + 16 * (p ^ swz_k(r));
    vld[i] = r * rs + 16 * (p ^ swz_v(r));
  }
  const int nrec = Nk * rs;
  const u32x4 rk = raw_buffer_rsrc(K + kbase, (uint32_t)nrec);
  const u32x4 rv = raw_buffer_rsrc(V + kbase, (uint32_t)nrec);

  // ---- Q operand: lane (h, n) holds Q[n][64s + 16h .. +16] and Q[n][64s + 32 + 16h .. +16]
  i32x8 qf[2];
  uint32_t qsc = 0x7F7F7F7Fu;
  {
    const uint8_t* qp = Q + qbase + (size_t)(row_ok ? qi : 0) * rs + 16 * hh;
#pragma unroll
    for (int s = 0; s < 2; ++s) {
      const u32x4 lo = row_ok ? *(const u32x4*)(qp + 64 * s) : u32x4{0u, 0u, 0u, 0u};
      const u32x4 hi = row_ok ? *(const u32x4*)(qp + 64 * s + 32) : u32x4{0u, 0u, 0u, 0u};
      qf[s] = i32x8{(int)lo[0], (int)lo[1], (int)lo[2], (int)lo[3], (int)hi[0], (int)hi[1], (int)hi[2], (int)hi[3]};
    }
    if (wave_rows && qw0 / 32 < sc.qblocks) qsc = *(const uint32_t*)(QS + sc.qbase + (size_t)(qw0 / 32) * sc.stride);
  }
  // byte 2s of (qsc >> 8h) is the scale of d block 2s + h: op_sel picks byte 2s
  const int qscale = (int)(qsc >> (8 * hh));

  // causal: key j is hidden from query i when j > i + diag (top-left: diag = 0)
  const int diag = bottom_right ? Nk - Nq : 0;
  const int kend = CAUSAL ? min(Nk, q0 + kBM + diag) : Nk;
  const int n_kt = (kend + kBN - 1) / kBN;

  floatx16 o[4];
#pragma unroll
  for (int i = 0; i < 4; ++i) o[i] = floatx16{};
  float m_run = kNegInf, l_run = 0.0f;
  unsigned long long cnt[4] = {0, 0, 0, 0};

  auto load_tiles = [&](int t, char* kd, char* vd) __attribute__((always_inline)) {
    const u32x4 rkt = advance_rsrc(rk, (uint32_t)t * tile_bytes), rvt = advance_rsrc(rv, (uint32_t)t * tile_bytes);
    const uint32_t kl = __builtin_amdgcn_readfirstlane(lds_address(kd)), vl = __builtin_amdgcn_readfirstlane(lds_address(vd));
#pragma unroll
    for (int i = 0; i < kLoads; ++i) {
      const uint32_t slot = 1024 * (wave + kWaves * i);
      dma16_at(rkt, kl + slot, kld[i]);
      dma16_at(rvt, vl + slot, vld[i]);
    }
  };

  // The scale words of tiles t0 .. t0 + kScaleTiles - 1 into LDS, one per
  // thread (0x7F = 2^0 past the last block). Read per tile from global
  // memory, each word's load would be issued after the next tile's DMA and,
  // vmcnt draining in order, waiting for it would wait for that DMA as well;
  // a refill runs where no DMA is in flight, once per kScaleTiles tiles, and
  // the per-tile reads become LDS reads next to the K fragment reads.
  auto refill_scales = [&](int t0) __attribute__((always_inline)) {
    const int w = tid % (2 * kScaleTiles);
    const int blk = 2 * t0 + w;
    const bool is_k = tid < 2 * kScaleTiles;
    const uint8_t* base = (is_k ? KS : VS) + sc.kbase;
    const uint32_t word = blk < sc.kblocks ? *(const uint32_t*)(base + (size_t)blk * sc.stride) : 0x7F7F7F7Fu;
    if (is_k)
      ksw[w] = word;
    else
      vsw[w] = word;
  };

  auto compute = [&](int t, const char* ks, const char* vs) __attribute__((always_inline)) {
    const int k0 = t * kBN;
    if ((CAUSAL && k0 > qw0 + 31 + diag) || !wave_rows) return;  // wave-uniform: nothing to add
    const int sw = (2 * t) % (2 * kScaleTiles);
    const uint32_t kw0 = ksw[sw], kw1 = ksw[sw + 1];
    const uint32_t vw0 = vsw[sw], vw1 = vsw[sw + 1];
    const int kscale[2] = {(int)(kw0 >> (8 * hh)), (int)(kw1 >> (8 * hh))};
    const int vscale = (int)(hh ? vw1 : vw0);  // lane half h supplies key block 2t + h; op_sel picks d block

    // S^T = K Q^T
    floatx16 s[2];
#pragma unroll
    for (int kb = 0; kb < 2; ++kb) {
      s[kb] = floatx16{};
      const char* kp = ks + kb * 32 * kRB;
#pragma unroll
      for (int st = 0; st < 2; ++st) {
        const u32x4 lo = *(const u32x4*)(kp + koff[st][0]);
        const u32x4 hi = *(const u32x4*)(kp + koff[st][1]);
        const i32x8 a = {(int)lo[0], (int)lo[1], (int)lo[2], (int)lo[3], (int)hi[0], (int)hi[1], (int)hi[2], (int)hi[3]};
        if (st == 0)
          s[kb] = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(a, qf[0], s[kb], 0, 0, 0, kscale[kb], 0, qscale);
        else
          s[kb] = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(a, qf[1], s[kb], 0, 0, 2, kscale[kb], 2, qscale);
      }
    }

    if ((CAUSAL && k0 + kBN - 1 > qw0 + diag) || (k0 + kBN > Nk)) {
#pragma unroll
      for (int kb = 0; kb < 2; ++kb)
#pragma unroll
        for (int e = 0; e < 16; ++e) {
          const int key = k0 + 32 * kb + 16 * hh + e;
          if (key >= Nk || (CAUSAL && key > qi + diag)) s[kb][e] = kNegInf;
        }
    }

    // block maxima (reused for the P scales) and the row max
    const float bm0 = pl_max_halves(max16(s[0]));
    const float bm1 = pl_max_halves(max16(s[1]));
    const float mx = vmax(bm0, bm1);
    const float m_new = vmax(m_run, mx);
    const float acc = (m_run - m_new) * c;
    const bool seen = mx > kNegInf;
    const bool commit = seen && !(acc >= -tau);
    const float alpha = commit ? exp2_hw(acc) : 1.0f;
    if (stats) {
      const bool step = seen && (m_run > kNegInf) && hh == 0 && row_ok;
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
      for (int db = 0; db < 4; ++db) o[db] *= alpha;
    }
    const float mc = (m_run > kNegInf) ? m_run * c : 0.0f;

    // P -> e4m3 per 32-key block: the scale X = 2^k from the reused block max
    // (P is monotone in s), its E8M0 byte sb = k + 127, and P / X taken
    // straight from the exponential, 2^(s*c - mc - k), so the quantiser needs
    // no multiply; l adds the block sums times X.
    float k0f, k1f;  // X = 2^k of each block
    if constexpr (PMODE == kPBlock) {
      k0f = p_scale_exponent(bm0, c, mc);
      k1f = p_scale_exponent(bm1, c, mc);
    } else {
      k0f = k1f = (float)-kMaxOffset;  // P is stored times 2^max_offset
    }
    const uint32_t sb0 = (uint32_t)((int)k0f + 127), sb1 = (uint32_t)((int)k1f + 127);
    const float bias0 = mc + k0f, bias1 = mc + k1f;
#pragma unroll
    for (int e = 0; e < 16; ++e) s[0][e] = exp2_sel<EMU16>(__builtin_fmaf(s[0][e], c, -bias0), e);
#pragma unroll
    for (int e = 0; e < 16; ++e) s[1][e] = exp2_sel<EMU16>(__builtin_fmaf(s[1][e], c, -bias1), e);
    const float x0 = __builtin_bit_cast(float, sb0 << 23), x1 = __builtin_bit_cast(float, sb1 << 23);
    l_run = __builtin_fmaf(l_run, alpha, __builtin_fmaf(sum16(s[0]), x0, sum16(s[1]) * x1));
    i32x8 pq;
#pragma unroll
    for (int w = 0; w < 4; ++w) {
      int lo = undef_dword(), hi = undef_dword();
      if constexpr (PMODE == kPFixedE5M2) {
        lo = __builtin_amdgcn_cvt_pk_bf8_f32(s[0][4 * w], s[0][4 * w + 1], lo, false);
        lo = __builtin_amdgcn_cvt_pk_bf8_f32(s[0][4 * w + 2], s[0][4 * w + 3], lo, true);
        hi = __builtin_amdgcn_cvt_pk_bf8_f32(s[1][4 * w], s[1][4 * w + 1], hi, false);
        hi = __builtin_amdgcn_cvt_pk_bf8_f32(s[1][4 * w + 2], s[1][4 * w + 3], hi, true);
      } else {
        lo = __builtin_amdgcn_cvt_pk_fp8_f32(s[0][4 * w], s[0][4 * w + 1], lo, false);
        lo = __builtin_amdgcn_cvt_pk_fp8_f32(s[0][4 * w + 2], s[0][4 * w + 3], lo, true);
        hi = __builtin_amdgcn_cvt_pk_fp8_f32(s[1][4 * w], s[1][4 * w + 1], hi, false);
        hi = __builtin_amdgcn_cvt_pk_fp8_f32(s[1][4 * w + 2], s[1][4 * w + 3], hi, true);
      }
      pq[w] = lo;
      pq[4 + w] = hi;
    }
    const int pscale = (int)(hh ? sb1 : sb0);
    constexpr int kPFmt = PMODE == kPFixedE5M2 ? 1 : 0;  // MFMA B-operand format: 0 = E4M3, 1 = E5M2

    // O^T += V^T P^T
#pragma unroll
    for (int db = 0; db < 4; ++db) {
      i32x8 a;
#pragma unroll
      for (int r = 0; r < 4; ++r) {  // keys 32*(r/2) + 16h + 8*(r%2) .. +8
        const char* vp = vs + voff[db] + (32 * (r >> 1) + 8 * (r & 1)) * kRB;
        const intx2 v = __builtin_amdgcn_ds_read_tr8_b64_v2i32((lds_intx2*)vp);
        a[2 * r] = v[0];
        a[2 * r + 1] = v[1];
      }
      switch (db) {
        case 0: o[0] = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(a, pq, o[0], 0, kPFmt, 0, vscale, 0, pscale); break;
        case 1: o[1] = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(a, pq, o[1], 0, kPFmt, 1, vscale, 0, pscale); break;
        case 2: o[2] = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(a, pq, o[2], 0, kPFmt, 2, vscale, 0, pscale); break;
        default: o[3] = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(a, pq, o[3], 0, kPFmt, 3, vscale, 0, pscale); break;
      }
    }
  };

  refill_scales(0);
  load_tiles(0, kb0, vb0);
  wait_own_loads();
  __syncthreads();
  for (int t = 0; t < n_kt; t += 2) {
    if (t > 0 && t % kScaleTiles == 0) {  // every wave is past compute(t - 1); no DMA in flight
      refill_scales(t);
      __syncthreads();
    }
    if (t + 1 < n_kt) load_tiles(t + 1, kb1, vb1);
    compute(t, kb0, vb0);
    wait_own_loads();
    __syncthreads();
    if (t + 1 >= n_kt) break;
    if (t + 2 < n_kt) load_tiles(t + 2, kb0, vb0);
    compute(t + 1, kb1, vb1);
    wait_own_loads();
    __syncthreads();
  }

  const float l_tot = pl_sum_halves(l_run);
  const float inv = l_tot > 0.0f ? 1.0f / l_tot : 0.0f;  // a row that saw no key: O = 0, LSE = -inf
  if (row_ok) {
    __bf16* op = O + qbase + (size_t)qi * rs + 4 * hh;
#pragma unroll
    for (int db = 0; db < 4; ++db)
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

template <bool CAUSAL, int EMU16, int PMODE, bool PACKED>
hipError_t launch_k(const FwdArgs& a, hipStream_t stream) {
  const int n_qt = (a.Nq + kBM - 1) / kBM;
  const long long grid = (long long)a.B * a.H * n_qt;
  hipLaunchKernelGGL((fwd_mxfp8_kernel<CAUSAL, EMU16, PMODE, PACKED>), dim3((unsigned)grid), dim3(kThreads), 0,
                     stream, (const uint8_t*)a.q, (const uint8_t*)a.k, (const uint8_t*)a.v, a.q_scale, a.k_scale,
                     a.v_scale, (__bf16*)a.o, a.lse, a.stats, a.H, a.Nq, a.Nk, n_qt, a.scale_log2, a.tau,
                     a.bottom_right, a.cu_q, a.cu_k, a.total_q, a.total_k, a.scale_off_q, a.scale_off_k,
                     a.scale_rows_q, a.scale_rows_k);
  return hipGetLastError();
}

template <bool CAUSAL, int EMU16, int PMODE>
hipError_t launch(const FwdArgs& a, hipStream_t stream) {
  return a.cu_q ? launch_k<CAUSAL, EMU16, PMODE, true>(a, stream) : launch_k<CAUSAL, EMU16, PMODE, false>(a, stream);
}

template <bool CAUSAL, int PMODE>
hipError_t launch_mode(const FwdArgs& a, hipStream_t stream) {
  switch (a.emu16) {
    case 0: return launch<CAUSAL, 0, PMODE>(a, stream);
    case 1: return launch<CAUSAL, 1, PMODE>(a, stream);
    case 2: return launch<CAUSAL, 2, PMODE>(a, stream);
    case 3: return launch<CAUSAL, 3, PMODE>(a, stream);
    case 4: return launch<CAUSAL, 4, PMODE>(a, stream);
    case 8: return launch<CAUSAL, 8, PMODE>(a, stream);
    case 16: return launch<CAUSAL, 16, PMODE>(a, stream);
    default: return hipErrorInvalidValue;
  }
}

template <int PMODE>
hipError_t launch_p(const FwdArgs& a, hipStream_t stream) {
  return a.causal ? launch_mode<true, PMODE>(a, stream) : launch_mode<false, PMODE>(a, stream);
}

}  // namespace

hipError_t launch_fwd_mxfp8(const FwdArgs& a, int p_mode, hipStream_t stream) {
  if (a.d != kD) return hipErrorInvalidValue;
  switch (p_mode) {
    case kPBlock: return launch_p<kPBlock>(a, stream);
    case kPFixedE4M3: return launch_p<kPFixedE4M3>(a, stream);
    case kPFixedE5M2: return launch_p<kPFixedE5M2>(a, stream);
    default: return hipErrorInvalidValue;
  }
}

}  // namespace attn
