// attn_api.cpp -- the C ABI declared in include/attn.h: argument validation,
// the exp2-mix tuning table and dispatch to the per-dtype launchers.
// Validation runs before any HIP call, so every error path works on a host
// without a GPU.
#include "attn.h"

#include <algorithm>
#include <cmath>
#include <cstdarg>
#include <cstdint>
#include <cstdio>

#include "attn_internal.h"

namespace {

thread_local char g_err[512] = "";

int fail(int code, const char* fmt, ...) {
  va_list ap;
  va_start(ap, fmt);
  vsnprintf(g_err, sizeof g_err, fmt, ap);
  va_end(ap);
  return code;
}

bool aligned16(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }

bool is_mx(int dtype) {
  return dtype == ATTN_MXFP8_E4M3 || dtype == ATTN_MXFP8_E4M3_PFIX_E4M3 || dtype == ATTN_MXFP8_E4M3_PFIX_E5M2;
}
constexpr int kPMaxOffset = 8;  // P scale exponent of the fixed-scale FP8 P dtypes

// Emulated share of P (16ths) for ATTN_EXP2_MIX, keyed by (dtype, d, causal).
// The first page reports the Blackwell kernel's shares ("FlashAttention-4's
// Softmax Tricks", section "The emulated exp2": 18.75 % non-causal d=128,
// 12.5 % causal d=128, 25 % FP8), chosen there because the exponential unit
// is a separate, narrow pipeline. On gfx950 v_exp_f32 issues on the vector ALU
// itself, and the software exp2 costs 7 more VALU instructions per value
// (SQ_INSTS_VALU per launch), so moving work there only pays if the ALU has
// idle issue slots. The entries are the fastest shares measured on MI355X
// with these kernels (HIP-event medians after a 2 s warm-up, shares 0, 1, 2
// and 4 sixteenths): bf16 d=128 non-causal and causal at B=4 H=16 N=4096,
// bf16 d=64 causal at B=2 H=32 N=8192 and MXFP8 at B=2 H=16 N=8192 (every P
// mode) are all fastest all-hardware. The float32 kernel follows the bf16
// entries.
int mix_table(int dtype, int d, int causal) {
  if (d != 64 && d != 128 && !(dtype == ATTN_BF16 && (d == 192 || d == 256))) return -1;
  switch (dtype) {
    case ATTN_BF16:
    case ATTN_F32:
    case ATTN_MXFP8_E4M3:
    case ATTN_MXFP8_E4M3_PFIX_E4M3:
    case ATTN_MXFP8_E4M3_PFIX_E5M2:
      return 0;
    default:
      return -1;
  }
}

// Checks shared by the dense and the packed entry points; sets *emu16.
int validate_common(int dtype, int d, int causal, float scale, int exp2_mode, float tau, int* emu16) {
  if (dtype != ATTN_F32 && dtype != ATTN_BF16 && !is_mx(dtype))
    return fail(ATTN_E_DTYPE, "dtype %d is not ATTN_F32, ATTN_BF16 or one of the ATTN_MXFP8 codes", dtype);
  if (dtype == ATTN_BF16 ? (d != 64 && d != 128 && d != 192 && d != 256) : (d != 64 && d != 128))
    return fail(ATTN_E_HEADDIM, "head dim d=%d is not supported for dtype %d (bf16: 64, 128, 192, 256; f32: 64, 128; "
                "MXFP8: 128)", d, dtype);
  if (causal < 0 || causal > 2)
    return fail(ATTN_E_SHAPE, "causal=%d is not 0 (none), 1 (top-left) or 2 (bottom-right)", causal);
  if (!std::isfinite(scale) || !(scale > 0.0f))
    return fail(ATTN_E_SCALE, "scale=%g must be finite and > 0 (the row max is kept in raw score units)",
                (double)scale);
  if (!std::isfinite(tau) || tau < 0.0f || tau > 64.0f)
    return fail(ATTN_E_TAU, "tau=%g must be finite and in [0, 64]", (double)tau);
  // A fixed P scale of 2^max_offset lets a lagging max push P up to
  // 2^(max_offset + tau), which must stay below the format's largest value.
  if (dtype == ATTN_MXFP8_E4M3_PFIX_E4M3 || dtype == ATTN_MXFP8_E4M3_PFIX_E5M2) {
    const double pmax = dtype == ATTN_MXFP8_E4M3_PFIX_E4M3 ? 448.0 : 57344.0;
    if (!(kPMaxOffset + (double)tau < std::log2(pmax)))
      return fail(ATTN_E_TAU, "tau=%g: with P scaled by 2^%d, max_offset + tau must stay below log2(%g) = %.3f",
                  (double)tau, kPMaxOffset, pmax, std::log2(pmax));
  }
  if (exp2_mode == ATTN_EXP2_HW) {
    *emu16 = 0;
  } else if (exp2_mode == ATTN_EXP2_EMU) {
    *emu16 = 16;
  } else if (exp2_mode == ATTN_EXP2_EMU4 || exp2_mode == ATTN_EXP2_EMU5) {
    if (is_mx(dtype))
      return fail(ATTN_E_EXP2MODE, "exp2_mode=%d (degree-%d software exp2) is for ATTN_F32 and ATTN_BF16", exp2_mode,
                  exp2_mode == ATTN_EXP2_EMU4 ? 4 : 5);
    *emu16 = exp2_mode == ATTN_EXP2_EMU4 ? attn::kEmuDeg4Code : attn::kEmuDeg5Code;
  } else if (exp2_mode == ATTN_EXP2_MIX) {
    *emu16 = mix_table(dtype, d, causal != 0);
  } else if (exp2_mode >= ATTN_EXP2_MIX_BASE && exp2_mode <= ATTN_EXP2_MIX_BASE + 16) {
    *emu16 = exp2_mode - ATTN_EXP2_MIX_BASE;
  } else {
    return fail(ATTN_E_EXP2MODE, "exp2_mode=%d is not HW (0), EMU (1), MIX (2), EMU4 (3), EMU5 (4) or MIX_BASE+k (16..32)",
                exp2_mode);
  }
  if (*emu16 < 0 || !attn::emu16_supported(*emu16))
    return fail(ATTN_E_EXP2MODE, "no kernel instance emulates %d/16 of the exponentials", *emu16);
  return ATTN_OK;
}

void fill(attn::FwdArgs& a, const void* Q, const void* K, const void* V, void* O, float* LSE, int B, int H, int Nq,
          int Nk, int d, int causal, float scale, float tau, int emu16) {
  a.q = Q;
  a.k = K;
  a.v = V;
  a.o = O;
  a.lse = LSE;
  a.q_scale = a.k_scale = a.v_scale = nullptr;
  a.stats = nullptr;
  a.B = B;
  a.H = H;
  a.Nq = Nq;
  a.Nk = Nk;
  a.d = d;
  a.causal = causal != 0;
  a.bottom_right = causal == 2;
  a.cu_q = a.cu_k = nullptr;
  a.total_q = a.total_k = 0;
  a.scale_off_q = a.scale_off_k = nullptr;
  a.scale_rows_q = a.scale_rows_k = 0;
  a.scale_log2 = (float)((double)scale * 1.4426950408889634073599246810019);
  a.tau = tau;
  a.emu16 = emu16;
}

int validate_and_fill(attn::FwdArgs& a, const void* Q, const void* K, const void* V, void* O, float* LSE,
                      int B, int H, int Nq, int Nk, int d, int causal, float scale, int exp2_mode, float tau,
                      int dtype, const uint8_t* qs, const uint8_t* ks, const uint8_t* vs, bool* nothing) {
  *nothing = false;
  if (dtype != ATTN_F32 && dtype != ATTN_BF16 && !is_mx(dtype))
    return fail(ATTN_E_DTYPE, "dtype %d is not ATTN_F32, ATTN_BF16 or one of the ATTN_MXFP8 codes", dtype);
  if (B < 0 || H < 0 || Nq < 0 || Nk < 0)
    return fail(ATTN_E_SHAPE, "negative size (B=%d H=%d Nq=%d Nk=%d)", B, H, Nq, Nk);
  int emu16;
  const bool mx = is_mx(dtype);
  const int rc = validate_common(dtype, d, causal, scale, exp2_mode, tau, &emu16);
  if (rc != ATTN_OK) return rc;

  const long long rows = (long long)B * H * Nq;
  if (rows == 0) {
    *nothing = true;
    return ATTN_OK;
  }
  if (Nk < 1) return fail(ATTN_E_SHAPE, "Nk=%d: softmax over an empty key set is undefined", Nk);
  const long long n_qt = (Nq + 127) / 128;
  if ((long long)B * H * n_qt > 0x7FFFFFFFLL || Nq > (1 << 30) || Nk > (1 << 30))
    return fail(ATTN_E_SHAPE, "sizes too large (B=%d H=%d Nq=%d Nk=%d)", B, H, Nq, Nk);
  // The kernels address one (batch, head) slice of Q, K or V through a buffer
  // resource with 32-bit byte offsets, up to one key tile past the end.
  const long long esize = dtype == ATTN_F32 ? 4 : dtype == ATTN_BF16 ? 2 : 1;
  if (((long long)std::max(Nq, Nk) + 256) * d * esize > 0x7FFFFFFFLL)
    return fail(ATTN_E_SHAPE, "one (batch, head) slice of Q, K or V must stay under 2 GiB (Nq=%d Nk=%d d=%d)", Nq,
                Nk, d);
  if (mx && (Nq % 32 != 0 || Nk % 32 != 0))
    return fail(ATTN_E_SHAPE, "MXFP8 needs Nq and Nk to be multiples of 32 (Nq=%d Nk=%d)", Nq, Nk);
  if (!Q || !K || !V || !O || !LSE) return fail(ATTN_E_NULLPTR, "Q, K, V, O and LSE must be non-NULL");
  if (mx && (!qs || !ks || !vs))
    return fail(ATTN_E_NULLPTR, "MXFP8 needs q_scale, k_scale and v_scale");
  if (mx && d != 128) return fail(ATTN_E_HEADDIM, "MXFP8 supports d=128 (got %d)", d);
  if (mx &&
      ((reinterpret_cast<uintptr_t>(qs) | reinterpret_cast<uintptr_t>(ks) | reinterpret_cast<uintptr_t>(vs)) & 3u))
    return fail(ATTN_E_ALIGN, "MX scale pointers must be 4-byte aligned");
  if (!aligned16(Q) || !aligned16(K) || !aligned16(V) || !aligned16(O) || !aligned16(LSE))
    return fail(ATTN_E_ALIGN, "Q, K, V, O and LSE must be 16-byte aligned");

  fill(a, Q, K, V, O, LSE, B, H, Nq, Nk, d, causal, scale, tau, emu16);
  a.q_scale = qs;
  a.k_scale = ks;
  a.v_scale = vs;
  return ATTN_OK;
}

int run(const attn::FwdArgs& a, int dtype, void* stream) {
  hipStream_t s = static_cast<hipStream_t>(stream);
  hipError_t e;
  switch (dtype) {
    case ATTN_BF16: e = attn::launch_fwd_bf16(a, s); break;
    case ATTN_F32: e = attn::launch_fwd_f32(a, s); break;
    default: e = attn::launch_fwd_mxfp8(a, dtype - ATTN_MXFP8_E4M3, s); break;
  }
  if (e != hipSuccess) return fail(ATTN_E_HIP, "kernel launch failed: %s", hipGetErrorString(e));
  return ATTN_OK;
}

// Shared by attn_fwd_split and attn_fwd_split_workspace_bytes: the split
// plan of a dense launch (no split for dtypes other than bf16).
int split_plan_of(const attn::FwdArgs& a, int dtype, int key_chunk, attn::SplitInfo* s) {
  *s = attn::SplitInfo{};
  if (key_chunk < 0 || (key_chunk > 0 && key_chunk % 64 != 0) || key_chunk > (1 << 30))
    return fail(ATTN_E_SHAPE, "key_chunk=%d must be 0 (the library's choice) or a positive multiple of 64", key_chunk);
  if (dtype != ATTN_BF16) return ATTN_OK;
  *s = attn::plan_fwd_split(a, key_chunk);
  if (s->chunk > 0 && (long long)a.B * a.H * s->units > 0x7FFFFFFFLL)
    return fail(ATTN_E_SHAPE, "key_chunk=%d cuts the launch into too many workgroups", key_chunk);
  return ATTN_OK;
}

}  // namespace

namespace attn {

int set_error(int code, const char* msg) { return fail(code, "%s", msg); }

int prepare_fwd_split(FwdArgs* a, SplitInfo* sp, bool* nothing, const void* Q, const void* K, const void* V, void* O,
                      float* LSE, int B, int H, int Nq, int Nk, int d, int causal, float scale, int exp2_mode,
                      float tau, int dtype, const uint8_t* q_scale, const uint8_t* k_scale, const uint8_t* v_scale,
                      int key_chunk, long long ws_cap) {
  int rc = validate_and_fill(*a, Q, K, V, O, LSE, B, H, Nq, Nk, d, causal, scale, exp2_mode, tau, dtype, q_scale,
                             k_scale, v_scale, nothing);
  if (rc != ATTN_OK) return rc;
  rc = split_plan_of(*a, dtype, key_chunk, sp);
  if (rc != ATTN_OK || *nothing || ws_cap < 0 || sp->ws_bytes <= ws_cap) return rc;
  if (key_chunk > 0)
    return fail(ATTN_E_SHAPE, "key_chunk=%d needs %lld bytes of workspace; the library's scratch holds %lld",
                key_chunk, sp->ws_bytes, ws_cap);
  // the library's chunk: grow it until the partials fit
  for (long long ch = 2LL * sp->chunk; ch <= (1 << 30); ch *= 2) {
    *sp = plan_fwd_split(*a, (int)ch);
    if (sp->ws_bytes == 0) break;       // no tile is cut any more
    if (sp->ws_bytes <= ws_cap) return ATTN_OK;
  }
  *sp = SplitInfo{};                     // run whole
  return ATTN_OK;
}

int run_fwd_split(const FwdArgs& a, int dtype, const SplitInfo& sp, float* ws, void* stream) {
  if (sp.chunk <= 0) return run(a, dtype, stream);
  hipError_t e = launch_fwd_bf16_split(a, sp, ws, static_cast<hipStream_t>(stream));
  if (e != hipSuccess) return fail(ATTN_E_HIP, "kernel launch failed: %s", hipGetErrorString(e));
  return ATTN_OK;
}

}  // namespace attn

extern "C" {

int attn_fwd_ex(const void* Q, const void* K, const void* V, void* O, float* LSE, int B, int H, int Nq, int Nk,
                int d, int causal, float scale, int exp2_mode, float tau, int dtype, const uint8_t* q_scale,
                const uint8_t* k_scale, const uint8_t* v_scale, void* stream) {
  attn::FwdArgs a;
  bool nothing;
  int rc = validate_and_fill(a, Q, K, V, O, LSE, B, H, Nq, Nk, d, causal, scale, exp2_mode, tau, dtype, q_scale,
                             k_scale, v_scale, &nothing);
  if (rc != ATTN_OK || nothing) return rc;
  return run(a, dtype, stream);
}

int attn_fwd(const void* Q, const void* K, const void* V, void* O, float* LSE, int B, int H, int Nq, int Nk, int d,
             int causal, float scale, int exp2_mode, float tau) {
  return attn_fwd_ex(Q, K, V, O, LSE, B, H, Nq, Nk, d, causal, scale, exp2_mode, tau, ATTN_BF16, nullptr, nullptr,
                     nullptr, nullptr);
}

long long attn_fwd_split_workspace_bytes(int B, int H, int Nq, int Nk, int d, int causal, int dtype,
                                         int key_chunk) {
  // validation of everything but the pointers (stand-ins that pass those checks)
  alignas(16) static char dummy[16];
  attn::FwdArgs a;
  bool nothing;
  const uint8_t* sc = reinterpret_cast<const uint8_t*>(dummy);
  if (validate_and_fill(a, dummy, dummy, dummy, dummy, reinterpret_cast<float*>(dummy), B, H, Nq, Nk, d, causal,
                        1.0f, ATTN_EXP2_HW, 0.0f, dtype, sc, sc, sc, &nothing) != ATTN_OK)
    return -1;
  if (nothing) return 0;
  attn::SplitInfo sp;
  if (split_plan_of(a, dtype, key_chunk, &sp) != ATTN_OK) return -1;
  return sp.ws_bytes;
}

int attn_fwd_split(const void* Q, const void* K, const void* V, void* O, float* LSE, int B, int H, int Nq, int Nk,
                   int d, int causal, float scale, int exp2_mode, float tau, int dtype, const uint8_t* q_scale,
                   const uint8_t* k_scale, const uint8_t* v_scale, int key_chunk, float* workspace,
                   long long workspace_bytes, void* stream) {
  attn::FwdArgs a;
  attn::SplitInfo sp;
  bool nothing;
  int rc = attn::prepare_fwd_split(&a, &sp, &nothing, Q, K, V, O, LSE, B, H, Nq, Nk, d, causal, scale, exp2_mode, tau,
                                   dtype, q_scale, k_scale, v_scale, key_chunk, -1);
  if (rc != ATTN_OK || nothing) return rc;
  if (sp.ws_bytes > 0) {
    if (workspace_bytes < sp.ws_bytes)
      return fail(ATTN_E_SHAPE, "workspace of %lld bytes; attn_fwd_split_workspace_bytes gives %lld", workspace_bytes,
                  sp.ws_bytes);
    if (!workspace) return fail(ATTN_E_NULLPTR, "this launch is split and needs a workspace");
    if (!aligned16(workspace)) return fail(ATTN_E_ALIGN, "workspace must be 16-byte aligned");
  }
  return attn::run_fwd_split(a, dtype, sp, workspace, stream);
}

int attn_fwd_stats(const void* Q, const void* K, const void* V, void* O, float* LSE, int B, int H, int Nq, int Nk,
                   int d, int causal, float scale, int exp2_mode, float tau, int dtype, const uint8_t* q_scale,
                   const uint8_t* k_scale, const uint8_t* v_scale, unsigned long long* stats, void* stream) {
  attn::FwdArgs a;
  bool nothing;
  int rc = validate_and_fill(a, Q, K, V, O, LSE, B, H, Nq, Nk, d, causal, scale, exp2_mode, tau, dtype, q_scale,
                             k_scale, v_scale, &nothing);
  if (rc != ATTN_OK) return rc;
  if (!stats) return fail(ATTN_E_NULLPTR, "stats must be non-NULL");
  if ((reinterpret_cast<uintptr_t>(stats) & 7u) != 0) return fail(ATTN_E_ALIGN, "stats must be 8-byte aligned");
  if (nothing) return ATTN_OK;
  a.stats = stats;
  return run(a, dtype, stream);
}

int attn_fwd_varlen_ex(const void* Q, const void* K, const void* V, void* O, float* LSE, const uint8_t* q_scale,
                       const uint8_t* k_scale, const uint8_t* v_scale, const int* cu_seqlens_q,
                       const int* cu_seqlens_k, const int* scale_offsets_q, const int* scale_offsets_k,
                       int scale_rows_q, int scale_rows_k, int B, int H, int max_seqlen_q, int total_q, int total_k,
                       int d, int causal, float scale, int exp2_mode, float tau, int dtype, void* stream) {
  if (dtype != ATTN_F32 && dtype != ATTN_BF16 && !is_mx(dtype))
    return fail(ATTN_E_DTYPE, "dtype %d is not ATTN_F32, ATTN_BF16 or one of the ATTN_MXFP8 codes", dtype);
  const bool mx = is_mx(dtype);
  if (B < 0 || H < 0 || max_seqlen_q < 0 || total_q < 0 || total_k < 0 || (mx && (scale_rows_q < 0 || scale_rows_k < 0)))
    return fail(ATTN_E_SHAPE, "negative size (B=%d H=%d max_seqlen_q=%d total_q=%d total_k=%d scale rows %d/%d)", B,
                H, max_seqlen_q, total_q, total_k, scale_rows_q, scale_rows_k);
  int emu16;
  const int rc = validate_common(dtype, d, causal, scale, exp2_mode, tau, &emu16);
  if (rc != ATTN_OK) return rc;
  if (mx && d != 128) return fail(ATTN_E_HEADDIM, "MXFP8 supports d=128 (got %d)", d);
  if ((long long)B * H * max_seqlen_q == 0 || total_q == 0) return ATTN_OK;
  if (max_seqlen_q > total_q)
    return fail(ATTN_E_SHAPE, "max_seqlen_q=%d exceeds total_q=%d", max_seqlen_q, total_q);
  const long long n_qt = (max_seqlen_q + 127) / 128;
  if ((long long)B * H * n_qt > 0x7FFFFFFFLL)
    return fail(ATTN_E_SHAPE, "sizes too large (B=%d H=%d max_seqlen_q=%d)", B, H, max_seqlen_q);
  // every row of one head's sequence is addressed with 32-bit byte offsets
  // from the sequence start, up to one key tile past the end
  const long long esize = dtype == ATTN_F32 ? 4 : dtype == ATTN_BF16 ? 2 : 1;
  if (((long long)std::max(total_q, total_k) + 256) * H * d * esize > 0x7FFFFFFFLL)
    return fail(ATTN_E_SHAPE, "packed Q, K or V must stay under 2 GiB (total_q=%d total_k=%d H=%d d=%d)",
                total_q, total_k, H, d);
  if (!Q || !K || !V || !O || !LSE || !cu_seqlens_q || !cu_seqlens_k)
    return fail(ATTN_E_NULLPTR, "Q, K, V, O, LSE, cu_seqlens_q and cu_seqlens_k must be non-NULL");
  if (mx && (!q_scale || !k_scale || !v_scale || !scale_offsets_q || !scale_offsets_k))
    return fail(ATTN_E_NULLPTR, "MXFP8 needs q_scale, k_scale, v_scale, scale_offsets_q and scale_offsets_k");
  if (!aligned16(Q) || !aligned16(K) || !aligned16(V) || !aligned16(O) || !aligned16(LSE))
    return fail(ATTN_E_ALIGN, "Q, K, V, O and LSE must be 16-byte aligned");
  uintptr_t small = reinterpret_cast<uintptr_t>(cu_seqlens_q) | reinterpret_cast<uintptr_t>(cu_seqlens_k);
  if (mx)
    small |= reinterpret_cast<uintptr_t>(q_scale) | reinterpret_cast<uintptr_t>(k_scale) |
             reinterpret_cast<uintptr_t>(v_scale) | reinterpret_cast<uintptr_t>(scale_offsets_q) |
             reinterpret_cast<uintptr_t>(scale_offsets_k);
  if (small & 3u)
    return fail(ATTN_E_ALIGN, "cu_seqlens, MX scale and scale offset pointers must be 4-byte aligned");
  attn::FwdArgs a;
  fill(a, Q, K, V, O, LSE, B, H, max_seqlen_q, total_k, d, causal, scale, tau, emu16);
  a.cu_q = cu_seqlens_q;
  a.cu_k = cu_seqlens_k;
  a.total_q = total_q;
  a.total_k = total_k;
  if (mx) {
    a.q_scale = q_scale;
    a.k_scale = k_scale;
    a.v_scale = v_scale;
    a.scale_off_q = scale_offsets_q;
    a.scale_off_k = scale_offsets_k;
    a.scale_rows_q = scale_rows_q;
    a.scale_rows_k = scale_rows_k;
  }
  return run(a, dtype, stream);
}

int attn_fwd_varlen(const void* Q, const void* K, const void* V, void* O, float* LSE, const int* cu_seqlens_q,
                    const int* cu_seqlens_k, int B, int H, int max_seqlen_q, int total_q, int total_k, int d,
                    int causal, float scale, int exp2_mode, float tau, int dtype, void* stream) {
  if (dtype != ATTN_F32 && dtype != ATTN_BF16)
    return fail(ATTN_E_DTYPE, "attn_fwd_varlen takes ATTN_F32 or ATTN_BF16 (got dtype %d); MXFP8 batches need "
                "their scales: attn_fwd_varlen_ex", dtype);
  return attn_fwd_varlen_ex(Q, K, V, O, LSE, nullptr, nullptr, nullptr, cu_seqlens_q, cu_seqlens_k, nullptr, nullptr,
                            0, 0, B, H, max_seqlen_q, total_q, total_k, d, causal, scale, exp2_mode, tau, dtype,
                            stream);
}

int attn_mx_scale_offsets(const int* cu_seqlens, int B, int total, int align, int* offsets, void* stream) {
  if (B < 0 || total < 0) return fail(ATTN_E_SHAPE, "negative size (B=%d total=%d)", B, total);
  if (align < 32 || align > 4096 || align % 32 != 0)
    return fail(ATTN_E_SHAPE, "align=%d must be a multiple of 32 in [32, 4096]", align);
  if ((long long)total / 32 + (long long)B * (align / 32 + 1) > 0x7FFFFFFFLL)
    return fail(ATTN_E_SHAPE, "scale rows would overflow int32 (B=%d total=%d align=%d)", B, total, align);
  if (!cu_seqlens || !offsets) return fail(ATTN_E_NULLPTR, "cu_seqlens and offsets must be non-NULL");
  if ((reinterpret_cast<uintptr_t>(cu_seqlens) | reinterpret_cast<uintptr_t>(offsets)) & 3u)
    return fail(ATTN_E_ALIGN, "cu_seqlens and offsets must be 4-byte aligned");
  hipError_t e = attn::launch_scale_offsets(cu_seqlens, B, total, align, offsets, static_cast<hipStream_t>(stream));
  if (e != hipSuccess) return fail(ATTN_E_HIP, "kernel launch failed: %s", hipGetErrorString(e));
  return ATTN_OK;
}

int attn_mx_scale_scatter(const uint8_t* src, const int* src_offsets, int src_rows, uint8_t* dst,
                          const int* dst_offsets, int dst_rows, const int* cu_seqlens, int B, int total, int H, int d,
                          void* stream) {
  if (B < 0 || total < 0 || H < 0 || src_rows < 0 || dst_rows < 0)
    return fail(ATTN_E_SHAPE, "negative size (B=%d total=%d H=%d src_rows=%d dst_rows=%d)", B, total, H, src_rows,
                dst_rows);
  if (d != 128) return fail(ATTN_E_HEADDIM, "MXFP8 supports d=128 (got %d)", d);
  if (B == 0 || H == 0 || dst_rows == 0) return ATTN_OK;
  if ((long long)std::max(src_rows, dst_rows) * H * (d / 32) > 0x7FFFFFFFLL)
    return fail(ATTN_E_SHAPE, "scale tensors must stay under 2 GiB (rows %d/%d, H=%d)", src_rows, dst_rows, H);
  if (!src || !src_offsets || !dst || !dst_offsets || !cu_seqlens)
    return fail(ATTN_E_NULLPTR, "src, src_offsets, dst, dst_offsets and cu_seqlens must be non-NULL");
  if ((reinterpret_cast<uintptr_t>(src) | reinterpret_cast<uintptr_t>(dst) |
       reinterpret_cast<uintptr_t>(src_offsets) | reinterpret_cast<uintptr_t>(dst_offsets) |
       reinterpret_cast<uintptr_t>(cu_seqlens)) & 3u)
    return fail(ATTN_E_ALIGN, "scale, offset and cu_seqlens pointers must be 4-byte aligned");
  hipError_t e = attn::launch_scale_scatter(src, src_offsets, src_rows, dst, dst_offsets, dst_rows, cu_seqlens, B,
                                            total, H * (d / 32), static_cast<hipStream_t>(stream));
  if (e != hipSuccess) return fail(ATTN_E_HIP, "kernel launch failed: %s", hipGetErrorString(e));
  return ATTN_OK;
}

long long attn_bwd_workspace_bytes(int B, int H, int Nq) {
  if (B < 0 || H < 0 || Nq < 0) return -1;
  return 8LL * B * H * Nq;
}

int attn_bwd_ex(const void* Q, const void* K, const void* V, const void* O, const void* dO, const float* LSE, void* dQ,
                void* dK, void* dV, float* workspace, long long workspace_bytes, int B, int H, int Nq, int Nk, int d,
                int causal, float scale, int dtype, const uint8_t* q_scale, const uint8_t* k_scale,
                const uint8_t* v_scale, const uint8_t* do_scale, void* stream) {
  if (dtype != ATTN_BF16 && dtype != ATTN_MXFP8_E4M3)
    return fail(ATTN_E_DTYPE, "the backward pass takes ATTN_BF16 or ATTN_MXFP8_E4M3 (got dtype %d)", dtype);
  const bool mx = dtype == ATTN_MXFP8_E4M3;
  if (B < 0 || H < 0 || Nq < 0 || Nk < 0)
    return fail(ATTN_E_SHAPE, "negative size (B=%d H=%d Nq=%d Nk=%d)", B, H, Nq, Nk);
  if (mx ? d != 128 : (d != 64 && d != 128))
    return fail(ATTN_E_HEADDIM, "the backward pass supports d=64 and d=128 for bf16, d=128 for MXFP8 (got %d)", d);
  if (causal < 0 || causal > 2) return fail(ATTN_E_SHAPE, "causal=%d is not 0, 1 or 2", causal);
  if (!(scale > 0.0f) || !std::isfinite(scale)) return fail(ATTN_E_SCALE, "scale=%g must be finite and > 0", scale);
  if ((long long)B * H == 0 || (Nq == 0 && Nk == 0)) return ATTN_OK;
  const long long n_t = (std::max(Nq, Nk) + 127) / 128;
  if ((long long)B * H * n_t > 0x7FFFFFFFLL || Nq > (1 << 30) || Nk > (1 << 30))
    return fail(ATTN_E_SHAPE, "sizes too large (B=%d H=%d Nq=%d Nk=%d)", B, H, Nq, Nk);
  if (mx && (Nq % 32 != 0 || Nk % 32 != 0))
    return fail(ATTN_E_SHAPE, "MXFP8 needs Nq and Nk to be multiples of 32 (Nq=%d Nk=%d)", Nq, Nk);
  // one (batch, head) slice of Q, K, V or dO is addressed with 32-bit byte
  // offsets, up to one tile past the end
  if (((long long)std::max(Nq, Nk) + 256) * d * (mx ? 1 : 2) > 0x7FFFFFFFLL)
    return fail(ATTN_E_SHAPE, "one (batch, head) slice must stay under 2 GiB (Nq=%d Nk=%d d=%d)", Nq, Nk, d);
  if (workspace_bytes < attn_bwd_workspace_bytes(B, H, Nq))
    return fail(ATTN_E_SHAPE, "workspace of %lld bytes; attn_bwd_workspace_bytes gives %lld", workspace_bytes,
                attn_bwd_workspace_bytes(B, H, Nq));
  // tensors with no elements (Nq = 0: Q, O, dO, LSE, dQ, workspace and the Q /
  // dO scales; Nk = 0: K, V, dK, dV and their scales) are never touched and
  // may be NULL
  if (Nq > 0 && (!Q || !O || !dO || !LSE || !dQ || !workspace || (mx && (!q_scale || !do_scale))))
    return fail(ATTN_E_NULLPTR, "Q, O, dO, LSE, dQ, workspace (and for MXFP8 q_scale, do_scale) must be non-NULL");
  if (Nk > 0 && (!K || !V || !dK || !dV || (mx && (!k_scale || !v_scale))))
    return fail(ATTN_E_NULLPTR, "K, V, dK, dV (and for MXFP8 k_scale, v_scale) must be non-NULL");
  if (!aligned16(Q) || !aligned16(K) || !aligned16(V) || !aligned16(O) || !aligned16(dO) || !aligned16(LSE) ||
      !aligned16(dQ) || !aligned16(dK) || !aligned16(dV) || !aligned16(workspace))
    return fail(ATTN_E_ALIGN, "every tensor and the workspace must be 16-byte aligned");
  if (mx && ((reinterpret_cast<uintptr_t>(q_scale) | reinterpret_cast<uintptr_t>(k_scale) |
              reinterpret_cast<uintptr_t>(v_scale) | reinterpret_cast<uintptr_t>(do_scale)) & 3u))
    return fail(ATTN_E_ALIGN, "MX scale pointers must be 4-byte aligned");
  attn::BwdArgs a;
  a.q = Q;
  a.k = K;
  a.v = V;
  a.o = O;
  a.d_o = dO;
  a.lse = LSE;
  a.d_q = dQ;
  a.d_k = dK;
  a.d_v = dV;
  a.ws = workspace;
  a.q_scale = q_scale;
  a.k_scale = k_scale;
  a.v_scale = v_scale;
  a.do_scale = do_scale;
  a.B = B;
  a.H = H;
  a.Nq = Nq;
  a.Nk = Nk;
  a.d = d;
  a.causal = causal != 0;
  a.bottom_right = causal == 2;
  a.scale = scale;
  a.scale_log2 = (float)((double)scale * 1.4426950408889634073599246810019);
  hipStream_t st = static_cast<hipStream_t>(stream);
  hipError_t e = mx ? attn::launch_bwd_mxfp8(a, st) : attn::launch_bwd_bf16(a, st);
  if (e != hipSuccess) return fail(ATTN_E_HIP, "kernel launch failed: %s", hipGetErrorString(e));
  return ATTN_OK;
}

int attn_bwd(const void* Q, const void* K, const void* V, const void* O, const void* dO, const float* LSE, void* dQ,
             void* dK, void* dV, float* workspace, long long workspace_bytes, int B, int H, int Nq, int Nk, int d,
             int causal, float scale, int dtype, void* stream) {
  if (dtype != ATTN_BF16)
    return fail(ATTN_E_DTYPE, "attn_bwd takes ATTN_BF16 (got dtype %d); MXFP8 needs its scales: attn_bwd_ex", dtype);
  return attn_bwd_ex(Q, K, V, O, dO, LSE, dQ, dK, dV, workspace, workspace_bytes, B, H, Nq, Nk, d, causal, scale,
                     dtype, nullptr, nullptr, nullptr, nullptr, stream);
}

int attn_mx_quantize(const void* x, uint8_t* q, uint8_t* scale, long long rows, int d, void* stream) {
  if (d != 128) return fail(ATTN_E_HEADDIM, "attn_mx_quantize supports d=128 (got %d)", d);
  if (rows < 0 || rows % 32 != 0 || rows / 32 > 0x7FFFFFFFLL)
    return fail(ATTN_E_SHAPE, "rows=%lld must be a non-negative multiple of 32 (blocks are 32x32)", rows);
  if (rows == 0) return ATTN_OK;
  if (!x || !q || !scale) return fail(ATTN_E_NULLPTR, "x, q and scale must be non-NULL");
  if (!aligned16(x) || !aligned16(q)) return fail(ATTN_E_ALIGN, "x and q must be 16-byte aligned");
  hipError_t e = attn::launch_mx_quantize(x, q, scale, rows, static_cast<hipStream_t>(stream));
  if (e != hipSuccess) return fail(ATTN_E_HIP, "kernel launch failed: %s", hipGetErrorString(e));
  return ATTN_OK;
}

int attn_exp2(const float* x, float* y, long n, int exp2_mode, void* stream) {
  if (exp2_mode != ATTN_EXP2_HW && exp2_mode != ATTN_EXP2_EMU && exp2_mode != ATTN_EXP2_EMU4 &&
      exp2_mode != ATTN_EXP2_EMU5)
    return fail(ATTN_E_EXP2MODE, "attn_exp2 takes ATTN_EXP2_HW (0), EMU (1), EMU4 (3) or EMU5 (4), got %d", exp2_mode);
  if (n < 0) return fail(ATTN_E_SHAPE, "n=%ld is negative", n);
  if (n == 0) return ATTN_OK;
  if (!x || !y) return fail(ATTN_E_NULLPTR, "x and y must be non-NULL");
  if ((reinterpret_cast<uintptr_t>(x) & 3u) || (reinterpret_cast<uintptr_t>(y) & 3u))
    return fail(ATTN_E_ALIGN, "x and y must be 4-byte aligned");
  const int degree = exp2_mode == ATTN_EXP2_HW ? 0 : exp2_mode == ATTN_EXP2_EMU ? 3 : exp2_mode == ATTN_EXP2_EMU4 ? 4 : 5;
  hipError_t e = attn::launch_exp2(x, y, n, degree, static_cast<hipStream_t>(stream));
  if (e != hipSuccess) return fail(ATTN_E_HIP, "kernel launch failed: %s", hipGetErrorString(e));
  return ATTN_OK;
}

int attn_mix_sixteenths(int dtype, int d, int causal) { return mix_table(dtype, d, causal ? 1 : 0); }

const char* attn_last_error(void) { return g_err; }

}  // extern "C"
