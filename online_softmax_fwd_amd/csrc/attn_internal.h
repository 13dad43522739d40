// attn_internal.h -- host-side interface between the C ABI (attn_api.cpp) and
// the kernel launchers (one .hip file per input dtype). Not installed.
#pragma once
#include <hip/hip_runtime_api.h>
#include <stdint.h>

namespace attn {

// Arguments after validation. Pointers are device pointers.
struct FwdArgs {
  const void* q;
  const void* k;
  const void* v;
  void* o;
  float* lse;
  const uint8_t* q_scale;   // MXFP8 only
  const uint8_t* k_scale;
  const uint8_t* v_scale;
  unsigned long long* stats;  // optional rescale counters (4 x uint64)
  int B, H, Nq, Nk, d;
  int causal;               // 0 or 1
  int bottom_right;         // causal: key j hidden from query i when j > i + (Nk - Nq) instead of j > i
  const int* cu_q;          // packed variable-length batch: sequence starts (B+1 entries), else nullptr
  const int* cu_k;
  int total_q, total_k;     // rows of the packed Q and K/V
  const int* scale_off_q;   // packed MXFP8: first scale row of each sequence (B+1 entries)
  const int* scale_off_k;
  int scale_rows_q, scale_rows_k;  // rows of the packed scale tensors
  float scale_log2;         // scale * log2(e)
  float tau;                // lagging-max threshold, log2 units
  int emu16;                // software-exp2 share of P, in 16ths (0 = all hardware)
};

struct BwdArgs {
  const void* q;
  const void* k;
  const void* v;
  const void* o;
  const void* d_o;
  const float* lse;
  void* d_q;
  void* d_k;
  void* d_v;
  float* ws;                // 2 floats per query row: LSE * log2(e), D = rowsum(dO * O)
  const uint8_t* q_scale;   // MXFP8: E8M0 per 32x32 block of Q, K, V, dO
  const uint8_t* k_scale;
  const uint8_t* v_scale;
  const uint8_t* do_scale;
  int B, H, Nq, Nk, d;
  int causal;               // 0 or 1
  int bottom_right;
  float scale;
  float scale_log2;         // scale * log2(e)
};

// Key-split plan of a dense bf16 launch: each query tile's keys cut into
// chunks of `chunk` keys run by separate workgroups and merged (chunk 0: the
// launch is not split).
struct SplitInfo {
  int chunk = 0;          // keys per chunk, a multiple of 64
  int units = 0;          // (query tile, chunk) units per (batch, head)
  int rows = 0;           // query rows per tile
  long long ws_bytes = 0; // float32 workspace the split launch needs
};
// key_chunk 0 lets the library choose (no split when the launch already fills
// the chip or its rows are too short to cut); otherwise that chunk size.
SplitInfo plan_fwd_split(const FwdArgs& a, int key_chunk);

// Validation and key-split plan of attn_fwd_split (attn_api.cpp), shared
// with its no-allocation variant: the arguments of attn_fwd_split without the
// workspace. ws_cap >= 0 bounds the workspace: with key_chunk 0 the library's
// chunk is doubled until its workspace fits (or no tile is cut any more and
// the launch runs whole); an explicit key_chunk that needs more is rejected
// (ATTN_E_SHAPE). ws_cap < 0: no bound. Returns ATTN_OK or an error code
// with the message set for attn_last_error; *nothing: no rows to compute.
int prepare_fwd_split(FwdArgs* a, SplitInfo* sp, bool* nothing, const void* Q, const void* K, const void* V, void* O,
                      float* LSE, int B, int H, int Nq, int Nk, int d, int causal, float scale, int exp2_mode,
                      float tau, int dtype, const uint8_t* q_scale, const uint8_t* k_scale, const uint8_t* v_scale,
                      int key_chunk, long long ws_cap);
// Runs a prepared launch: whole (sp.chunk == 0) or split with workspace ws.
int run_fwd_split(const FwdArgs& a, int dtype, const SplitInfo& sp, float* ws, void* stream);
// Sets this thread's message for attn_last_error and returns code.
int set_error(int code, const char* msg);

// Each returns hipSuccess or the launch error; none synchronises.
// Split launch (bf16, dense): the split kernel, then the merge kernel, on `stream`.
hipError_t launch_fwd_bf16_split(const FwdArgs& a, const SplitInfo& s, float* ws, hipStream_t stream);
hipError_t launch_fwd_bf16(const FwdArgs& a, hipStream_t stream);
hipError_t launch_fwd_f32(const FwdArgs& a, hipStream_t stream);
// prep pass, dK/dV kernel, dQ kernel, in that order on `stream`
hipError_t launch_bwd_bf16(const BwdArgs& a, hipStream_t stream);
hipError_t launch_bwd_mxfp8(const BwdArgs& a, hipStream_t stream);
// bf16 [rows, 128] -> e4m3 + one E8M0 byte per 32x32 block; rows % 32 == 0
hipError_t launch_mx_quantize(const void* x, uint8_t* q, uint8_t* scale, long long rows, hipStream_t stream);
// p_mode: 0 = P scaled per 32-key block, 1 = fixed 2^8 scale with E4M3 P,
// 2 = fixed 2^8 scale with E5M2 P
hipError_t launch_fwd_mxfp8(const FwdArgs& a, int p_mode, hipStream_t stream);
// Packed MXFP8 scale layouts: first scale row of each sequence for a given
// row alignment, and the copy of compact scale rows into another layout.
hipError_t launch_scale_offsets(const int* cu, int B, int total, int align, int* off, hipStream_t stream);
hipError_t launch_scale_scatter(const uint8_t* src, const int* src_off, int src_rows, uint8_t* dst,
                                const int* dst_off, int dst_rows, const int* cu, int B, int total, int row_bytes,
                                hipStream_t stream);
// degree 0 = hardware exp2, 3..5 = the software exp2 with that polynomial
hipError_t launch_exp2(const float* x, float* y, long n, int degree, hipStream_t stream);

// Codes for full emulation with the degree-4 / degree-5 polynomial (the same
// values as kEmuDeg4 / kEmuDeg5 in attn_device.h).
constexpr int kEmuDeg4Code = 17, kEmuDeg5Code = 18;
// Emulated shares (in 16ths) that have a compiled kernel instance.
bool emu16_supported(int emu16);

}  // namespace attn
