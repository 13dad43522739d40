// attn_mx_layout.hip -- scale-tensor layout kernels for packed MXFP8 batches.
//
// "PyTorch FlashAttention-4 adds MXFP8 block-scaled forward and backward for
// Blackwell", section "Quantization along both axes and jagged tensors": with
// jagged sequence lengths the FP8 data stays compact and only the small scale
// tensors are laid out for the kernel, each sequence's scale rows starting at
// an aligned position; light scatter kernels move the scales from the compact
// jagged layout into that one. On gfx950 the scaled MFMA takes its scale
// bytes from VGPRs and the attention kernel reads each (block, head) scale
// word with one aligned load from any row, so alignment is a choice of the
// caller here (32 = compact, 128 = the page's padded positions); the kernel
// only needs each sequence's first scale row, which these kernels produce.
//
// Scale tensors are [rows, H, d/32] E8M0 bytes; row r of sequence b holds the
// scales of its tokens 32r' .. 32r'+31 with r' = r - off[b].
#include "attn_device.h"
#include "attn_internal.h"

namespace attn {
namespace {

constexpr int kScanThreads = 256;

// off[b] = sum over b' < b of ceil(len(b') / align) * (align / 32), for
// b = 0..B, with len(b) = cu[b+1] - cu[b] after clamping cu to [0, total].
// One workgroup scans the sequences in chunks of 256 (Hillis-Steele in LDS).
__global__ __attribute__((amdgpu_flat_work_group_size(kScanThreads, kScanThreads)))
void scale_offsets_kernel(const int* __restrict__ cu, int B, int total, int align, int* __restrict__ off) {
  __shared__ int buf[kScanThreads];
  const int tid = threadIdx.x;
  const int per = align / 32;
  int carry = 0;
  for (int base = 0; base <= B; base += kScanThreads) {
    const int b = base + tid;
    int v = 0;
    if (b < B) {
      const int s = min(max(cu[b], 0), total);
      const int e = min(max(cu[b + 1], s), total);
      v = (e - s + align - 1) / align * per;
    }
    buf[tid] = v;
    __syncthreads();
    for (int w = 1; w < kScanThreads; w <<= 1) {
      const int add = tid >= w ? buf[tid - w] : 0;
      __syncthreads();
      buf[tid] += add;
      __syncthreads();
    }
    if (b <= B) off[b] = carry + buf[tid] - v;
    carry += buf[kScanThreads - 1];
    __syncthreads();  // buf is rewritten by the next chunk
  }
}

// One workgroup per sequence: destination rows dst_off[b] .. dst_off[b+1]-1
// (clamped to [0, dst_rows]) receive the sequence's ceil(len / 32) source rows
// from src_off[b] in order; the remaining (padding) rows, and rows whose source
// lies past src_rows, get E8M0 127 (scale 1). Rows are copied as 32-bit words.
__global__ __attribute__((amdgpu_flat_work_group_size(256, 256)))
void scale_scatter_kernel(const uint32_t* __restrict__ src, const int* __restrict__ src_off, int src_rows,
                          uint32_t* __restrict__ dst, const int* __restrict__ dst_off, int dst_rows,
                          const int* __restrict__ cu, int total, int words_per_row) {
  const int b = blockIdx.x;
  const int s = min(max(cu[b], 0), total);
  const int e = min(max(cu[b + 1], s), total);
  const int nblk = (e - s + 31) / 32;
  const int d0 = min(max(dst_off[b], 0), dst_rows);
  const int d1 = min(max(dst_off[b + 1], d0), dst_rows);
  const int s0 = src_off[b];
  const long long n = (long long)(d1 - d0) * words_per_row;
  for (long long i = threadIdx.x; i < n; i += blockDim.x) {
    const int r = (int)(i / words_per_row), w = (int)(i - (long long)r * words_per_row);
    const long long sr = (long long)s0 + r;
    const bool have = r < nblk && sr >= 0 && sr < src_rows;
    dst[(size_t)(d0 + r) * words_per_row + w] = have ? src[(size_t)sr * words_per_row + w] : 0x7F7F7F7Fu;
  }
}

}  // namespace

hipError_t launch_scale_offsets(const int* cu, int B, int total, int align, int* off, hipStream_t stream) {
  hipLaunchKernelGGL(scale_offsets_kernel, dim3(1), dim3(kScanThreads), 0, stream, cu, B, total, align, off);
  return hipGetLastError();
}

hipError_t launch_scale_scatter(const uint8_t* src, const int* src_off, int src_rows, uint8_t* dst,
                                const int* dst_off, int dst_rows, const int* cu, int B, int total, int row_bytes,
                                hipStream_t stream) {
  hipLaunchKernelGGL(scale_scatter_kernel, dim3((unsigned)B), dim3(256), 0, stream, (const uint32_t*)src, src_off,
                     src_rows, (uint32_t*)dst, dst_off, dst_rows, cu, total, row_bytes / 4);
  return hipGetLastError();
}

}  // namespace attn
