// attn_exp2.hip -- runs the attention kernels' own device exp2 (hardware or
// software path, from attn_device.h) over a buffer, so the software exp2 can
// be checked element by element against its float32 definition.
#include "attn_device.h"
#include "attn_internal.h"

namespace attn {
namespace {

template <bool EMU>
__global__ __attribute__((amdgpu_flat_work_group_size(256, 256)))
void exp2_kernel(const float* __restrict__ x, float* __restrict__ y, long n) {
  const long stride = (long)gridDim.x * blockDim.x;
  for (long i = (long)blockIdx.x * blockDim.x + threadIdx.x; i < n; i += stride)
    y[i] = EMU ? exp2_emu(x[i]) : exp2_hw(x[i]);
}

}  // namespace

hipError_t launch_exp2(const float* x, float* y, long n, int emulated, hipStream_t stream) {
  if (n <= 0) return hipSuccess;
  long blocks = (n + 255) / 256;
  if (blocks > 8192) blocks = 8192;
  if (emulated)
    hipLaunchKernelGGL((exp2_kernel<true>), dim3((unsigned)blocks), dim3(256), 0, stream, x, y, n);
  else
    hipLaunchKernelGGL((exp2_kernel<false>), dim3((unsigned)blocks), dim3(256), 0, stream, x, y, n);
  return hipGetLastError();
}

}  // namespace attn
