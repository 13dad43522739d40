// attn_exp2.hip -- runs the attention kernels' own device exp2 (hardware or
// software path, from attn_device.h) over a buffer, so the software exp2 can
// be checked element by element against its float32 definition.
#include "attn_device.h"
#include "attn_internal.h"

namespace attn {
namespace {

template <int DEG>
__global__ __attribute__((amdgpu_flat_work_group_size(256, 256)))
void exp2_kernel(const float* __restrict__ x, float* __restrict__ y, long n) {
  const long stride = (long)gridDim.x * blockDim.x;
  for (long i = (long)blockIdx.x * blockDim.x + threadIdx.x; i < n; i += stride)
    y[i] = DEG == 0 ? exp2_hw(x[i]) : exp2_emu_deg<DEG == 0 ? 3 : DEG>(x[i]);
}

}  // namespace

hipError_t launch_exp2(const float* x, float* y, long n, int degree, hipStream_t stream) {
  if (n <= 0) return hipSuccess;
  long blocks = (n + 255) / 256;
  if (blocks > 8192) blocks = 8192;
  switch (degree) {
    case 0: hipLaunchKernelGGL((exp2_kernel<0>), dim3((unsigned)blocks), dim3(256), 0, stream, x, y, n); break;
    case 3: hipLaunchKernelGGL((exp2_kernel<3>), dim3((unsigned)blocks), dim3(256), 0, stream, x, y, n); break;
    case 4: hipLaunchKernelGGL((exp2_kernel<4>), dim3((unsigned)blocks), dim3(256), 0, stream, x, y, n); break;
    case 5: hipLaunchKernelGGL((exp2_kernel<5>), dim3((unsigned)blocks), dim3(256), 0, stream, x, y, n); break;
    default: return hipErrorInvalidValue;
  }
  return hipGetLastError();
}

}  // namespace attn
