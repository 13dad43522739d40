// issue_rates.hip -- gfx950 issue-rate microbenchmark for the attention
// kernels' design decisions (a measurement tool; the library does not use it).
//
// Measures, in shader-clock cycles (s_memtime) per wave:
//   * v_mfma_f32_32x32x16_bf16 and v_mfma_f32_16x16x32_bf16 throughput, one
//     wave per SIMD;
//   * v_fma_f32 and v_exp_f32 throughput with eight independent chains;
//   * what an MFMA issued by one wave costs a VALU wave on the same SIMD
//     (accumulator in VGPRs or in AGPRs, FMA or exp on the VALU side): the
//     question whether the exponential path co-issues with the matrix core
//     and how much vector-ALU time each MFMA takes;
//   * LDS read bandwidth with ds_read_b128 and ds_read_b64_tr_b16, and LDS
//     reads next to MFMAs of another wave.
//
// Layout: 256 workgroups x 8 waves; waves w and w + 4 of a workgroup run on
// the same SIMD. Waves 0-3 run the FIRST job, waves 4-7 the SECOND. Every
// loop has a fixed trip count; the only global memory touched is the output
// and cycle arrays (one entry per thread / per wave); every LDS address lies
// inside the 64 KiB array (lane * 16 + offset <= 1008 + 7168 + 16).
//
// Build and run: python -m online_softmax_fwd_amd.microbench
#include <hip/hip_runtime.h>

#include <cstdio>
#include <cstdlib>

namespace {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float floatx16 __attribute__((ext_vector_type(16)));
typedef float floatx4 __attribute__((ext_vector_type(4)));
typedef unsigned u32x4 __attribute__((ext_vector_type(4)));

#define CHECK(x)                                                                   \
  do {                                                                             \
    hipError_t e_ = (x);                                                           \
    if (e_ != hipSuccess) {                                                        \
      std::printf("HIP error %s at line %d\n", hipGetErrorString(e_), __LINE__);   \
      std::exit(1);                                                                \
    }                                                                              \
  } while (0)

constexpr int kGrid = 256, kThreads = 512;
constexpr int kMfma = 4096;   // 32x32x16 MFMAs per MFMA wave (twice as many 16x16x32)
constexpr int kValu = 8192;   // groups of eight VALU instructions per VALU wave
constexpr int kLds = 2048;    // groups of eight LDS reads per LDS wave

enum Job { NONE = 0, MFMA32_V = 1, MFMA32_A = 2, MFMA16_V = 4, FMA = 8, EXP = 16, LDS128 = 32, LDSTR = 64 };

__device__ float run_mfma(int job, int lane, float seed) {
  bf16x8 a, b;
#pragma unroll
  for (int i = 0; i < 8; ++i) {
    a[i] = (__bf16)(seed * (float)(lane & 7) + (float)i);
    b[i] = (__bf16)(seed - (float)i);
  }
  float res = 0.0f;
  if (job == MFMA16_V) {
    floatx4 c0 = {}, c1 = {}, c2 = {}, c3 = {};
    for (int it = 0; it < kMfma / 2; ++it) {
      asm volatile("v_mfma_f32_16x16x32_bf16 %0, %1, %2, %0" : "+v"(c0) : "v"(a), "v"(b));
      asm volatile("v_mfma_f32_16x16x32_bf16 %0, %1, %2, %0" : "+v"(c1) : "v"(a), "v"(b));
      asm volatile("v_mfma_f32_16x16x32_bf16 %0, %1, %2, %0" : "+v"(c2) : "v"(a), "v"(b));
      asm volatile("v_mfma_f32_16x16x32_bf16 %0, %1, %2, %0" : "+v"(c3) : "v"(a), "v"(b));
    }
#pragma unroll
    for (int i = 0; i < 4; ++i) res += c0[i] + c1[i] + c2[i] + c3[i];
    return res;
  }
  floatx16 c0 = {}, c1 = {}, c2 = {}, c3 = {};
  if (job == MFMA32_V) {
    for (int it = 0; it < kMfma / 4; ++it) {
      asm volatile("v_mfma_f32_32x32x16_bf16 %0, %1, %2, %0" : "+v"(c0) : "v"(a), "v"(b));
      asm volatile("v_mfma_f32_32x32x16_bf16 %0, %1, %2, %0" : "+v"(c1) : "v"(a), "v"(b));
      asm volatile("v_mfma_f32_32x32x16_bf16 %0, %1, %2, %0" : "+v"(c2) : "v"(a), "v"(b));
      asm volatile("v_mfma_f32_32x32x16_bf16 %0, %1, %2, %0" : "+v"(c3) : "v"(a), "v"(b));
    }
  } else {
    for (int it = 0; it < kMfma / 4; ++it) {
      asm volatile("v_mfma_f32_32x32x16_bf16 %0, %1, %2, %0" : "+a"(c0) : "v"(a), "v"(b));
      asm volatile("v_mfma_f32_32x32x16_bf16 %0, %1, %2, %0" : "+a"(c1) : "v"(a), "v"(b));
      asm volatile("v_mfma_f32_32x32x16_bf16 %0, %1, %2, %0" : "+a"(c2) : "v"(a), "v"(b));
      asm volatile("v_mfma_f32_32x32x16_bf16 %0, %1, %2, %0" : "+a"(c3) : "v"(a), "v"(b));
    }
  }
#pragma unroll
  for (int i = 0; i < 16; ++i) res += c0[i] + c1[i] + c2[i] + c3[i];
  return res;
}

__device__ float run_valu(int job, int tid, float seed) {
  float x0 = seed * 1e-3f + (float)tid * 1e-6f, x1 = 2.0f * x0, x2 = 3.0f * x0, x3 = 4.0f * x0;
  float x4 = 5.0f * x0, x5 = 6.0f * x0, x6 = 7.0f * x0, x7 = 8.0f * x0;
  if (job == FMA) {
    for (int it = 0; it < kValu; ++it)
      asm volatile(
          "v_fma_f32 %0, %0, 0.5, 1.0\n\tv_fma_f32 %1, %1, 0.5, 1.0\n\tv_fma_f32 %2, %2, 0.5, 1.0\n\t"
          "v_fma_f32 %3, %3, 0.5, 1.0\n\tv_fma_f32 %4, %4, 0.5, 1.0\n\tv_fma_f32 %5, %5, 0.5, 1.0\n\t"
          "v_fma_f32 %6, %6, 0.5, 1.0\n\tv_fma_f32 %7, %7, 0.5, 1.0"
          : "+v"(x0), "+v"(x1), "+v"(x2), "+v"(x3), "+v"(x4), "+v"(x5), "+v"(x6), "+v"(x7));
  } else {
    for (int it = 0; it < kValu; ++it)
      asm volatile(
          "v_exp_f32 %0, %0\n\tv_exp_f32 %1, %1\n\tv_exp_f32 %2, %2\n\tv_exp_f32 %3, %3\n\t"
          "v_exp_f32 %4, %4\n\tv_exp_f32 %5, %5\n\tv_exp_f32 %6, %6\n\tv_exp_f32 %7, %7"
          : "+v"(x0), "+v"(x1), "+v"(x2), "+v"(x3), "+v"(x4), "+v"(x5), "+v"(x6), "+v"(x7));
  }
  return x0 + x1 + x2 + x3 + x4 + x5 + x6 + x7;
}

// Eight reads per group, conflict-free (each 16- or 32-lane group reads 256
// contiguous bytes), at most four in flight before the group's wait.
__device__ float run_lds(int job, int lane, const char* lds) {
  const unsigned base = (unsigned)(size_t)(const __attribute__((address_space(3))) char*)lds;
  if (job == LDS128) {
    const unsigned addr = base + (unsigned)lane * 16u;
    u32x4 r;
    for (int it = 0; it < kLds; ++it)
      asm volatile(
          "ds_read_b128 %0, %1 offset:0\n\tds_read_b128 %0, %1 offset:1024\n\t"
          "ds_read_b128 %0, %1 offset:2048\n\tds_read_b128 %0, %1 offset:3072\n\t"
          "ds_read_b128 %0, %1 offset:4096\n\tds_read_b128 %0, %1 offset:5120\n\t"
          "ds_read_b128 %0, %1 offset:6144\n\tds_read_b128 %0, %1 offset:7168\n\t"
          "s_waitcnt lgkmcnt(4)"
          : "=v"(r)
          : "v"(addr)
          : "memory");
    asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");
    return __builtin_bit_cast(float, r[0]);
  }
  const unsigned addr = base + (unsigned)lane * 8u;
  unsigned long long r;
  for (int it = 0; it < kLds; ++it)
    asm volatile(
        "ds_read_b64_tr_b16 %0, %1 offset:0\n\tds_read_b64_tr_b16 %0, %1 offset:512\n\t"
        "ds_read_b64_tr_b16 %0, %1 offset:1024\n\tds_read_b64_tr_b16 %0, %1 offset:1536\n\t"
        "ds_read_b64_tr_b16 %0, %1 offset:2048\n\tds_read_b64_tr_b16 %0, %1 offset:2560\n\t"
        "ds_read_b64_tr_b16 %0, %1 offset:3072\n\tds_read_b64_tr_b16 %0, %1 offset:3584\n\t"
        "s_waitcnt lgkmcnt(4)"
        : "=v"(r)
        : "v"(addr)
        : "memory");
  asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");
  return (float)(r & 0xffffu);
}

template <int FIRST, int SECOND>
__global__ __attribute__((amdgpu_flat_work_group_size(kThreads, kThreads))) void probe(float* out, long long* cyc,
                                                                                        float seed) {
  __shared__ __attribute__((aligned(1024))) char lds[65536];
  const int tid = threadIdx.x, w = tid >> 6, lane = tid & 63;
  const int job = w < 4 ? FIRST : SECOND;
  for (int i = tid; i < 65536 / 4; i += kThreads) ((float*)lds)[i] = (float)i;
  __syncthreads();
  const long long t0 = clock64();
  float res = 0.0f;
  if (job & (MFMA32_V | MFMA32_A | MFMA16_V)) res = run_mfma(job, lane, seed);
  if (job & (FMA | EXP)) res = run_valu(job, tid, seed);
  if (job & (LDS128 | LDSTR)) res = run_lds(job, lane, lds);
  const long long t1 = clock64();
  out[blockIdx.x * kThreads + tid] = res;
  if (lane == 0) cyc[blockIdx.x * 8 + w] = t1 - t0;
}

struct Result {
  double first, second;  // mean cycles per wave of waves 0-3 and 4-7 (0 when idle)
};

template <int F, int S>
Result run(float* out, long long* cyc, long long* host) {
  for (int r = 0; r < 3; ++r) hipLaunchKernelGGL((probe<F, S>), dim3(kGrid), dim3(kThreads), 0, 0, out, cyc, 1.0f);
  CHECK(hipGetLastError());
  CHECK(hipDeviceSynchronize());
  CHECK(hipMemcpy(host, cyc, kGrid * 8 * sizeof(long long), hipMemcpyDeviceToHost));
  double a = 0, b = 0;
  for (int i = 0; i < kGrid; ++i)
    for (int w = 0; w < 8; ++w) (w < 4 ? a : b) += (double)host[i * 8 + w];
  return {F ? a / (4 * kGrid) : 0.0, S ? b / (4 * kGrid) : 0.0};
}

}  // namespace

int main() {
  float* out;
  long long* cyc;
  long long* host = (long long*)std::malloc(kGrid * 8 * sizeof(long long));
  CHECK(hipMalloc(&out, kGrid * kThreads * sizeof(float)));
  CHECK(hipMalloc(&cyc, kGrid * 8 * sizeof(long long)));
  for (int r = 0; r < 10; ++r) run<MFMA32_V, FMA>(out, cyc, host);  // clocks up

  const double nv = 8.0 * kValu, nm = kMfma;
  const Result m32 = run<MFMA32_V, NONE>(out, cyc, host);
  const Result m32a = run<MFMA32_A, NONE>(out, cyc, host);
  const Result m16 = run<MFMA16_V, NONE>(out, cyc, host);
  const Result fma = run<NONE, FMA>(out, cyc, host);
  const Result ex = run<NONE, EXP>(out, cyc, host);
  std::printf("alone, one wave per SIMD (cycles per instruction):\n");
  std::printf("  v_mfma_f32_32x32x16_bf16, acc in VGPRs  %6.2f\n", m32.first / nm);
  std::printf("  v_mfma_f32_32x32x16_bf16, acc in AGPRs  %6.2f\n", m32a.first / nm);
  std::printf("  v_mfma_f32_16x16x32_bf16                %6.2f\n", m16.first / (2 * nm));
  std::printf("  v_fma_f32 (8 chains)                    %6.2f\n", fma.second / nv);
  std::printf("  v_exp_f32 (8 chains)                    %6.2f\n", ex.second / nv);

  struct Pair {
    const char* name;
    Result r;
    double alone, mfmas;
  };
  const Pair pairs[] = {
      {"32x32x16 (VGPR acc) + v_fma_f32", run<MFMA32_V, FMA>(out, cyc, host), fma.second, nm},
      {"32x32x16 (AGPR acc) + v_fma_f32", run<MFMA32_A, FMA>(out, cyc, host), fma.second, nm},
      {"16x16x32 (VGPR acc) + v_fma_f32", run<MFMA16_V, FMA>(out, cyc, host), fma.second, 2 * nm},
      {"32x32x16 (VGPR acc) + v_exp_f32", run<MFMA32_V, EXP>(out, cyc, host), ex.second, nm},
      {"32x32x16 (AGPR acc) + v_exp_f32", run<MFMA32_A, EXP>(out, cyc, host), ex.second, nm},
  };
  std::printf("MFMA wave + VALU wave on the same SIMD:\n");
  for (const Pair& p : pairs)
    std::printf("  %-34s MFMA wave %6.2f cycles/MFMA; VALU wave +%5.2f cycles per MFMA of the other wave\n",
                p.name, p.r.first / p.mfmas, (p.r.second - p.alone) / p.mfmas);

  const double lds128 = 8.0 * 1024 * kLds, ldstr = 8.0 * 512 * kLds;  // bytes per LDS wave
  const Result l8 = run<LDS128, LDS128>(out, cyc, host);
  const Result l4 = run<LDS128, NONE>(out, cyc, host);
  const Result t8 = run<LDSTR, LDSTR>(out, cyc, host);
  const Result ml = run<MFMA32_A, LDS128>(out, cyc, host);
  std::printf("LDS reads (bytes per clock per CU, from the slowest wave group):\n");
  std::printf("  ds_read_b128, 8 waves          %6.1f\n", 8 * lds128 / (l8.first > l8.second ? l8.first : l8.second));
  std::printf("  ds_read_b128, 4 waves          %6.1f\n", 4 * lds128 / l4.first);
  std::printf("  ds_read_b64_tr_b16, 8 waves    %6.1f\n", 8 * ldstr / (t8.first > t8.second ? t8.first : t8.second));
  std::printf("  ds_read_b128 (4 waves) next to 32x32x16 MFMAs (4 waves): MFMA %6.2f cycles/MFMA, LDS %6.1f B/clk\n",
              ml.first / nm, 4 * lds128 / ml.second);
  std::free(host);
  return 0;
}
