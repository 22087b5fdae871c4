// MFMA-throughput microbenchmark for the roofline of the GEMM kernels: every wave
// issues v_mfma_f32_32x32x16_bf16 back to back on four independent accumulator
// sets with register operands, so the matrix cores run with no memory or LDS
// traffic. Its rate under full load is the MFMA peak the part reaches at the clock
// it sustains, reported beside the data-sheet peak.
#include "forge_internal.h"

namespace forge {

typedef float f32x16 __attribute__((ext_vector_type(16)));

constexpr int kProbeThreads = 256;   // 4 waves
constexpr int kProbeMfmaPerIter = 8;  // per wave: 2 on each of 4 accumulator sets

// out[thread] = sum of the thread's 64 accumulator values. With every element of A
// equal to a and of B equal to b, each accumulator element gains 16 a b per MFMA,
// so out = 2 * iters * 4 * 16 elements * 16 a b = 2048 iters a b.
__global__ __launch_bounds__(kProbeThreads) void mfma_peak_kernel(float* out, int32_t iters, float a, float b) {
  bf16x8 av, bv;
#pragma unroll
  for (int j = 0; j < 8; ++j) {
    av[j] = (__bf16)a;
    bv[j] = (__bf16)b;
  }
  f32x16 acc0 = {}, acc1 = {}, acc2 = {}, acc3 = {};
  for (int it = 0; it < iters; ++it) {
#pragma unroll
    for (int r = 0; r < 2; ++r) {
      acc0 = __builtin_amdgcn_mfma_f32_32x32x16_bf16(av, bv, acc0, 0, 0, 0);
      acc1 = __builtin_amdgcn_mfma_f32_32x32x16_bf16(av, bv, acc1, 0, 0, 0);
      acc2 = __builtin_amdgcn_mfma_f32_32x32x16_bf16(av, bv, acc2, 0, 0, 0);
      acc3 = __builtin_amdgcn_mfma_f32_32x32x16_bf16(av, bv, acc3, 0, 0, 0);
    }
  }
  float s = 0.f;
#pragma unroll
  for (int e = 0; e < 16; ++e) s += (acc0[e] + acc1[e]) + (acc2[e] + acc3[e]);
  out[(int64_t)blockIdx.x * kProbeThreads + threadIdx.x] = s;
}

}  // namespace forge

using namespace forge;

extern "C" {

int forge_mfma_peak(float* out, int32_t n_workgroups, int32_t iters, float a, float b, forge_stream_t stream) {
  if (!out) return FORGE_ERR_NULL;
  if (n_workgroups < 1 || n_workgroups > (1 << 20) || iters < 1 || iters > (1 << 24)) return FORGE_ERR_UNSUPPORTED;
  if ((uintptr_t)out & 3u) return FORGE_ERR_ALIGN;
  hipLaunchKernelGGL(mfma_peak_kernel, dim3((unsigned)n_workgroups), dim3(kProbeThreads), 0,
                     static_cast<hipStream_t>(stream), out, iters, a, b);
  return hipGetLastError() == hipSuccess ? FORGE_OK : FORGE_ERR_HIP;
}

double forge_mfma_peak_flops(int32_t n_workgroups, int32_t iters) {
  return 2.0 * 32 * 32 * 16 * (double)kProbeMfmaPerIter * iters * (kProbeThreads / 64) * (double)n_workgroups;
}

}  // extern "C"
