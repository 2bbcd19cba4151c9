// Matrix-core calibration probe (gfx950): the v_mfma_f32_32x32x16_bf16 mix of
// one attention step, with no memory traffic, so that the sustained bf16 MFMA
// rate of the device can be timed beside the attention kernel.
#include "ra_common.h"

namespace ra {
namespace {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x16 __attribute__((ext_vector_type(16)));

// Per iteration and wave: one dependent chain of eight products (the score
// product's shape) and four chains of two (the value product's shape).  The
// dynamic LDS allocation keeps one workgroup (eight waves, two per SIMD) on
// each compute unit, as for the attention kernel.
__global__ __launch_bounds__(kProbeThreads) void mfma_probe_kernel(float* sink, int64_t iters) {
  extern __shared__ char hold[];
  bf16x8 a, b;
#pragma unroll
  for (int e = 0; e < 8; ++e) {
    a[e] = (__bf16)((threadIdx.x & 7) * 0.125f + e * 0.0625f);
    b[e] = (__bf16)(0.5f - e * 0.03125f);
  }
  f32x16 s = {}, o0 = {}, o1 = {}, o2 = {}, o3 = {};
  for (int64_t it = 0; it < iters; ++it) {
#pragma unroll
    for (int k = 0; k < 8; ++k) s = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, s, 0, 0, 0);
#pragma unroll
    for (int k = 0; k < 2; ++k) {
      o0 = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, o0, 0, 0, 0);
      o1 = __builtin_amdgcn_mfma_f32_32x32x16_bf16(b, a, o1, 0, 0, 0);
      o2 = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, a, o2, 0, 0, 0);
      o3 = __builtin_amdgcn_mfma_f32_32x32x16_bf16(b, b, o3, 0, 0, 0);
    }
  }
  float acc = hold[0] * 0.f;
#pragma unroll
  for (int i = 0; i < 16; ++i) acc += s[i] + o0[i] + o1[i] + o2[i] + o3[i];
  sink[(int64_t)blockIdx.x * kProbeThreads + threadIdx.x] = acc;
}

constexpr int kProbeLds = 96 * 1024;

}  // namespace

double mfma_probe_flop(int64_t iters, int32_t n_workgroups) {
  // 16 products of 32 x 32 x 16 per iteration and wave, 2 FLOP per multiply-add.
  return 2.0 * 32 * 32 * 16 * 16 * (double)iters * (kProbeThreads / 64) * n_workgroups;
}

hipError_t launch_mfma_probe(int64_t iters, float* sink, int32_t n_workgroups, hipStream_t stream) {
  hipError_t e = hipFuncSetAttribute((const void*)mfma_probe_kernel,
                                     hipFuncAttributeMaxDynamicSharedMemorySize, kProbeLds);
  if (e != hipSuccess) return e;
  hipLaunchKernelGGL(mfma_probe_kernel, dim3(n_workgroups), dim3(kProbeThreads), kProbeLds, stream, sink,
                     iters);
  return hipGetLastError();
}

}  // namespace ra
