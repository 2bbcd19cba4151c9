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
// each compute unit, as for the attention kernel.  Operands: mode 0 repeats
// two fixed, low-entropy fragments; mode 1 cycles through eight fragments of
// pseudo-random N(0,1)-like bf16 values per lane (a matrix unit's power draw,
// and with it the clock the chip can hold, depends on the operand bits).
__device__ inline float probe_normal(uint32_t x) {
  // Sum of four uniforms from a 32-bit integer hash (approximately normal).
  float acc = 0.f;
#pragma unroll
  for (int r = 0; r < 4; ++r) {
    x ^= x >> 16;
    x *= 0x7feb352du;
    x ^= x >> 15;
    x *= 0x846ca68bu;
    x ^= x >> 16;
    acc += (float)(x >> 8) * (1.0f / 16777216.0f);
  }
  return (acc - 2.0f) * 1.7320508f;
}

__global__ __launch_bounds__(kProbeThreads) void mfma_probe_kernel(float* sink, int64_t iters, int mode) {
  extern __shared__ char hold[];
  bf16x8 a[8], b[8];
#pragma unroll
  for (int f = 0; f < 8; ++f)
#pragma unroll
    for (int e = 0; e < 8; ++e) {
      const uint32_t key = ((blockIdx.x * kProbeThreads + threadIdx.x) * 8u + f) * 8u + e;
      a[f][e] = (__bf16)(mode ? probe_normal(2u * key + 1u) : (threadIdx.x & 7) * 0.125f + e * 0.0625f);
      b[f][e] = (__bf16)(mode ? probe_normal(2u * key + 2u) : 0.5f - e * 0.03125f);
    }
  f32x16 s = {}, o0 = {}, o1 = {}, o2 = {}, o3 = {};
  for (int64_t it = 0; it < iters; ++it) {
#pragma unroll
    for (int k = 0; k < 8; ++k) s = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a[k], b[k], s, 0, 0, 0);
#pragma unroll
    for (int k = 0; k < 2; ++k) {
      o0 = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a[4 * k], b[4 * k + 1], o0, 0, 0, 0);
      o1 = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a[4 * k + 1], b[4 * k + 2], o1, 0, 0, 0);
      o2 = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a[4 * k + 2], b[4 * k + 3], o2, 0, 0, 0);
      o3 = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a[4 * k + 3], b[4 * k], o3, 0, 0, 0);
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

hipError_t launch_mfma_probe(int64_t iters, int32_t mode, float* sink, int32_t n_workgroups, hipStream_t stream) {
  hipError_t e = hipFuncSetAttribute((const void*)mfma_probe_kernel,
                                     hipFuncAttributeMaxDynamicSharedMemorySize, kProbeLds);
  if (e != hipSuccess) return e;
  hipLaunchKernelGGL(mfma_probe_kernel, dim3(n_workgroups), dim3(kProbeThreads), kProbeLds, stream, sink,
                     iters, (int)mode);
  return hipGetLastError();
}

}  // namespace ra
