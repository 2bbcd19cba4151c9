// Measurement aid, not part of the attention library: a stream of
// independent 32x32x16 bf16 matrix-core products on operands held in
// registers, with no memory traffic inside the loop.  It gives the rate the
// chip sustains on the matrix cores alone for a given operand distribution
// (the board's power limit lowers the clock when the operand bits switch a
// lot), to set beside the attention kernel's rate on the same data.
//
// Each thread makes its 64 bf16 operand values once (A fragments 0..3, then
// B fragments 0..3) from a per-thread xorshift32 stream (Marsaglia, "Xorshift
// RNGs", J. Stat. Softw. 8(14), 2003), each value the sum of four uniforms
// on [-0.5, 0.5) scaled to unit variance (the Irwin-Hall approximation of
// N(0, 1)), or zero; then every wave issues 16 products per iteration into
// four accumulators (no product waits for the one before it).  Operands
// made in the kernel rather than loaded: with loaded operands the compiler's
// register assignment held the same loop to about 70 % of the rate even on
// zero operands.
#include <hip/hip_runtime.h>

#include <cstdint>

namespace {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x16 __attribute__((ext_vector_type(16)));

constexpr int kThreads = 512;  // 8 waves: two per SIMD

__device__ inline uint32_t xorshift32(uint32_t x) {
  x ^= x << 13;
  x ^= x >> 17;
  x ^= x << 5;
  return x;
}

__device__ inline float unit_normal(uint32_t& state) {
  float sum = 0.f;
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    state = xorshift32(state);
    sum += (float)(state >> 8) * (1.0f / 16777216.0f) - 0.5f;
  }
  return sum * 1.7320508f;  // the sum of four U(-1/2, 1/2) has variance 1/3
}

__global__ __launch_bounds__(kThreads) void mfma_stream_kernel(int iters, int zero_operands, uint32_t seed,
                                                                float* __restrict__ out) {
  const uint32_t tid = blockIdx.x * kThreads + threadIdx.x;
  // Per-thread start: Knuth's multiplicative hash of the thread id (the
  // golden-ratio multiplier, The Art of Computer Programming vol. 3, 6.4).
  uint32_t state = (tid + 1u) * 2654435761u ^ seed;
  state = state ? state : 1u;  // xorshift32 never leaves a nonzero state, never reaches one from zero
  bf16x8 a[4], b[4];
#pragma unroll
  for (int i = 0; i < 4; ++i)
#pragma unroll
    for (int e = 0; e < 8; ++e) {
      const float va = unit_normal(state), vb = unit_normal(state);
      a[i][e] = (__bf16)(zero_operands ? 0.f : va);
      b[i][e] = (__bf16)(zero_operands ? 0.f : vb);
    }
  f32x16 c0 = {}, c1 = {}, c2 = {}, c3 = {};
  for (int it = 0; it < iters; ++it) {
#pragma unroll
    for (int s = 0; s < 4; ++s) {
      c0 = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a[s], b[s], c0, 0, 0, 0);
      c1 = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a[(s + 1) & 3], b[s], c1, 0, 0, 0);
      c2 = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a[(s + 2) & 3], b[s], c2, 0, 0, 0);
      c3 = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a[(s + 3) & 3], b[s], c3, 0, 0, 0);
    }
  }
  float r = 0.f;
#pragma unroll
  for (int i = 0; i < 16; ++i) r += c0[i] + c1[i] + c2[i] + c3[i];
  out[tid] = r;  // keeps the products live
}

}  // namespace

// out: n_wg * 512 floats (device).  Returns a hipError_t code.  FLOP per
// launch: n_wg * 8 waves * iters * 16 products * 32 * 32 * 16 * 2.
extern "C" int mfma_stream(int n_wg, int iters, int zero_operands, uint32_t seed, float* out, void* stream) {
  if (!out || n_wg < 1 || iters < 0) return (int)hipErrorInvalidValue;
  hipLaunchKernelGGL(mfma_stream_kernel, dim3((unsigned)n_wg), dim3(kThreads), 0, (hipStream_t)stream, iters,
                     zero_operands, seed, out);
  return (int)hipGetLastError();
}
