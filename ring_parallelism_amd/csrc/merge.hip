// Merge of partial (out, lse) results over disjoint key sets.
//
// LSE = log sum_k exp(lse_k), out = sum_k exp(lse_k - LSE) out_k: the fold a
// ring step applies to the state it carries ("Sequence / context
// parallelism" notes, section 4).  Parts with lse = -inf hold no keys; a row
// whose parts are all -inf yields (0, -inf).
//
// HBM-bound: each thread owns 4 consecutive elements of one row (16-byte fp32
// or 8-byte bf16 accesses) and consecutive threads cover consecutive memory,
// so every wavefront reads and writes contiguous bytes.  The parts are folded
// in one pass with a running max (the weights of earlier parts are rescaled
// when a later lse is larger), so each part's data and lse are loaded
// together and nothing waits on a separate max pass.
#include "ra_common.h"

namespace ra {
namespace {

typedef __bf16 bf16x4 __attribute__((ext_vector_type(4)));

template <typename T>
__device__ inline float4 load4(const void* base, int64_t idx) {
  if constexpr (sizeof(T) == 4) {
    return *(const float4*)((const float*)base + idx);
  } else {
    const bf16x4 v = *(const bf16x4*)((const __bf16*)base + idx);
    return float4{(float)v[0], (float)v[1], (float)v[2], (float)v[3]};
  }
}

template <typename T>
__device__ inline void store4(void* base, int64_t idx, float4 x) {
  if constexpr (sizeof(T) == 4) {
    *(float4*)((float*)base + idx) = x;
  } else {
    bf16x4 v;
    v[0] = (__bf16)x.x;
    v[1] = (__bf16)x.y;
    v[2] = (__bf16)x.z;
    v[3] = (__bf16)x.w;
    *(bf16x4*)((__bf16*)base + idx) = v;
  }
}

template <typename PartT, typename OutT>
__global__ __launch_bounds__(256) void merge_kernel(MergeParams p, int row_shift, int64_t total) {
  const int64_t u = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;  // 4-element group
  if (u >= total) return;
  const int64_t r = u >> row_shift;  // head_dim / 4 groups per row (a power of two)
  const int64_t idx = u * 4;
  float m = -INFINITY, z = 0.f;
  float4 acc = {0.f, 0.f, 0.f, 0.f};
  for (int k = 0; k < p.n_parts; ++k) {
    const void* ok = p.strided ? (const void*)((const PartT*)p.outs_base + k * p.out_stride) : p.outs[k];
    const float* lk = p.strided ? p.lses_base + k * p.lse_stride : p.lses[k];
    const float l = lk[r];
    const float4 o = load4<PartT>(ok, idx);
    if (l == -INFINITY) continue;  // no keys in this part (its out is not read)
    if (l > m) {
      const float s = expf(m - l);  // 0 while m = -inf
      acc.x *= s;
      acc.y *= s;
      acc.z *= s;
      acc.w *= s;
      z *= s;
      m = l;
    }
    const float w = expf(l - m);
    z += w;
    acc.x = fmaf(w, o.x, acc.x);
    acc.y = fmaf(w, o.y, acc.y);
    acc.z = fmaf(w, o.z, acc.z);
    acc.w = fmaf(w, o.w, acc.w);
  }
  const float inv = z > 0.f ? 1.f / z : 0.f;
  // A thread writes only the elements (and lse) it has read, so out/lse may
  // alias part 0.
  store4<OutT>(p.out, idx, float4{acc.x * inv, acc.y * inv, acc.z * inv, acc.w * inv});
  if ((u & ((1 << row_shift) - 1)) == 0) p.lse[r] = z > 0.f ? m + logf(z) : -INFINITY;
}

}  // namespace

hipError_t launch_merge(const MergeParams& p, int32_t parts_dtype, int32_t out_dtype,
                        hipStream_t stream) {
  const int per_row = p.head_dim / 4;  // a power of two (head_dim is a multiple of 4 dividing 256)
  int shift = 0;
  while ((1 << shift) < per_row) ++shift;
  if ((1 << shift) != per_row) return hipErrorInvalidValue;
  const int64_t total = p.n_rows * per_row;
  const int64_t grid = (total + 255) / 256;
  if (grid > 0x7fffffff) return hipErrorInvalidConfiguration;
  const dim3 gd((unsigned)grid), bd(256);
  if (parts_dtype == RA_F32 && out_dtype == RA_F32)
    hipLaunchKernelGGL((merge_kernel<float, float>), gd, bd, 0, stream, p, shift, total);
  else if (parts_dtype == RA_F32)
    hipLaunchKernelGGL((merge_kernel<float, __bf16>), gd, bd, 0, stream, p, shift, total);
  else if (out_dtype == RA_F32)
    hipLaunchKernelGGL((merge_kernel<__bf16, float>), gd, bd, 0, stream, p, shift, total);
  else
    hipLaunchKernelGGL((merge_kernel<__bf16, __bf16>), gd, bd, 0, stream, p, shift, total);
  return hipGetLastError();
}

}  // namespace ra
