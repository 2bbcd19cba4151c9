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

typedef float f32x4 __attribute__((ext_vector_type(4)));

// Parts are read once: non-temporal loads (streaming cache policy).
template <typename T>
__device__ inline float4 load4(const void* base, int64_t idx) {
  if constexpr (sizeof(T) == 4) {
    const f32x4 v = __builtin_nontemporal_load((const f32x4*)((const float*)base + idx));
    return float4{v[0], v[1], v[2], v[3]};
  } else {
    const bf16x4 v = __builtin_nontemporal_load((const bf16x4*)((const __bf16*)base + idx));
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

// G threads per 4-element group (G = 1, or 8 for merges of many parts over
// few rows): thread j of a group folds parts j, j+G, j+2G, ..., then the G
// states are combined by lane exchanges and thread 0 writes.
template <typename PartT, typename OutT, int G>
__global__ __launch_bounds__(256) void merge_kernel(MergeParams p, int row_shift, int64_t total) {
  const int64_t t = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  const int64_t u = t / G;  // 4-element group (G divides 64: a group never straddles a wavefront)
  const int j = (int)(t % G);
  if (u >= total) return;
  const int64_t r = u >> row_shift;  // head_dim / 4 groups per row (a power of two)
  const int64_t idx = u * 4;
  float m = -INFINITY, z = 0.f;
  float4 acc = {0.f, 0.f, 0.f, 0.f};
  auto part_out = [&](int k) -> const void* {
    return p.strided ? (const void*)((const PartT*)p.outs_base + k * p.out_stride) : p.outs[k];
  };
  auto part_lse = [&](int k) -> const float* { return p.strided ? p.lses_base + k * p.lse_stride : p.lses[k]; };
  auto fold = [&](float l, const float4& o) {
    if (l == -INFINITY) return;  // no keys in this part
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
  };
  // This thread's parts in chunks of KU: a chunk's loads are all issued
  // before its fold, so many-part merges wait for memory once per chunk.
  constexpr int KU = 8;
  int k = j;
  for (; k + (KU - 1) * G < p.n_parts; k += KU * G) {
    float lv[KU];
    float4 ov[KU];
#pragma unroll
    for (int q = 0; q < KU; ++q) {
      lv[q] = part_lse(k + q * G)[r];
      ov[q] = load4<PartT>(part_out(k + q * G), idx);
    }
#pragma unroll
    for (int q = 0; q < KU; ++q) fold(lv[q], ov[q]);
  }
  for (; k < p.n_parts; k += G) fold(part_lse(k)[r], load4<PartT>(part_out(k), idx));
  if constexpr (G > 1) {
#pragma unroll
    for (int off = 1; off < G; off <<= 1) {
      const float m2 = __shfl_xor(m, off), z2 = __shfl_xor(z, off);
      const float4 a2 = {__shfl_xor(acc.x, off), __shfl_xor(acc.y, off), __shfl_xor(acc.z, off),
                         __shfl_xor(acc.w, off)};
      const float mn = fmaxf(m, m2);
      if (mn != -INFINITY) {  // both empty: stay (0, -inf)
        const float s1 = expf(m - mn), s2 = expf(m2 - mn);
        z = z * s1 + z2 * s2;
        acc = float4{acc.x * s1 + a2.x * s2, acc.y * s1 + a2.y * s2, acc.z * s1 + a2.z * s2,
                     acc.w * s1 + a2.w * s2};
        m = mn;
      }
    }
    if (j != 0) return;
  }
  const float inv = z > 0.f ? 1.f / z : 0.f;
  // A group writes only the elements (and lse) its thread 0 has read, so out
  // may alias part 0; lse may alias part 0's lse only with G = 1 (a row's
  // groups are then in one wavefront, which reads before it writes).
  store4<OutT>(p.out, idx, float4{acc.x * inv, acc.y * inv, acc.z * inv, acc.w * inv});
  if ((u & ((1 << row_shift) - 1)) == 0) p.lse[r] = z > 0.f ? m + logf(z) : -INFINITY;
}

template <int G>
void launch_merge_g(const MergeParams& p, int32_t parts_dtype, int32_t out_dtype, int shift, int64_t total,
                    hipStream_t stream, dim3 gd, dim3 bd) {
  if (parts_dtype == RA_F32 && out_dtype == RA_F32)
    hipLaunchKernelGGL((merge_kernel<float, float, G>), gd, bd, 0, stream, p, shift, total);
  else if (parts_dtype == RA_F32)
    hipLaunchKernelGGL((merge_kernel<float, __bf16, G>), gd, bd, 0, stream, p, shift, total);
  else if (out_dtype == RA_F32)
    hipLaunchKernelGGL((merge_kernel<__bf16, float, G>), gd, bd, 0, stream, p, shift, total);
  else
    hipLaunchKernelGGL((merge_kernel<__bf16, __bf16, G>), gd, bd, 0, stream, p, shift, total);
}

}  // namespace

hipError_t launch_merge(const MergeParams& p, int32_t parts_dtype, int32_t out_dtype,
                        hipStream_t stream) {
  const int per_row = p.head_dim / 4;  // a power of two (head_dim is a multiple of 4 dividing 256)
  int shift = 0;
  while ((1 << shift) < per_row) ++shift;
  if ((1 << shift) != per_row) return hipErrorInvalidValue;
  const int64_t total = p.n_rows * per_row;
  // Many parts over few rows: spread each group's parts over 8 threads,
  // unless lse is written in place over part 0's (a row then spans several
  // wavefronts, and one could overwrite a value another has yet to read).
  const bool lse_in_place = (p.strided ? p.lses_base : p.lses[0]) == p.lse;
  const int G = (p.n_parts >= 16 && total <= (int64_t)1 << 16 && !lse_in_place) ? 8 : 1;
  const int64_t grid = (total * G + 255) / 256;
  if (grid > 0x7fffffff) return hipErrorInvalidConfiguration;
  const dim3 gd((unsigned)grid), bd(256);
  if (G == 8)
    launch_merge_g<8>(p, parts_dtype, out_dtype, shift, total, stream, gd, bd);
  else
    launch_merge_g<1>(p, parts_dtype, out_dtype, shift, total, stream, gd, bd);
  return hipGetLastError();
}

}  // namespace ra
