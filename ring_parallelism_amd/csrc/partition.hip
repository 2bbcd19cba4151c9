// Token placement (perm) and shard-major gather / natural-order scatter.
//
// Placement rules: contiguous runs ("Sequence / context parallelism" notes,
// section 1), zig-zag chunks k and 2c-1-k of 2c ("Splitting the Sequence",
// intro and Terms), round-robin stripes (notes, section 5).  The kernels are
// plain HBM copies: one thread per 16-, 8-, 4- or 1-byte unit, consecutive
// threads on consecutive bytes of a row so every wavefront reads and writes
// contiguous memory.
#include "ra_common.h"

namespace ra {
namespace {

__global__ void perm_kernel(int64_t S, int64_t n_loc, int32_t c, int32_t split, int64_t* perm) {
  const int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  if (i >= S) return;
  perm[i] = token_pos(i / n_loc, i % n_loc, n_loc, c, split);
}

// Unit type U moves sizeof(U) bytes; a row has units_per_row units.
// gather  (inverse == false): dst[r][o][t] = src[o][pos(r,t)]
// scatter (inverse == true):  dst[o][pos(r,t)] = src[r][o][t]
template <typename U, bool INVERSE>
__global__ void move_rows_kernel(const U* __restrict__ src, U* __restrict__ dst, int64_t S,
                                 int64_t n_loc, int32_t c, int32_t split, int64_t outer,
                                 int64_t units_per_row, int64_t total_units) {
  const int64_t stride = (int64_t)gridDim.x * blockDim.x;
  for (int64_t u = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; u < total_units; u += stride) {
    const int64_t e = u % units_per_row;
    const int64_t row = u / units_per_row;          // shard-major row index r*outer*n_loc + o*n_loc + t
    const int64_t t = row % n_loc;
    const int64_t o = (row / n_loc) % outer;
    const int64_t r = row / (n_loc * outer);
    const int64_t pos = token_pos(r, t, n_loc, c, split);
    const int64_t nat = (o * S + pos) * units_per_row + e;
    if (INVERSE)
      dst[nat] = src[u];
    else
      dst[u] = src[nat];
  }
}

template <bool INVERSE>
hipError_t launch_move(const void* src, void* dst, int64_t S, int64_t n_loc, int32_t c,
                       int32_t split, int64_t outer, int64_t inner_bytes, hipStream_t stream) {
  const uintptr_t a = (uintptr_t)src | (uintptr_t)dst | (uintptr_t)inner_bytes;
  const int threads = 256;
  auto grid_for = [&](int64_t units) {
    int64_t g = (units + threads - 1) / threads;
    return (unsigned)(g > 65536 * 4 ? 65536 * 4 : g);
  };
  if (a % 16 == 0) {
    const int64_t upr = inner_bytes / 16, tot = upr * S * outer;
    hipLaunchKernelGGL((move_rows_kernel<uint4, INVERSE>), dim3(grid_for(tot)), dim3(threads), 0,
                       stream, (const uint4*)src, (uint4*)dst, S, n_loc, c, split, outer, upr, tot);
  } else if (a % 8 == 0) {
    const int64_t upr = inner_bytes / 8, tot = upr * S * outer;
    hipLaunchKernelGGL((move_rows_kernel<uint2, INVERSE>), dim3(grid_for(tot)), dim3(threads), 0,
                       stream, (const uint2*)src, (uint2*)dst, S, n_loc, c, split, outer, upr, tot);
  } else if (a % 4 == 0) {
    const int64_t upr = inner_bytes / 4, tot = upr * S * outer;
    hipLaunchKernelGGL((move_rows_kernel<uint32_t, INVERSE>), dim3(grid_for(tot)), dim3(threads),
                       0, stream, (const uint32_t*)src, (uint32_t*)dst, S, n_loc, c, split, outer,
                       upr, tot);
  } else {
    const int64_t upr = inner_bytes, tot = upr * S * outer;
    hipLaunchKernelGGL((move_rows_kernel<uint8_t, INVERSE>), dim3(grid_for(tot)), dim3(threads),
                       0, stream, (const uint8_t*)src, (uint8_t*)dst, S, n_loc, c, split, outer,
                       upr, tot);
  }
  return hipGetLastError();
}

}  // namespace

hipError_t launch_partition(int64_t S, int32_t c, int32_t split, int64_t* perm, const void* src,
                            void* dst, int64_t outer, int64_t inner_bytes, bool inverse,
                            hipStream_t stream) {
  const int64_t n_loc = S / c;
  if (perm) {
    const int threads = 256;
    hipLaunchKernelGGL(perm_kernel, dim3((unsigned)((S + threads - 1) / threads)), dim3(threads),
                       0, stream, S, n_loc, c, split, perm);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
  }
  if (src && dst) {
    return inverse ? launch_move<true>(src, dst, S, n_loc, c, split, outer, inner_bytes, stream)
                   : launch_move<false>(src, dst, S, n_loc, c, split, outer, inner_bytes, stream);
  }
  return hipSuccess;
}

}  // namespace ra
