// Device-side building blocks shared by the bf16 attention kernels (gfx950):
// vector types, half-wave reductions, the LDS-direct buffer load, compile-time
// loops, and the XOR swizzles of the K / V tiles in LDS.
#ifndef RA_TILE_COMMON_H
#define RA_TILE_COMMON_H

#include <type_traits>

namespace ra {
namespace {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x4 __attribute__((ext_vector_type(4)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef __attribute__((address_space(3))) char lds_char;
typedef __attribute__((address_space(3))) unsigned int lds_u32;

constexpr float kLn2 = 0.6931471805599453f;
constexpr int kRsrcWord3 = 0x00020000;  // raw buffer resource, 32-bit data format

// Combine a value across the two half-waves (lanes l and l ^ 32).  The swap
// returns the pair {own, partner} (in an order that depends on the half), so
// max and sum of the pair are the same in both halves, bit for bit.
__device__ inline float halves_max(float x) {
  auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return fmaxf(__uint_as_float(r[0]), __uint_as_float(r[1]));
}

__device__ inline float halves_sum(float x) {
  auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return __uint_as_float(r[0]) + __uint_as_float(r[1]);
}

// 16 bytes per lane from a buffer resource straight into LDS: lane i's data
// lands at dst + 16 * i (dst is wave-uniform); the byte offset is the lane's
// voff plus the wave-uniform soff, and out-of-range offsets read 0.
// Kept as a plain device function: the host pass of a kernel template that
// names this builtin directly emits no launch stub.
__device__ inline void lds_load16(__amdgpu_buffer_rsrc_t r, lds_char* dst, uint32_t voff, uint32_t soff) {
  __builtin_amdgcn_raw_ptr_buffer_load_lds(r, dst, 16, voff, soff, 0, 0);
}
// The same with the non-temporal (streaming) cache policy (cache-policy
// operand bit 1, "nt"), for data that is read once.
__device__ inline void lds_load16_nt(__amdgpu_buffer_rsrc_t r, lds_char* dst, uint32_t voff, uint32_t soff) {
  __builtin_amdgcn_raw_ptr_buffer_load_lds(r, dst, 16, voff, soff, 0, 2);
}

template <int V>
using Ic = std::integral_constant<int, V>;

// Calls f(Ic<I>), f(Ic<I+1>), ..., f(Ic<N-1>) while each call returns true.
template <int I, int N, typename F>
__device__ inline bool unrolled_steps(F& f) {
  if constexpr (I == N) {
    return true;
  } else {
    if (!f(Ic<I>{})) return false;
    return unrolled_steps<I + 1, N>(f);
  }
}

// Calls f(Ic<I>), ..., f(Ic<N-1>).
template <int I, int N, typename F>
__device__ inline void static_for(F&& f) {
  if constexpr (I < N) {
    f(Ic<I>{});
    static_for<I + 1, N>(f);
  }
}

// LDS layout of a tile of D-wide bf16 rows: 16-byte chunk c of row r sits
// in slot k_slot / v_slot (an involution in c), so that the reads of a tile
// hit distinct banks.
template <int D>
struct Swizzle {
  static_assert(D == 64 || D == 128, "head_dim");
  static constexpr int ROWB = D * 2;        // bytes per row
  static constexpr int CHUNKS = ROWB / 16;  // 16-byte chunks per row
  // K (ds_read_b128 of one chunk by rows r..r+15): 16 different slots.
  __device__ static int k_slot(int r, int c) { return c ^ (r & (CHUNKS - 1)); }
  // V: the transposing reads of a half-wave touch rows r..r+3 (4 chunks each
  // for d = 128); moving each row's chunk group keeps them apart.
  __device__ static int v_slot(int r, int c) {
    return D == 128 ? c ^ ((r & 3) << 2) : c ^ (((r >> 1) & 1) << 2);
  }
};

}  // namespace
}  // namespace ra

#endif  // RA_TILE_COMMON_H
