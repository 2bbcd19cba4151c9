// Split-KV decode on CDNA4 matrix cores (gfx950).
//
// Decode has one query token per sequence, so the parallelism is over the
// keys: the key/value cache spread over the ring's devices is cut into
// ranges, each range yields a partial (out, lse), and the partials are
// gathered and folded ("Sequence / context parallelism" notes, section 7:
// decode over a distributed cache is a split-K with a gather of partial
// results).  The new token follows every cached key, so no key is masked.
//
// One wavefront per (block, key range, batch, kv head).  Its 32 MFMA columns
// are the g = h_q / h_kv query heads that share the kv head (zero-padded to
// 32; the padding columns are computed and dropped), so one pass over the
// range's K and V serves the whole group.  Per 32-key tile:
//   S^T = K Q^T      (v_mfma_f32_32x32x16_bf16; K from LDS, Q^T in registers)
//   online softmax   (per column: tile max over the 32 keys, rescale of O and
//                     l when the max rises, exp2 in the log2 domain)
//   O^T += V^T P^T   (V^T by transposing LDS reads, P^T from the registers).
// The wave streams its range HBM -> LDS with LDS-direct buffer loads into a
// private ring of tiles (no workgroup barriers): the next tiles are in flight
// while tile j is computed.  HBM-bound: K and V are read once, with the
// non-temporal cache policy (measured 13 % faster than the default policy).
#include "ra_common.h"
#include "tile_common.h"

namespace ra {
namespace {

#ifndef RA_DEC_WAVES
#define RA_DEC_WAVES 4
#endif
#ifndef RA_DEC_STAGES
#define RA_DEC_STAGES 2
#endif
constexpr int kDecWaves = RA_DEC_WAVES;    // independent waves per workgroup
constexpr int kDecStages = RA_DEC_STAGES;  // tiles in each wave's LDS ring

template <int D>
__global__ __launch_bounds__(kDecWaves * 64) void decode_kernel(DecodeParams p) {
  using Z = Swizzle<D>;
  constexpr int ROWB = Z::ROWB;
  constexpr int TILEB = 32 * ROWB;         // one 32-key K or V tile
  constexpr int LOADS = TILEB / 1024;      // 1 KiB LDS-direct loads per tensor per tile
  constexpr int RPI = 1024 / ROWB;         // rows per load
  constexpr int WAVEB = kDecStages * 2 * TILEB;  // the wave's ring of K and V tiles
  static_assert(kDecStages >= 2 && kDecStages <= 4, "ring depth");
  __shared__ __attribute__((aligned(1024))) char smem[kDecWaves * WAVEB];

  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int lane = threadIdx.x & 63;
  const int lc = lane & 31;  // MFMA column: query head of the group
  const int g = lane >> 5;   // half-wave
  const int item = blockIdx.x * kDecWaves + wave;
  if (item >= p.n_items) return;  // waves are independent: no barrier follows

  const int hk = item % p.h_kv;
  const int b = (item / p.h_kv) % p.batch;
  const int part = item / (p.h_kv * p.batch);
  const int t = part / p.n_splits;
  const int sp = part % p.n_splits;
  const int64_t n = p.n_loc;
  const int64_t k0 = sp * n / p.n_splits, k1 = (sp + 1) * n / p.n_splits;
  const int n_keys = (int)(k1 - k0);
  const int n_tiles = (n_keys + 31) / 32;

  const int64_t kv_off = ((int64_t)b * p.h_kv + hk) * n * D;
  const __amdgpu_buffer_rsrc_t rk = __builtin_amdgcn_make_buffer_rsrc(
      (void*)((const __bf16*)p.k[t] + kv_off), (short)0, (int)(uint32_t)(n * ROWB), kRsrcWord3);
  const __amdgpu_buffer_rsrc_t rv = __builtin_amdgcn_make_buffer_rsrc(
      (void*)((const __bf16*)p.v[t] + kv_off), (short)0, (int)(uint32_t)(n * ROWB), kRsrcWord3);
  lds_char* base = (lds_char*)smem + wave * WAVEB;  // stage s: K at s * 2 * TILEB, V after it

  // LDS-direct load roles: lane -> (row in its 1 KiB group, 16-byte slot).
  const int ld_row = lane / Z::CHUNKS, ld_slot = lane % Z::CHUNKS;
  // The tile offset is part of each lane's offset (not the scalar offset,
  // which the buffer range check does not cover), so rows past the block end
  // read as zeros: the last tile of a range may run past it.
  auto issue = [&](int j, int st) {
    const uint32_t toff = (uint32_t)(k0 + 32 * j) * ROWB;
#pragma unroll
    for (int u = 0; u < LOADS; ++u) {
      const int row = u * RPI + ld_row;
      lds_load16_nt(rk, base + st * 2 * TILEB + u * 1024, toff + row * ROWB + Z::k_slot(row, ld_slot) * 16, 0);
      lds_load16_nt(rv, base + st * 2 * TILEB + TILEB + u * 1024,
                    toff + row * ROWB + Z::v_slot(row, ld_slot) * 16, 0);
    }
  };

  // Q^T fragments: column lc is query head hk * group + lc (zero past the group).
  const int h = hk * p.group + lc;
  const bool col_ok = lc < p.group;
  bf16x8 qreg[D / 16];
  {
    const __bf16* qp = (const __bf16*)p.q + ((int64_t)b * p.h_q + (col_ok ? h : 0)) * D + g * 8;
#pragma unroll
    for (int s = 0; s < D / 16; ++s) qreg[s] = col_ok ? *(const bf16x8*)(qp + s * 16) : bf16x8{};
  }

  // Per-lane LDS read addresses in stage 0 (stage s: + s * 2 * TILEB immediate).
  const uint32_t lds0 = (uint32_t)(uintptr_t)base;
  uint32_t kaddr[D / 16];
#pragma unroll
  for (int s = 0; s < D / 16; ++s) kaddr[s] = lds0 + lc * ROWB + Z::k_slot(lc, 2 * s + g) * 16;
  const int qg = lane >> 4, jj = lane & 15;
  const int v_row = 4 * g + (jj >> 2);
  const int v_d = 16 * (qg & 1) + 4 * (jj & 3);
  uint32_t vaddr[D / 32];
#pragma unroll
  for (int db = 0; db < D / 32; ++db) {
    const int d = db * 32 + v_d;
    vaddr[db] = lds0 + TILEB + v_row * ROWB + Z::v_slot(v_row, d >> 3) * 16 + (d & 7) * 2;
  }

  f32x16 oacc[D / 32];
#pragma unroll
  for (int db = 0; db < D / 32; ++db) oacc[db] = f32x16{};
  float m = -INFINITY, l = 0.f;

  for (int j = 0; j < kDecStages && j < n_tiles; ++j) issue(j, j);

  // One tile in LDS stage ST (compile-time, so the stage offset is an immediate).
  auto tile = [&](int j, auto ST) {
    constexpr int OFF = decltype(ST)::value * 2 * TILEB;
    // The ring holds tiles j .. j+kDecStages-1: tile j has landed once at
    // most the loads of the later ones remain.
    const int later = min(kDecStages - 1, n_tiles - 1 - j);
    if (later >= 3) {
      asm volatile("s_waitcnt vmcnt(%0)" ::"n"(6 * LOADS) : "memory");
    } else if (later == 2) {
      asm volatile("s_waitcnt vmcnt(%0)" ::"n"(4 * LOADS) : "memory");
    } else if (later == 1) {
      asm volatile("s_waitcnt vmcnt(%0)" ::"n"(2 * LOADS) : "memory");
    } else {
      asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
    }
    // S^T = K Q^T (eight K reads, then the products).
    bf16x8 a[D / 16];
    static_for<0, D / 16>([&a, &kaddr](auto I) {
      asm volatile("ds_read_b128 %0, %1 offset:%2" : "=v"(a[I]) : "v"(kaddr[I]), "n"(OFF));
    });
    bf16x8 va[D / 32][2];
    static_for<0, D / 32>([&vaddr, &va](auto DB) {
      static_for<0, 2>([&vaddr, &va](auto K16) {
        constexpr int db = decltype(DB)::value, k16 = decltype(K16)::value;
        constexpr int o = OFF + k16 * 16 * ROWB;
        bf16x4 lo, hi;
        asm volatile("ds_read_b64_tr_b16 %0, %1 offset:%2" : "=v"(lo) : "v"(vaddr[db]), "n"(o));
        asm volatile("ds_read_b64_tr_b16 %0, %1 offset:%2" : "=v"(hi) : "v"(vaddr[db]), "n"(o + 8 * ROWB));
        va[db][k16] = __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7);
      });
    });
    // All of this tile's LDS reads have returned before the stage is refilled.
    static_for<0, D / 16>([&a](auto I) { asm volatile("s_waitcnt lgkmcnt(0)" : "+v"(a[I])::"memory"); });
    static_for<0, D / 32>([&va](auto DB) {
      asm volatile("s_waitcnt lgkmcnt(0)" : "+v"(va[DB][0]), "+v"(va[DB][1])::"memory");
    });
    // Tile j is in registers: its stage takes tile j+kDecStages.
    if (j + kDecStages < n_tiles) issue(j + kDecStages, decltype(ST)::value);
    f32x16 sacc = f32x16{};
#pragma unroll
    for (int s = 0; s < D / 16; ++s) sacc = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a[s], qreg[s], sacc, 0, 0, 0);
    // Keys past the range end (last tile only) are masked.  Element i is key
    // (i/4)*8 + g*4 + i%4 of the tile.
    const int lim = n_keys - 32 * j - 4 * g;
    if (lim < 28) {
#pragma unroll
      for (int i = 0; i < 16; ++i) sacc[i] = ((i / 4) * 8 + (i % 4) < lim) ? sacc[i] : -INFINITY;
    }
    float mx = -INFINITY;
#pragma unroll
    for (int i = 0; i < 16; ++i) mx = fmaxf(mx, sacc[i]);
    const float mt = halves_max(mx) * p.scale_log2;
    const float m_new = fmaxf(m, mt);  // finite: every tile has a visible key
    if (__builtin_amdgcn_ballot_w64(m_new > m) != 0) {
      const float alpha = __builtin_amdgcn_exp2f(m - m_new);  // 0 while m = -inf
      l *= alpha;
#pragma unroll
      for (int db = 0; db < D / 32; ++db) oacc[db] *= alpha;
      m = m_new;
    }
    bf16x8 pb[2];
#pragma unroll
    for (int hh = 0; hh < 2; ++hh) {
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        const float pe = __builtin_amdgcn_exp2f(__builtin_fmaf(sacc[hh * 8 + e], p.scale_log2, -m));
        l += pe;
        pb[hh][e] = (__bf16)pe;
      }
    }
#pragma unroll
    for (int db = 0; db < D / 32; ++db) {
      oacc[db] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(va[db][0], pb[0], oacc[db], 0, 0, 0);
      oacc[db] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(va[db][1], pb[1], oacc[db], 0, 0, 0);
    }
  };
  for (int j = 0; j < n_tiles; j += kDecStages) {
    static_for<0, kDecStages>([&](auto ST) {
      if (j + decltype(ST)::value < n_tiles) tile(j + decltype(ST)::value, ST);
    });
  }

  // out = O / l for the group's heads; lse = ln 2 * (m + log2 l).
  const float lt = halves_sum(l);
  if (col_ok) {
    const float inv = lt > 0.f ? 1.f / lt : 0.f;
    float* op = p.out_parts + (((int64_t)part * p.batch + b) * p.h_q + h) * D;
#pragma unroll
    for (int db = 0; db < D / 32; ++db)
#pragma unroll
      for (int i4 = 0; i4 < 4; ++i4) {
        const int d0 = db * 32 + i4 * 8 + g * 4;
        *(float4*)(op + d0) = float4{oacc[db][i4 * 4] * inv, oacc[db][i4 * 4 + 1] * inv,
                                     oacc[db][i4 * 4 + 2] * inv, oacc[db][i4 * 4 + 3] * inv};
      }
    if (g == 0)
      p.lse_parts[((int64_t)part * p.batch + b) * p.h_q + h] =
          lt > 0.f ? (m + __log2f(lt)) * kLn2 : -INFINITY;
  }
}

}  // namespace

hipError_t launch_decode_bf16(const DecodeParams& p, int32_t head_dim, hipStream_t stream) {
  const int64_t grid = ((int64_t)p.n_items + kDecWaves - 1) / kDecWaves;
  if (grid < 1) return hipSuccess;
  if (grid > 0x7fffffff) return hipErrorInvalidConfiguration;
  if (head_dim == 128)
    hipLaunchKernelGGL(decode_kernel<128>, dim3((unsigned)grid), dim3(kDecWaves * 64), 0, stream, p);
  else
    hipLaunchKernelGGL(decode_kernel<64>, dim3((unsigned)grid), dim3(kDecWaves * 64), 0, stream, p);
  return hipGetLastError();
}

}  // namespace ra
