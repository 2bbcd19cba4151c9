// bf16 shard forward on CDNA4 matrix cores (gfx950).
//
// One device's share of ring attention: the shard's query tile is folded
// against the key/value blocks in ring order with the online softmax
// (running max, normaliser, rescale when the max rises; "Sequence / context
// parallelism" notes, section 4; "Sequence Parallelism and Ring Attention
// Quiz", Q3 and Q7).  Blocks that would arrive over the ring are streamed
// HBM -> registers -> LDS, the next tile's loads in flight while the current
// tile is computed (double-buffered LDS).  The causal mask is resolved per
// (block, tile) from token positions: tiles entirely after the query tile are
// never loaded, tiles entirely before it run unmasked, and only the few
// tiles that straddle the diagonal apply an elementwise mask.
//
// Matrix-core formulation (v_mfma_f32_32x32x16_bf16, fp32 accumulation):
//   S^T = K Q^T : A = a 32-key slice of K (LDS), B = Q^T (registers).  Each
//                 lane then owns one query column and 16 of its scores, so a
//                 row max is an in-lane max plus one permlane32 swap.
//   O^T += V^T P^T : A = V^T (LDS, stored transposed), B = P^T straight from
//                 the score registers after the exp and a bf16 cast; the key
//                 order inside each 16-key step is the accumulator's own row
//                 order, matched on the V^T side.
// The softmax works in the log2 domain (scale * log2 e folded into one fma
// before v_exp_f32).  The reference max only moves when a tile's max exceeds
// it by more than 8 (log2 units), so exp2 arguments stay <= 8 and the output
// rescale runs on a few tiles per row instead of every tile; the result is
// the same up to rounding because l and O use the same reference.
//
// Workgroup: NW wavefronts x NB 32-row blocks = BQ query rows of one
// (batch, head).  Each workgroup takes query tiles p and n_qtiles-1-p of the
// shard: under a causal mask their visible key counts add to a constant for
// both contiguous and zig-zag placement, so every workgroup does the same work
// (the zig-zag balancing idea applied to tiles inside one shard).
// Consecutive workgroup ids are placed on one XCD, so the query heads that
// share a key/value head stream the same K/V through one L2.
#include "ra_common.h"

namespace ra {
namespace {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x4 __attribute__((ext_vector_type(4)));
typedef float f32x16 __attribute__((ext_vector_type(16)));

constexpr float kRescaleThreshold = 8.0f;
constexpr float kLn2 = 0.6931471805599453f;

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

__device__ inline uint32_t word_of(const uint4& v, int i) {
  return i == 0 ? v.x : (i == 1 ? v.y : (i == 2 ? v.z : v.w));
}

template <int D, int NW, int NB, int BK>
struct Cfg {
  static constexpr int NT = NW * 64;        // threads
  static constexpr int BQ = NW * NB * 32;   // query rows per tile
  static constexpr int KSTR = D + 8;        // K row stride (bf16): +16 B keeps ds_read_b128 conflict-free
  static constexpr int VSTR = BK + 4;       // V^T row stride (bf16): +8 B keeps ds_read_b64 conflict-free
  static constexpr int KTILE = BK * KSTR;
  static constexpr int VTILE = D * VSTR;
  static constexpr int STAGE = KTILE + VTILE;
  static constexpr int KCH = BK * (D / 8) / NT;   // 16-byte K chunks per thread per tile
  static constexpr int VKPT = BK * (D / 8) / NT;  // keys per thread in the V transpose
  static constexpr int VKG = BK / VKPT;           // key groups
  static_assert(BK == 64, "two 32-key MFMA blocks per tile");
  static_assert(KCH >= 1 && BK * (D / 8) % NT == 0, "tile must split evenly over threads");
  static_assert(VKPT == 2 || VKPT == 4, "V transpose packs 2 or 4 keys");
};

template <int D, int NW, int NB, int BK, typename OutT>
__global__ __launch_bounds__(NW * 64) void fwd_bf16_kernel(FwdParams p) {
  using C = Cfg<D, NW, NB, BK>;
  __shared__ __attribute__((aligned(16))) __bf16 smem[2 * C::STAGE];

  const int tid = threadIdx.x;
  const int wave = tid >> 6;
  const int lane = tid & 63;
  const int lc = lane & 31;  // query column inside a 32-block
  const int g = lane >> 5;   // half-wave

  // XCD-aware work decode: hardware deals workgroup ids round-robin over the
  // 8 XCDs, so id -> (id % 8) * (G / 8) + id / 8 keeps consecutive logical
  // items on one XCD.
  const int G = gridDim.x;
  const int bid = blockIdx.x;
  const int wl = (G % 8 == 0) ? (bid % 8) * (G / 8) + bid / 8 : bid;
  const int h = wl % p.h_q;
  const int pair = (wl / p.h_q) % p.n_pairs;
  const int b = wl / (p.h_q * p.n_pairs);
  const int hk = h / p.group;
  const int n_loc = (int)p.n_loc;
  const int64_t kv_off = ((int64_t)b * p.h_kv + hk) * n_loc * D;
  const int64_t q_off = ((int64_t)b * p.h_q + h) * n_loc;

  // Loader thread roles.
  const int v_kg = tid % C::VKG;  // key group of the V transpose
  const int v_dc = tid / C::VKG;  // 8-wide d chunk of the V transpose

  uint32_t pairs_partial = 0;  // per lane, masked tiles only

  const int n_q = (p.n_qtiles - 1 - pair != pair) ? 2 : 1;

  for (int qi = 0; qi < n_q; ++qi) {
    const int qt = qi == 0 ? pair : p.n_qtiles - 1 - pair;
    const int i0 = qt * C::BQ;
    const bool rows_full = i0 + C::BQ <= n_loc;
    const int last_row = (rows_full ? i0 + C::BQ : n_loc) - 1;
    const int pos_first = token_pos32(p.rank, i0, n_loc, p.c, p.split);
    const int pos_last = token_pos32(p.rank, last_row, n_loc, p.c, p.split);

    // Query rows of this lane (one per 32-block) and their positions; Q^T
    // operand fragments stay in registers for the whole pass.
    int posq[NB];
    bf16x8 qreg[NB][D / 16];
#pragma unroll
    for (int nb = 0; nb < NB; ++nb) {
      const int row = i0 + (wave * NB + nb) * 32 + lc;
      const bool ok = row < n_loc;
      // Rows past the shard end get -2: below every key "position" the mask
      // uses (-1 marks any valid key when the mask is not causal).
      posq[nb] = ok ? token_pos32(p.rank, row, n_loc, p.c, p.split) : -2;
      const __bf16* qp = (const __bf16*)p.q + (q_off + (ok ? row : 0)) * D + g * 8;
#pragma unroll
      for (int s = 0; s < D / 16; ++s) qreg[nb][s] = ok ? *(const bf16x8*)(qp + s * 16) : bf16x8{};
    }

    // Online-softmax state, one query row per lane per 32-block.
    f32x16 oacc[D / 32][NB];
#pragma unroll
    for (int db = 0; db < D / 32; ++db)
#pragma unroll
      for (int nb = 0; nb < NB; ++nb) oacc[db][nb] = f32x16{};
    float m_ref[NB], l_part[NB];
#pragma unroll
    for (int nb = 0; nb < NB; ++nb) {
      m_ref[nb] = -INFINITY;
      l_part[nb] = 0.f;
    }

    // Tile iterator over (block t, key tile kt), skipping blocks with no visible key.
    auto block_counts = [&](int t, int& n_vis, int& n_full) {
      const int j = p.owner[t];
      const int c_last = p.causal ? count_upto32(j, pos_last, n_loc, p.c, p.split) : n_loc;
      const int c_first = p.causal ? count_upto32(j, pos_first, n_loc, p.c, p.split) : n_loc;
      n_vis = (c_last + BK - 1) / BK;
      n_full = rows_full ? c_first / BK : 0;
    };
    auto next_block = [&](int& t, int& kt, int& n_vis, int& n_full) {
      ++t;
      while (t < p.n_blocks) {
        block_counts(t, n_vis, n_full);
        if (n_vis > 0) break;
        ++t;
      }
      kt = 0;
    };
    int cur_t = -1, cur_kt = 0, cur_vis = 0, cur_full = 0;
    next_block(cur_t, cur_kt, cur_vis, cur_full);

    uint4 kreg[C::KCH], vreg[C::VKPT];
    auto load_regs = [&](int t, int kt) {
      const __bf16* kp = (const __bf16*)p.k[t] + kv_off;
      const __bf16* vp = (const __bf16*)p.v[t] + kv_off;
      const int key0 = kt * BK;
#pragma unroll
      for (int u = 0; u < C::KCH; ++u) {
        const int cid = tid + C::NT * u;
        const int key = key0 + cid / (D / 8), ch = cid % (D / 8);
        kreg[u] = key < n_loc ? *(const uint4*)(kp + key * D + ch * 8) : uint4{0, 0, 0, 0};
      }
#pragma unroll
      for (int u = 0; u < C::VKPT; ++u) {
        const int key = key0 + v_kg * C::VKPT + u;
        vreg[u] = key < n_loc ? *(const uint4*)(vp + key * D + v_dc * 8) : uint4{0, 0, 0, 0};
      }
    };
    auto store_lds = [&](int buf) {
      __bf16* ks = smem + buf * C::STAGE;
      __bf16* vt = ks + C::KTILE;
#pragma unroll
      for (int u = 0; u < C::KCH; ++u) {
        const int cid = tid + C::NT * u;
        const int kk = cid / (D / 8), ch = cid % (D / 8);
        *(uint4*)(ks + kk * C::KSTR + ch * 8) = kreg[u];
      }
      // Transpose: element e of the 8-wide d chunk goes to row v_dc*8+e of V^T.
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        const int sh = (e & 1) * 16;
        uint32_t pk[C::VKPT / 2];
#pragma unroll
        for (int u2 = 0; u2 < C::VKPT / 2; ++u2) {
          const uint32_t a = (word_of(vreg[2 * u2], e / 2) >> sh) & 0xffffu;
          const uint32_t c = (word_of(vreg[2 * u2 + 1], e / 2) >> sh) & 0xffffu;
          pk[u2] = a | (c << 16);
        }
        __bf16* dst = vt + (v_dc * 8 + e) * C::VSTR + v_kg * C::VKPT;
        if constexpr (C::VKPT == 4) {
          *(uint2*)dst = uint2{pk[0], pk[1]};
        } else {
          *(uint32_t*)dst = pk[0];
        }
      }
    };

    if (cur_t < p.n_blocks) {
      load_regs(cur_t, cur_kt);
      store_lds(0);
    }
    __syncthreads();
    int buf = 0;

    while (cur_t < p.n_blocks) {
      // Advance a copy of the iterator and put the next tile's loads in flight.
      int nt = cur_t, nkt = cur_kt + 1, nvis = cur_vis, nfull = cur_full;
      if (nkt >= nvis) next_block(nt, nkt, nvis, nfull);
      const bool has_next = nt < p.n_blocks;
      if (has_next) load_regs(nt, nkt);

      const __bf16* ks = smem + buf * C::STAGE;
      const __bf16* vt = ks + C::KTILE;

      // S^T = K Q^T for the tile's two 32-key blocks.
      f32x16 sacc[2][NB];
#pragma unroll
      for (int mb = 0; mb < 2; ++mb)
#pragma unroll
        for (int nb = 0; nb < NB; ++nb) sacc[mb][nb] = f32x16{};
#pragma unroll
      for (int s = 0; s < D / 16; ++s) {
#pragma unroll
        for (int mb = 0; mb < 2; ++mb) {
          const bf16x8 a = *(const bf16x8*)(ks + (mb * 32 + lc) * C::KSTR + s * 16 + g * 8);
#pragma unroll
          for (int nb = 0; nb < NB; ++nb)
            sacc[mb][nb] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, qreg[nb][s], sacc[mb][nb], 0, 0, 0);
        }
      }

      // Elementwise mask on tiles that straddle the diagonal or the shard end.
      // Accumulator element i of block mb is key mb*32 + (i/4)*8 + g*4 + i%4.
      if (cur_kt >= cur_full) {
        const int j = p.owner[cur_t];
        const int key0 = cur_kt * BK + g * 4;
#pragma unroll
        for (int mb = 0; mb < 2; ++mb)
#pragma unroll
          for (int i = 0; i < 16; ++i) {
            const int jj = key0 + mb * 32 + (i / 4) * 8 + (i % 4);
            // Keys past the shard end get a position no query reaches.
            const int pk = jj < n_loc ? (p.causal ? token_pos32(j, jj, n_loc, p.c, p.split) : -1)
                                      : 0x7fffffff;
#pragma unroll
            for (int nb = 0; nb < NB; ++nb) {
              const bool vis = pk <= posq[nb];
              pairs_partial += vis ? 1u : 0u;
              if (!vis) sacc[mb][nb][i] = -INFINITY;
            }
          }
      }

      // Online softmax (log2 domain).
      float mt[NB];
      bool need = false;
#pragma unroll
      for (int nb = 0; nb < NB; ++nb) {
        float mx = -INFINITY;
#pragma unroll
        for (int mb = 0; mb < 2; ++mb)
#pragma unroll
          for (int i = 0; i < 16; ++i) mx = fmaxf(mx, sacc[mb][nb][i]);
        mx = halves_max(mx);
        mt[nb] = mx * p.scale_log2;
        need |= mt[nb] > m_ref[nb] + kRescaleThreshold;
      }
      if (__builtin_amdgcn_ballot_w64(need) != 0) {
#pragma unroll
        for (int nb = 0; nb < NB; ++nb) {
          const float m_new = fmaxf(m_ref[nb], mt[nb]);
          const float alpha = (m_new == -INFINITY) ? 1.f : __builtin_amdgcn_exp2f(m_ref[nb] - m_new);
          l_part[nb] *= alpha;
#pragma unroll
          for (int db = 0; db < D / 32; ++db) oacc[db][nb] *= alpha;
          m_ref[nb] = m_new;
        }
      }
      bf16x8 pb[NB][4];
#pragma unroll
      for (int nb = 0; nb < NB; ++nb) {
        const float msub = (m_ref[nb] == -INFINITY) ? 0.f : m_ref[nb];
        float ls = 0.f;
#pragma unroll
        for (int mb = 0; mb < 2; ++mb)
#pragma unroll
          for (int half = 0; half < 2; ++half) {
            bf16x8 v8;
#pragma unroll
            for (int e = 0; e < 8; ++e) {
              const float pe = __builtin_amdgcn_exp2f(__builtin_fmaf(sacc[mb][nb][half * 8 + e], p.scale_log2, -msub));
              ls += pe;
              v8[e] = (__bf16)pe;
            }
            pb[nb][mb * 2 + half] = v8;
          }
        l_part[nb] += ls;
      }

      // O^T += V^T P^T, 16 keys per MFMA step.
#pragma unroll
      for (int db = 0; db < D / 32; ++db) {
#pragma unroll
        for (int ks16 = 0; ks16 < 4; ++ks16) {
          const int kb = (ks16 >> 1) * 32 + (ks16 & 1) * 16 + g * 4;
          const __bf16* vr = vt + (db * 32 + lc) * C::VSTR + kb;
          const bf16x4 lo = *(const bf16x4*)(vr);
          const bf16x4 hi = *(const bf16x4*)(vr + 8);
          const bf16x8 a = __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7);
#pragma unroll
          for (int nb = 0; nb < NB; ++nb)
            oacc[db][nb] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, pb[nb][ks16], oacc[db][nb], 0, 0, 0);
        }
      }

      if (has_next) store_lds(buf ^ 1);
      __syncthreads();
      buf ^= 1;
      cur_t = nt;
      cur_kt = nkt;
      cur_vis = nvis;
      cur_full = nfull;
    }

    // Epilogue: out = O / l, lse = ln 2 * (m_ref + log2 l).
#pragma unroll
    for (int nb = 0; nb < NB; ++nb) {
      const float lt = halves_sum(l_part[nb]);
      const float inv = lt > 0.f ? 1.f / lt : 0.f;
      const int row = i0 + (wave * NB + nb) * 32 + lc;
      if (row < n_loc) {
        const int64_t ro = q_off + row;
        OutT* op = (OutT*)p.out + ro * D;
#pragma unroll
        for (int db = 0; db < D / 32; ++db)
#pragma unroll
          for (int i4 = 0; i4 < 4; ++i4) {
            const int d0 = db * 32 + i4 * 8 + g * 4;
            if constexpr (sizeof(OutT) == 4) {
              float4 v4;
              v4.x = oacc[db][nb][i4 * 4 + 0] * inv;
              v4.y = oacc[db][nb][i4 * 4 + 1] * inv;
              v4.z = oacc[db][nb][i4 * 4 + 2] * inv;
              v4.w = oacc[db][nb][i4 * 4 + 3] * inv;
              *(float4*)(op + d0) = v4;
            } else {
              bf16x4 v4;
              v4[0] = (__bf16)(oacc[db][nb][i4 * 4 + 0] * inv);
              v4[1] = (__bf16)(oacc[db][nb][i4 * 4 + 1] * inv);
              v4[2] = (__bf16)(oacc[db][nb][i4 * 4 + 2] * inv);
              v4[3] = (__bf16)(oacc[db][nb][i4 * 4 + 3] * inv);
              *(bf16x4*)(op + d0) = v4;
            }
          }
        if (g == 0) p.lse[ro] = lt > 0.f ? (m_ref[nb] + __log2f(lt)) * kLn2 : -INFINITY;
      }
    }
  }

  if (p.stats) {
    // Tile classes and full-tile pairs are workgroup-uniform: recount them
    // here from the same per-block visible-key counts the loop used.
    unsigned long long pairs_full = 0, t_full = 0, t_part = 0, t_skip = 0;
    for (int qi = 0; qi < n_q; ++qi) {
      const int qt = qi == 0 ? pair : p.n_qtiles - 1 - pair;
      const int i0 = qt * C::BQ;
      const bool rows_full = i0 + C::BQ <= n_loc;
      const int last_row = (rows_full ? i0 + C::BQ : n_loc) - 1;
      const int pos_first = token_pos32(p.rank, i0, n_loc, p.c, p.split);
      const int pos_last = token_pos32(p.rank, last_row, n_loc, p.c, p.split);
      for (int t = 0; t < p.n_blocks; ++t) {
        const int j = p.owner[t];
        const int c_last = p.causal ? count_upto32(j, pos_last, n_loc, p.c, p.split) : n_loc;
        const int c_first = p.causal ? count_upto32(j, pos_first, n_loc, p.c, p.split) : n_loc;
        const int n_vis = (c_last + BK - 1) / BK;
        const int n_full = rows_full ? c_first / BK : 0;
        t_full += n_full;
        t_part += n_vis - n_full;
        t_skip += p.n_ktiles - n_vis;
        pairs_full += (unsigned long long)n_full * C::BQ * BK;
      }
    }
    unsigned long long v = pairs_partial;
#pragma unroll
    for (int off = 32; off > 0; off >>= 1) v += __shfl_xor(v, off);
    if (lane == 0 && v) atomicAdd(p.stats + 0, v);
    if (tid == 0) {
      atomicAdd(p.stats + 0, pairs_full);
      atomicAdd(p.stats + 1, t_full);
      atomicAdd(p.stats + 2, t_part);
      atomicAdd(p.stats + 3, t_skip);
    }
  }
}

constexpr int kNW = 4, kNB = 1, kBK = 64;

template <int D, typename OutT>
hipError_t launch_one(const FwdParams& p, hipStream_t stream) {
  using C = Cfg<D, kNW, kNB, kBK>;
  const int64_t grid = (int64_t)p.batch * p.h_q * p.n_pairs;
  if (grid > 0x7fffffff) return hipErrorInvalidConfiguration;
  hipLaunchKernelGGL((fwd_bf16_kernel<D, kNW, kNB, kBK, OutT>), dim3((unsigned)grid), dim3(C::NT),
                     0, stream, p);
  return hipGetLastError();
}

}  // namespace

void tile_shape_bf16(int32_t head_dim, int32_t* tq, int32_t* tk) {
  (void)head_dim;
  *tq = kNW * kNB * 32;
  *tk = kBK;
}

hipError_t launch_fwd_bf16(const FwdParams& p0, int32_t head_dim, int32_t out_dtype,
                           hipStream_t stream) {
  FwdParams p = p0;
  const int bq = kNW * kNB * 32;
  p.n_qtiles = (int32_t)((p.n_loc + bq - 1) / bq);
  p.n_ktiles = (int32_t)((p.n_loc + kBK - 1) / kBK);
  p.n_pairs = (p.n_qtiles + 1) / 2;
  if (head_dim == 128)
    return out_dtype == RA_F32 ? launch_one<128, float>(p, stream) : launch_one<128, __bf16>(p, stream);
  return out_dtype == RA_F32 ? launch_one<64, float>(p, stream) : launch_one<64, __bf16>(p, stream);
}

}  // namespace ra
