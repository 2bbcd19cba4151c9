// bf16 shard forward on CDNA4 matrix cores (gfx950).
//
// One device's share of ring attention: the shard's query tile is folded
// against the key/value blocks in ring order with the online softmax
// (running max, normaliser, rescale when the max rises; "Sequence / context
// parallelism" notes, section 4; "Sequence Parallelism and Ring Attention
// Quiz", Q3 and Q7).  Blocks that would arrive over the ring are streamed
// HBM -> LDS by the buffer unit's LDS-direct loads (no register staging),
// the next tile in flight while the current one is computed (double-buffered
// LDS).  The causal mask is resolved per (block, tile) from token positions:
// tiles entirely after the query tile are never loaded, tiles entirely before
// it run unmasked, and only tiles that straddle the diagonal (or the shard
// end) apply an elementwise mask.
//
// Matrix-core formulation (v_mfma_f32_32x32x16_bf16, fp32 accumulation):
//   S^T = K Q^T    A = a 32-key slice of K (LDS, ds_read_b128), B = Q^T
//                  (registers for the whole pass).  Each lane then owns one
//                  query column and 16 of its scores, so a row max is an
//                  in-lane max plus one permlane32 swap.
//   O^T += V^T P^T A = V^T, read from the row-major V tile with the
//                  transposing LDS read (ds_read_b64_tr_b16); B = P^T taken
//                  straight from the score registers after exp2 and a bf16
//                  cast.  The key order inside each 16-key step is the score
//                  accumulator's row order, matched on the V side.
// LDS tiles are stored with an XOR swizzle of their 16-byte chunks so both
// the ds_read_b128 of K and the transposing reads of V hit distinct banks.
//
// The softmax works in the log2 domain (scale * log2 e folded into one fma
// before v_exp_f32).  The reference max only moves when a tile's max exceeds
// it by more than 8 (log2 units), so exp2 arguments stay <= 8 and the output
// rescale runs on a few tiles per row instead of every tile; l and O share
// the reference, so the result is the same up to rounding.
//
// Workgroup: NW wavefronts x NB 32-row blocks = BQ query rows of one
// (batch, head).  Each workgroup takes query tiles p and n_qtiles-1-p of the
// shard: under a causal mask their visible key counts add to a constant for
// contiguous, zig-zag and striped placement alike, so every workgroup does the
// same work (the zig-zag balancing idea applied to tiles inside one shard).
// Consecutive workgroup ids are placed on one XCD, so the query heads that
// share a key/value head stream the same K/V through one L2.
#include "ra_common.h"

namespace ra {
namespace {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x4 __attribute__((ext_vector_type(4)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef __attribute__((address_space(3))) char lds_char;

constexpr float kRescaleThreshold = 8.0f;
constexpr float kLn2 = 0.6931471805599453f;
constexpr int kBK = 64;                 // keys per tile
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
// lands at dst + 16 * i (dst is wave-uniform); out-of-range offsets read 0.
// Kept as a plain device function: the host pass of a kernel template that
// names this builtin directly emits no launch stub.
__device__ inline void lds_load16(__amdgpu_buffer_rsrc_t r, lds_char* dst, uint32_t voff) {
  __builtin_amdgcn_raw_ptr_buffer_load_lds(r, dst, 16, voff, 0, 0, 0);
}

template <int D, int NW, int NB>
struct Cfg {
  static constexpr int NT = NW * 64;
  static constexpr int BQ = NW * NB * 32;
  static constexpr int ROWB = D * 2;                  // bytes per K / V row
  static constexpr int CHUNKS = ROWB / 16;            // 16-byte chunks per row
  static constexpr int TILEB = kBK * ROWB;            // bytes per K or V tile
  static constexpr int STAGEB = 2 * TILEB;            // K tile then V tile
  static constexpr int RPI = 1024 / ROWB;             // rows per 64-lane 16-byte load
  static constexpr int LOADS = TILEB / 1024 / NW;     // loads per wave per tile, each tensor
  static_assert(LOADS >= 1 && TILEB % (1024 * NW) == 0, "tile must split evenly over waves");
  static_assert(D == 64 || D == 128, "head_dim");

  // 16-byte slot holding chunk c of tile row r (an involution in c).
  // K: rows r..r+15 read at one chunk land in 16 different slots.
  __device__ static int k_slot(int r, int c) { return c ^ (r & (CHUNKS - 1)); }
  // V: the transposing reads of a half-wave touch rows r..r+3 (4 chunks each
  // for d = 128); moving each row's chunk group keeps them apart.
  __device__ static int v_slot(int r, int c) {
    return D == 128 ? c ^ ((r & 3) << 2) : c ^ (((r >> 1) & 1) << 2);
  }
};

template <int D, int NW, int NB, typename OutT>
__global__ __launch_bounds__(NW * 64) void fwd_bf16_kernel(FwdParams p) {
  using C = Cfg<D, NW, NB>;
  __shared__ __attribute__((aligned(1024))) char smem[2 * C::STAGEB];
  lds_char* const lds = (lds_char*)smem;

  const int tid = threadIdx.x;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
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
  const int kv_bytes = n_loc * C::ROWB;  // one (batch, kv head) slice of a block

  // LDS-direct load roles: lane -> (row in its 1 KiB group, 16-byte slot).
  const int ld_row = lane / C::CHUNKS;
  const int ld_slot = lane % C::CHUNKS;

  // Transposing-read roles for V: 16-lane group qg, lane jj inside it.
  const int qg = lane >> 4, jj = lane & 15;
  const int v_row = 4 * g + (jj >> 2);           // + 16 * step (+ 8 for the high half)
  const int v_d = 16 * (qg & 1) + 4 * (jj & 3);  // + 32 * d-block

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
      posq[nb] = ok ? token_pos32(p.rank, row, n_loc, p.c, p.split) : -1;  // -1: past the shard end
      const __bf16* qp = (const __bf16*)p.q + (q_off + (ok ? row : 0)) * D + g * 8;
#pragma unroll
      for (int s = 0; s < D / 16; ++s) qreg[nb][s] = ok ? *(const bf16x8*)(qp + s * 16) : bf16x8{};
    }

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
      n_vis = (c_last + kBK - 1) / kBK;
      n_full = rows_full ? c_first / kBK : 0;
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

    // Put tile (t, kt)'s K and V into LDS stage `st`.  Rows past the shard
    // end fall outside the buffer resource and read as zeros.
    auto issue_loads = [&](int st, int t, int kt) {
      const __amdgpu_buffer_rsrc_t rk = __builtin_amdgcn_make_buffer_rsrc(
          (void*)((const __bf16*)p.k[t] + kv_off), (short)0, kv_bytes, kRsrcWord3);
      const __amdgpu_buffer_rsrc_t rv = __builtin_amdgcn_make_buffer_rsrc(
          (void*)((const __bf16*)p.v[t] + kv_off), (short)0, kv_bytes, kRsrcWord3);
      lds_char* kdst = lds + st * C::STAGEB;
      lds_char* vdst = kdst + C::TILEB;
#pragma unroll
      for (int u = 0; u < C::LOADS; ++u) {
        const int grp = wave * C::LOADS + u;  // 1 KiB group of the tile
        const int row = grp * C::RPI + ld_row;
        const uint32_t rowoff = (uint32_t)(kt * kBK + row) * C::ROWB;
        lds_load16(rk, kdst + grp * 1024, rowoff + C::k_slot(row, ld_slot) * 16);
        lds_load16(rv, vdst + grp * 1024, rowoff + C::v_slot(row, ld_slot) * 16);
      }
    };

    if (cur_t < p.n_blocks) issue_loads(0, cur_t, cur_kt);
    asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
    __syncthreads();
    int st = 0;

    while (cur_t < p.n_blocks) {
      // Advance a copy of the iterator and put the next tile's loads in flight.
      int nt = cur_t, nkt = cur_kt + 1, nvis = cur_vis, nfull = cur_full;
      if (nkt >= nvis) next_block(nt, nkt, nvis, nfull);
      const bool has_next = nt < p.n_blocks;
      if (has_next) issue_loads(st ^ 1, nt, nkt);

      const lds_char* ks = lds + st * C::STAGEB;
      const lds_char* vs = ks + C::TILEB;

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
          const int row = mb * 32 + lc;
          const bf16x8 a = *(const __attribute__((address_space(3))) bf16x8*)(
              ks + row * C::ROWB + C::k_slot(row, 2 * s + g) * 16);
#pragma unroll
          for (int nb = 0; nb < NB; ++nb)
            sacc[mb][nb] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, qreg[nb][s], sacc[mb][nb], 0, 0, 0);
        }
      }

      // Elementwise mask on tiles that straddle the diagonal or the shard end.
      // Key positions ascend inside a block, so the keys a query sees there
      // are the block's first count_upto(j, pos_q) rows: one bound per row.
      // Accumulator element i of block mb is key mb*32 + (i/4)*8 + g*4 + i%4.
      if (cur_kt >= cur_full) {
        const int j = p.owner[cur_t];
        int lim[NB];
#pragma unroll
        for (int nb = 0; nb < NB; ++nb) {
          const int cnt = posq[nb] < 0 ? 0
                          : (p.causal ? count_upto32(j, posq[nb], n_loc, p.c, p.split) : n_loc);
          lim[nb] = cnt - cur_kt * kBK - g * 4;
        }
#pragma unroll
        for (int mb = 0; mb < 2; ++mb)
#pragma unroll
          for (int i = 0; i < 16; ++i) {
            const int off = mb * 32 + (i / 4) * 8 + (i % 4);
#pragma unroll
            for (int nb = 0; nb < NB; ++nb) {
              const bool vis = off < lim[nb];
              pairs_partial += vis ? 1u : 0u;
              sacc[mb][nb][i] = vis ? sacc[mb][nb][i] : -INFINITY;
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
          for (int hh = 0; hh < 2; ++hh) {
            bf16x8 v8;
#pragma unroll
            for (int e = 0; e < 8; ++e) {
              const float pe = __builtin_amdgcn_exp2f(
                  __builtin_fmaf(sacc[mb][nb][hh * 8 + e], p.scale_log2, -msub));
              ls += pe;
              v8[e] = (__bf16)pe;
            }
            pb[nb][mb * 2 + hh] = v8;
          }
        l_part[nb] += ls;
      }

      // O^T += V^T P^T, 16 keys per MFMA step.
#pragma unroll
      for (int db = 0; db < D / 32; ++db) {
#pragma unroll
        for (int k16 = 0; k16 < 4; ++k16) {
          const int row = k16 * 16 + v_row;
          const int d = db * 32 + v_d;
          const int off = row * C::ROWB + C::v_slot(row, d >> 3) * 16 + (d & 7) * 2;
          const bf16x4 lo = __builtin_amdgcn_ds_read_tr16_b64_v4bf16(
              (__attribute__((address_space(3))) bf16x4*)(vs + off));
          const bf16x4 hi = __builtin_amdgcn_ds_read_tr16_b64_v4bf16(
              (__attribute__((address_space(3))) bf16x4*)(vs + off + 8 * C::ROWB));
          const bf16x8 a = __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7);
#pragma unroll
          for (int nb = 0; nb < NB; ++nb)
            oacc[db][nb] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, pb[nb][k16], oacc[db][nb], 0, 0, 0);
        }
      }

      // The next tile's LDS-direct loads must have landed before anyone
      // reads that stage, and this stage must be drained before it is
      // refilled: one wait and one barrier per tile.
      asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
      __syncthreads();
      st ^= 1;
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
        const int n_vis = (c_last + kBK - 1) / kBK;
        const int n_full = rows_full ? c_first / kBK : 0;
        t_full += n_full;
        t_part += n_vis - n_full;
        t_skip += p.n_ktiles - n_vis;
        pairs_full += (unsigned long long)n_full * C::BQ * kBK;
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

constexpr int kNW = 4, kNB = 2;

template <int D, typename OutT>
hipError_t launch_one(const FwdParams& p, hipStream_t stream) {
  using C = Cfg<D, kNW, kNB>;
  const int64_t grid = (int64_t)p.batch * p.h_q * p.n_pairs;
  if (grid > 0x7fffffff) return hipErrorInvalidConfiguration;
  hipLaunchKernelGGL((fwd_bf16_kernel<D, kNW, kNB, OutT>), dim3((unsigned)grid), dim3(C::NT), 0,
                     stream, p);
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
