// bf16 shard forward on CDNA4 matrix cores (gfx950).
//
// One device's share of ring attention: the shard's query tile is folded
// against the key/value blocks in ring order with the online softmax
// (running max, normaliser, rescale when the max rises; "Sequence / context
// parallelism" notes, section 4; "Sequence Parallelism and Ring Attention
// Quiz", Q3 and Q7).  Blocks that would arrive over the ring are streamed
// HBM -> LDS by the buffer unit's LDS-direct loads (no register staging)
// into a ring of LDS stages, so that the tiles after the one being computed
// are already in flight (the prefetch that hides the ring's transfers); a
// tile's K fragments move on from LDS into registers one step before its
// score products.  The causal mask is resolved per (block, tile) from token
// positions: tiles entirely after the query tile are never loaded, tiles
// entirely before it run unmasked, and only tiles that straddle the diagonal
// (or the shard end) apply an elementwise mask.
//
// Matrix-core formulation (v_mfma_f32_32x32x16_bf16, fp32 accumulation):
//   S^T = K Q^T    A = a 32-key slice of K (LDS, ds_read_b128), B = Q^T
//                  (registers for the whole pass).  Each lane then owns one
//                  query column and 16 of its scores, so a row reduction is
//                  in-lane plus one permlane32 swap.
//   O^T += V^T P^T A = V^T, read from the row-major V tile with the
//                  transposing LDS read (ds_read_b64_tr_b16); B = P^T taken
//                  straight from the score registers after exp2 and a bf16
//                  cast.  The key order inside each 16-key step is the score
//                  accumulator's row order, matched on the V side.
// LDS tiles are stored with an XOR swizzle of their 16-byte chunks so both
// the ds_read_b128 of K and the transposing reads of V hit distinct banks.
//
// The softmax works in the log2 domain (scale * log2 e folded into one fma
// before v_exp_f32) against a per-row reference m.  Any reference gives the
// same result as long as O and l share it (O / l and m + log2 l do not
// depend on it), and nothing is lost by a reference below the running max as
// long as no exponential overflows: fp32 and bf16 keep their relative
// precision at every magnitude.  So the first tile sets m to its exact row
// max and afterwards no per-tile max is taken.  At every workgroup barrier
// (every G steps) a row whose lane sum l has passed 2^32 -- some scores rose
// more than 32 log2 units above m -- raises m by the integer part of log2 l
// and rescales O and l by that exact power of two.  Between two checks a
// score would have to jump roughly 90 log2 units or more above every earlier
// one for fp32 to overflow (an exponential, the row sum or the output); if
// that happens -- seen as a non-finite sum or output after the pass -- or a
// row of the first tile sees no key, as some block orders allow, the query
// tile is recomputed from scratch by the plain per-tile online softmax (exact
// tile max, rescale whenever it rises).
//
// Workgroup: NW wavefronts x NB 32-row blocks = BQ query rows of one
// (batch, head).  Each workgroup takes query tiles p and n_qtiles-1-p of the
// shard: under a causal mask their visible key counts add to a constant for
// contiguous, zig-zag and striped placement alike, so every workgroup does the
// same work (the zig-zag balancing idea applied to tiles inside one shard).
// Consecutive workgroup ids are placed on one XCD, so the query heads that
// share a key/value head stream the same K/V through one L2.  The grid may
// also be split over groups of blocks (each group writes a partial result to
// be merged), q / out / lse may be addressed at global token positions of
// natural-order tensors instead of shard order, and every rank's pass may run
// in one launch (the rank taken from the work index, each XCD given a slice
// of every rank).
#include <type_traits>

#include "ra_common.h"
#include "tile_common.h"

// Tile configuration: waves per workgroup, LDS ring stages, steps per
// workgroup barrier.  (Compile-time knobs for tuning sweeps.)
#ifndef RA_FWD_NW
#define RA_FWD_NW 8
#endif
#ifndef RA_FWD_STAGES
#define RA_FWD_STAGES 10
#endif
#ifndef RA_FWD_GROUP
#define RA_FWD_GROUP 4
#endif
#ifndef RA_FWD_WPE
#define RA_FWD_WPE 1
#endif

namespace ra {
namespace {

// A row's lane sum l above this raises the reference (at a barrier).
constexpr float kRaiseAt = 4294967296.0f;  // 2^32
#ifndef RA_FWD_PINP
#define RA_FWD_PINP 0
#endif
constexpr bool kPinP = RA_FWD_PINP != 0;

constexpr int gcd2(int a, int b) { return b == 0 ? a : gcd2(b, a % b); }
constexpr int lcm3(int a, int b, int c) {
  const int ab = a / gcd2(a, b) * b;
  return ab / gcd2(ab, c) * c;
}

template <int D, int NW, int NB>
struct Cfg {
  static constexpr int NT = NW * 64;
  static constexpr int BQ = NW * NB * 32;
  static constexpr int BK = 32;                       // keys per tile (one 32-key MFMA block)
  static constexpr int ROWB = D * 2;                  // bytes per K / V row
  static constexpr int CHUNKS = ROWB / 16;            // 16-byte chunks per row
  static constexpr int TILEB = BK * ROWB;             // bytes per K or V tile
  static constexpr int STAGES = RA_FWD_STAGES;        // LDS ring depth
  static constexpr int G = RA_FWD_GROUP;              // steps per barrier (loads issued G tiles at a time)
  static constexpr int AHEAD = STAGES - G;            // tiles in flight before a group's loads
  // The K fragments of tile i+2 are read during step i, so that tile must
  // have been published by the barrier of an earlier group: AHEAD >= G + 2.
  static_assert(AHEAD >= G + 2 && G >= 1 && G <= 4, "stage / group configuration");
  // Tiles of a group's loads that the next group does not read yet (they may
  // stay in flight across its closing barrier), and the matching vmcnt.
  static constexpr int LATE = (AHEAD - G - 2) < G ? (AHEAD - G - 2) : G;
  // LDS reads name their stage by the instruction's 16-bit immediate; a ring
  // longer than 64 KiB addresses its later stages from a second base 64 KiB
  // higher (a tile never straddles the boundary: 64 KiB is a whole number of
  // tiles).
  static_assert(65536 % TILEB == 0 && STAGES * TILEB <= 2 * 65536, "stage offsets");
  static_assert(2 * STAGES * TILEB <= 160 * 1024, "the ring must fit the 160 KiB of LDS");
  static_assert(NW * 4 <= TILEB, "the per-wave votes live in the last K stage");
  template <int S> static constexpr uint32_t stage_hi = (uint32_t)(S * TILEB) & ~0xffffu;
  template <int S> static constexpr int stage_lo = (S * TILEB) & 0xffff;
  static constexpr int RPI = 1024 / ROWB;             // rows per 64-lane 16-byte load
  static constexpr int LOADS = TILEB / 1024 / NW;     // loads per wave per tile, each tensor
  static_assert(LOADS >= 1 && TILEB % (1024 * NW) == 0, "tile must split evenly over waves");
  static_assert(D == 64 || D == 128, "head_dim");

  __device__ static int k_slot(int r, int c) { return Swizzle<D>::k_slot(r, c); }
  __device__ static int v_slot(int r, int c) { return Swizzle<D>::v_slot(r, c); }
};

template <int D, int NW, int NB, typename OutT>
__global__ __launch_bounds__(NW * 64, RA_FWD_WPE) void fwd_bf16_kernel(FwdParams p) {
  using C = Cfg<D, NW, NB>;
  constexpr int kBK = C::BK;
  constexpr int NS = C::STAGES;
  constexpr int G = C::G;
  // One LDS array: the K tiles of the ring stages, then their V tiles.  Every
  // LDS read of the tile loop is inline assembly with the stage offset as the
  // instruction's immediate, so per-lane addresses are computed once.  (The
  // compiler cannot tell which stage an LDS-direct load fills, and would make
  // compiler-visible reads wait for all loads in flight.)
  __shared__ __attribute__((aligned(1024))) char smem[2 * NS * C::TILEB];
  auto k_tile = [&](auto S) -> lds_char* { return (lds_char*)smem + decltype(S)::value * C::TILEB; };
  auto v_tile = [&](auto S) -> lds_char* {
    return (lds_char*)smem + (NS + decltype(S)::value) * C::TILEB;
  };

  const int tid = threadIdx.x;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int lane = tid & 63;
  const int lc = lane & 31;  // query column inside a 32-block
  const int g = lane >> 5;   // half-wave

  // XCD-aware work decode: hardware deals workgroup ids round-robin over the
  // 8 XCDs, so id -> (id % 8) * (G / 8) + id / 8 keeps consecutive logical
  // items on one XCD.
  const int n_wg = gridDim.x;
  const int bid = blockIdx.x;
  const int wl_grid = (n_wg % 8 == 0) ? (bid % 8) * (n_wg / 8) + bid / 8 : bid;
  // Every rank's ring pass in one launch: q / out / lse of a rank sit at rank
  // strides, and its block order is the ring order (owner (rank - t) mod c,
  // block table indexed by owner).  Each XCD takes the same slice of every
  // rank's work items -- so that the XCDs finish together even where the
  // ranks' work differs (causal contiguous placement) and neighbouring heads,
  // which share a key/value head, stay on one L2 -- in decreasing rank order,
  // the heaviest first under causal contiguous placement.
  int rank = p.rank, wl_all = wl_grid;
  if (p.all_ranks) {
    if (n_wg % 8 == 0 && p.grid_per_rank % 8 == 0) {
      const int per_xcd = p.grid_per_rank / 8;  // items of one rank on one XCD
      const int u = bid / 8;                    // dispatch order inside the XCD
      rank = p.c - 1 - u / per_xcd;
      wl_all = (bid % 8) * per_xcd + u % per_xcd;
    } else {
      rank = wl_grid / p.grid_per_rank;
      wl_all = wl_grid % p.grid_per_rank;
    }
  }
  // (0 <= rank, t < c, so (rank - t) mod c needs no division.)
  auto ring_owner = [&](int t) { return rank >= t ? rank - t : rank - t + p.c; };
  auto owner_of = [&](int t) { return p.all_ranks ? ring_owner(t) : p.owner[t]; };
  auto block_k = [&](int t) { return p.k[p.all_ranks ? ring_owner(t) : t]; };
  auto block_v = [&](int t) { return p.v[p.all_ranks ? ring_owner(t) : t]; };
  // Split of the block list (one group when n_splits = 1): this workgroup
  // folds blocks [t0, t1) and writes its own partial result.
  const int split = wl_all / p.grid_per_split;
  const int wl = wl_all % p.grid_per_split;
  const int t0 = split * p.n_blocks / p.n_splits, t1 = (split + 1) * p.n_blocks / p.n_splits;
  OutT* const out_base = (OutT*)p.out + split * p.part_stride_out + rank * p.rank_stride_out;
  float* const lse_base = p.lse + split * p.part_stride_lse + rank * p.rank_stride_lse;
  const __bf16* const q_base = (const __bf16*)p.q + rank * p.rank_stride_q;
  const int h = wl % p.h_q;
  const int pair = (wl / p.h_q) % p.n_pairs;
  const int b = wl / (p.h_q * p.n_pairs);
  const int hk = h / p.group;
  const int n_loc = (int)p.n_loc;
  const int64_t kv_off = ((int64_t)b * p.h_kv + hk) * n_loc * D;
  const int64_t q_off = ((int64_t)b * p.h_q + h) * p.qo_rows;  // q / out / lse rows of (b, h)
  // Bytes of one (batch, kv head) slice of a block (< 2^32: n_loc * d < 2^31).
  const int kv_bytes = (int)((uint32_t)n_loc * C::ROWB);

  // LDS-direct load roles: lane -> (row in its 1 KiB group, 16-byte slot).
  const int ld_row = lane / C::CHUNKS;
  const int ld_slot = lane % C::CHUNKS;
  // Byte offsets inside a tile (a whole number of 32-row groups: the
  // swizzles only look at the low row bits).
  uint32_t ld_koff[C::LOADS], ld_voff[C::LOADS];
#pragma unroll
  for (int u = 0; u < C::LOADS; ++u) {
    const int row = (wave * C::LOADS + u) * C::RPI + ld_row;
    ld_koff[u] = row * C::ROWB + C::k_slot(row, ld_slot) * 16;
    ld_voff[u] = row * C::ROWB + C::v_slot(row, ld_slot) * 16;
  }

  // Transposing-read roles for V: 16-lane group qg, lane jj inside it.
  const int qg = lane >> 4, jj = lane & 15;
  const int v_row = 4 * g + (jj >> 2);           // + 16 * step (+ 8 for the high half)
  const int v_d = 16 * (qg & 1) + 4 * (jj & 3);  // + 32 * d-block

  // LDS addresses of this lane's reads in stage 0 (other stages: + immediate).
  const uint32_t lds0 = (uint32_t)(uintptr_t)(lds_char*)smem;
  uint32_t kaddr[D / 16];  // K: key row lc, 16-byte chunk 2s+g
#pragma unroll
  for (int s16 = 0; s16 < D / 16; ++s16) kaddr[s16] = lds0 + lc * C::ROWB + C::k_slot(lc, 2 * s16 + g) * 16;
  uint32_t vaddr[D / 32];  // V: rows v_row (+8, +16, +24), columns v_d of d-slice db
#pragma unroll
  for (int db = 0; db < D / 32; ++db) {
    const int d = db * 32 + v_d;
    vaddr[db] = lds0 + NS * C::TILEB + v_row * C::ROWB + C::v_slot(v_row, d >> 3) * 16 + (d & 7) * 2;
  }

  uint32_t pairs_partial = 0;  // per lane, masked tiles only
  uint32_t n_raise = 0;        // per lane (g == 0 counts its row): mid-pass reference raises
  uint32_t n_exact = 0;        // query tiles recomputed by the exact path (workgroup-uniform)

  const int n_q = (p.n_qtiles - 1 - pair != pair) ? 2 : 1;

  for (int qi = 0; qi < n_q; ++qi) {
    const int qt = qi == 0 ? pair : p.n_qtiles - 1 - pair;
    const int i0 = qt * C::BQ;
    const bool rows_full = i0 + C::BQ <= n_loc;
    const int last_row = (rows_full ? i0 + C::BQ : n_loc) - 1;
    const int pos_first = token_pos32(rank, i0, n_loc, p.c, p.split);
    const int pos_last = token_pos32(rank, last_row, n_loc, p.c, p.split);

    // Query rows of this lane (one per 32-block) and their positions; Q^T
    // operand fragments stay in registers for the whole pass.
    int posq[NB];
    bf16x8 qreg[NB][D / 16];
#pragma unroll
    for (int nb = 0; nb < NB; ++nb) {
      const int row = i0 + (wave * NB + nb) * 32 + lc;
      const bool ok = row < n_loc;
      posq[nb] = ok ? token_pos32(rank, row, n_loc, p.c, p.split) : -1;  // -1: past the shard end
      const int qrow = ok ? (p.qo_natural ? posq[nb] : row) : 0;
      const __bf16* qp = q_base + (q_off + qrow) * D + g * 8;
#pragma unroll
      for (int s = 0; s < D / 16; ++s) qreg[nb][s] = ok ? *(const bf16x8*)(qp + s * 16) : bf16x8{};
    }

    f32x16 oacc[D / 32][NB];
    float m_ref[NB], l_part[NB], neg_sub[NB];
    auto reset_state = [&]() {
#pragma unroll
      for (int db = 0; db < D / 32; ++db)
#pragma unroll
        for (int nb = 0; nb < NB; ++nb) oacc[db][nb] = f32x16{};
#pragma unroll
      for (int nb = 0; nb < NB; ++nb) {
        m_ref[nb] = -INFINITY;
        l_part[nb] = 0.f;
        neg_sub[nb] = 0.f;  // -m_ref, or 0 while m_ref is -inf
      }
    };
    reset_state();

    // Tile iterator over (block t, key tile kt), skipping blocks with no
    // visible key.  A state is (t, kt, n_vis, n_full); t >= t1: done.
    // The cursor of the tile loads also carries the block's K and V base
    // addresses, read from the argument block once per block (a scalar load
    // in the per-tile path would make every tile wait for all of the wave's
    // LDS reads as well); the counting pass and the masking cursor need only
    // the counts and read no address.
    struct Tile {
      int t, kt, vis, full;
      const __bf16* kb;
      const __bf16* vb;
    };
    // Per-block tile counts of this query tile, in lanes: lane u of
    // register h holds block 64h + u's visible and full key-tile counts (0
    // outside [t0, t1)).  Computed once per query tile on the vector unit --
    // every wave would otherwise repeat the same scalar arithmetic on the
    // compute unit's one scalar unit -- and read by a cursor entering a
    // block with one v_readlane.
    int lvis[2], lfull[2];
#pragma unroll
    for (int h = 0; h < 2; ++h) {
      lvis[h] = 0;
      lfull[h] = 0;
      if (h == 0 || t1 > 64) {
        const int t = 64 * h + lane;
        if (t >= t0 && t < t1) {
          const int j = p.all_ranks ? ring_owner(t) : p.owner[t];
          const int c_last = p.causal ? count_upto32(j, pos_last, n_loc, p.c, p.split) : n_loc;
          const int c_first = p.causal ? count_upto32(j, pos_first, n_loc, p.c, p.split) : n_loc;
          lvis[h] = (c_last + kBK - 1) / kBK;
          lfull[h] = rows_full ? c_first / kBK : 0;
        }
      }
    }
    auto block_counts = [&](Tile& x) {
      const int u = x.t & 63;
      x.vis = x.t < 64 ? __builtin_amdgcn_readlane(lvis[0], u) : __builtin_amdgcn_readlane(lvis[1], u);
      x.full = x.t < 64 ? __builtin_amdgcn_readlane(lfull[0], u) : __builtin_amdgcn_readlane(lfull[1], u);
    };
    auto block_addrs = [&](Tile& x) {
      x.kb = (const __bf16*)block_k(x.t) + kv_off;
      x.vb = (const __bf16*)block_v(x.t) + kv_off;
    };
    auto advance = [&](Tile x, auto WithAddrs) {
      if (__builtin_expect(x.t >= t1, 0)) return x;
      if (__builtin_expect(++x.kt < x.vis, 1)) return x;
      x.kt = 0;
      while (++x.t < t1) {
        block_counts(x);
        if (x.vis > 0) break;
      }
      if constexpr (decltype(WithAddrs)::value != 0) {
        if (x.t < t1) block_addrs(x);
      }
      return x;
    };

    // Put tile x's K and V into LDS stage `st`.  The tile offset is part of
    // each lane's offset, so the buffer range check covers it: rows past the
    // shard end fall outside the (batch, kv head) slice and read as zeros.
    auto issue_loads = [&](auto S, const Tile& x) {
      const __amdgpu_buffer_rsrc_t rk =
          __builtin_amdgcn_make_buffer_rsrc((void*)x.kb, (short)0, kv_bytes, kRsrcWord3);
      const __amdgpu_buffer_rsrc_t rv =
          __builtin_amdgcn_make_buffer_rsrc((void*)x.vb, (short)0, kv_bytes, kRsrcWord3);
      const uint32_t tile_off = (uint32_t)(x.kt * kBK) * C::ROWB;
#pragma unroll
      for (int u = 0; u < C::LOADS; ++u) {
        const int grp = wave * C::LOADS + u;  // 1 KiB group of the tile
        lds_load16(rk, k_tile(S) + grp * 1024, ld_koff[u] + tile_off, 0);
        lds_load16(rv, v_tile(S) + grp * 1024, ld_voff[u] + tile_off, 0);
      }
    };

    // S^T = K Q^T for the tile in stage S: D/16 16-wide slices of d, up to
    // six K reads in flight ahead of the products (lgkmcnt counts LDS reads
    // in issue order, and the wait before slice s allows the reads issued
    // after it).  Used where no other LDS read is in flight.
    auto qk = [&](f32x16 (&sacc)[NB], auto S) {
      constexpr int OFF = C::template stage_lo<decltype(S)::value>;
      constexpr uint32_t HI = C::template stage_hi<decltype(S)::value>;
      constexpr int NR = D / 16, PF = NR < 6 ? NR : 6;
      bf16x8 a[NR];
#pragma unroll
      for (int nb = 0; nb < NB; ++nb) sacc[nb] = f32x16{};
      // (Explicit captures: clang does not capture variables that a generic
      // lambda uses only as inline-assembly operands.)
      static_for<0, PF>([&a, &kaddr](auto I) {
        asm volatile("ds_read_b128 %0, %1 offset:%2" : "=v"(a[I]) : "v"(kaddr[I] + HI), "n"(OFF));
      });
      static_for<0, NR>([&a, &kaddr, &sacc, &qreg](auto I) {
        constexpr int sl = decltype(I)::value;
        if constexpr (sl + PF < NR)
          asm volatile("ds_read_b128 %0, %1 offset:%2" : "=v"(a[sl + PF]) : "v"(kaddr[sl + PF] + HI), "n"(OFF));
        constexpr int issued = sl + PF < NR ? sl + PF + 1 : NR;
        asm volatile("s_waitcnt lgkmcnt(%1)" : "+v"(a[sl]) : "n"(issued - sl - 1));
#pragma unroll
        for (int nb = 0; nb < NB; ++nb)
          sacc[nb] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a[sl], qreg[nb][sl], sacc[nb], 0, 0, 0);
      });
    };

    // Elementwise mask on a tile that straddles the diagonal or the shard
    // end (works on raw or shifted scores alike).  Key positions ascend inside
    // a block, so the keys a query sees there are the block's first
    // count_upto(j, pos_q) rows: one bound per row.  Accumulator element i is
    // key (i/4)*8 + g*4 + i%4 of the tile.
    auto mask = [&](f32x16 (&sacc)[NB], const Tile& x) {
      const int j = owner_of(x.t);
      int lim[NB];
#pragma unroll
      for (int nb = 0; nb < NB; ++nb) {
        const int cnt = posq[nb] < 0 ? 0
                        : (p.causal ? count_upto32(j, posq[nb], n_loc, p.c, p.split) : n_loc);
        lim[nb] = cnt - x.kt * kBK - g * 4;
      }
#pragma unroll
      for (int i = 0; i < 16; ++i) {
        const int off = (i / 4) * 8 + (i % 4);
#pragma unroll
        for (int nb = 0; nb < NB; ++nb) {
          const bool vis = off < lim[nb];
          pairs_partial += vis ? 1u : 0u;
          sacc[nb][i] = vis ? sacc[nb][i] : -INFINITY;
        }
      }
    };

    // Tile max of the scaled scores (log2 units), both half-waves combined.
    auto row_max = [&](const f32x16 (&sacc)[NB], float (&mt)[NB]) {
#pragma unroll
      for (int nb = 0; nb < NB; ++nb) {
        float mx = -INFINITY;
#pragma unroll
        for (int i = 0; i < 16; ++i) mx = fmaxf(mx, sacc[nb][i]);
        mt[nb] = halves_max(mx) * p.scale_log2;
      }
    };

    // x = scale*log2(e)*s - m_ref, in place (m_ref = -inf: shifted by 0).
    auto shift = [&](f32x16 (&sacc)[NB]) {
#pragma unroll
      for (int nb = 0; nb < NB; ++nb)
#pragma unroll
        for (int i = 0; i < 16; ++i) sacc[nb][i] = __builtin_fmaf(sacc[nb][i], p.scale_log2, neg_sub[nb]);
    };

    // Raise the reference to the tile max mt (absolute, log2 units) where it
    // is higher: rescale O and l, and re-shift the tile's x values.
    auto rescale = [&](const float (&mt)[NB], f32x16 (&xs)[NB]) {
#pragma unroll
      for (int nb = 0; nb < NB; ++nb) {
        const float m_new = fmaxf(m_ref[nb], mt[nb]);
        const float alpha = (m_new == -INFINITY) ? 1.f : __builtin_amdgcn_exp2f(m_ref[nb] - m_new);
        const float new_neg = (m_new == -INFINITY) ? 0.f : -m_new;
        const float dx = new_neg - neg_sub[nb];
        l_part[nb] *= alpha;
#pragma unroll
        for (int db = 0; db < D / 32; ++db) oacc[db][nb] *= alpha;
#pragma unroll
        for (int i = 0; i < 16; ++i) xs[nb][i] += dx;
        m_ref[nb] = m_new;
        neg_sub[nb] = new_neg;
      }
    };

    // P = bf16(exp2(x)) as the B operand of the value product; ls gets the
    // lane's fp32 sum of the tile (the log-sum-exp needs it unrounded).
    auto exps = [&](const f32x16 (&x)[NB], bf16x8 (&pb)[NB][2], float (&ls)[NB]) {
#pragma unroll
      for (int nb = 0; nb < NB; ++nb) {
        float sum = 0.f;
#pragma unroll
        for (int hh = 0; hh < 2; ++hh) {
          bf16x8 v8;
#pragma unroll
          for (int e = 0; e < 8; ++e) {
            const float pe = __builtin_amdgcn_exp2f(x[nb][hh * 8 + e]);
            sum = (hh == 0 && e == 0) ? pe : sum + pe;
            v8[e] = (__bf16)pe;
          }
          pb[nb][hh] = v8;
        }
        ls[nb] = sum;
      }
    };

    // The transposing reads of the V tile in stage S (for each 32-wide slice
    // of d, two 16-key halves of 8 rows each).
    auto v_reads = [&vaddr](auto S, bf16x8 (&va)[D / 32][2]) {
      constexpr int OFF = C::template stage_lo<decltype(S)::value>;
      constexpr uint32_t HI = C::template stage_hi<decltype(S)::value>;
      static_for<0, D / 32>([&vaddr, &va](auto DB) {
        static_for<0, 2>([&vaddr, &va](auto K16) {
          constexpr int db = decltype(DB)::value, k16 = decltype(K16)::value;
          constexpr int o = OFF + k16 * 16 * C::ROWB;
          bf16x4 lo, hi;
          asm volatile("ds_read_b64_tr_b16 %0, %1 offset:%2" : "=v"(lo) : "v"(vaddr[db] + HI), "n"(o));
          asm volatile("ds_read_b64_tr_b16 %0, %1 offset:%2" : "=v"(hi) : "v"(vaddr[db] + HI), "n"(o + 8 * C::ROWB));
          va[db][k16] = __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7);
        });
      });
    };

    // O^T += V^T P^T, 16 keys per MFMA step, straight after v_reads (no
    // other LDS read in between: the wait before slice db lets the reads of
    // the later slices stay in flight).
    auto pv = [&](bf16x8 (&va)[D / 32][2], const bf16x8 (&pb)[NB][2]) {
      static_for<0, D / 32>([&va, &pb, this_oacc = &oacc](auto DB) {
        auto& oacc = *this_oacc;
        constexpr int db = decltype(DB)::value;
        asm volatile("s_waitcnt lgkmcnt(%2)" : "+v"(va[db][0]), "+v"(va[db][1]) : "n"(4 * (D / 32 - 1 - db)));
#pragma unroll
        for (int k16 = 0; k16 < 2; ++k16)
#pragma unroll
          for (int nb = 0; nb < NB; ++nb)
            oacc[db][nb] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(va[db][k16], pb[nb][k16], oacc[db][nb], 0, 0, 0);
      });
    };

    // The K fragments of tile i+2 are read into registers during the value
    // product of step i (that tile was published by an earlier barrier): the
    // score products of step i+1 then start without an LDS wait, and a
    // step's LDS reads split between its halves -- V beside the score
    // products, K beside the value product.
    auto k_reads = [&kaddr](auto S, bf16x8 (&kf)[D / 16]) {
      constexpr int OFF = C::template stage_lo<decltype(S)::value>;
      constexpr uint32_t HI = C::template stage_hi<decltype(S)::value>;
      static_for<0, D / 16>([&kaddr, &kf](auto I) {
        asm volatile("ds_read_b128 %0, %1 offset:%2" : "=v"(kf[I]) : "v"(kaddr[I] + HI), "n"(OFF));
      });
    };
    // S^T = K Q^T from fragments read by k_reads a step earlier (the last LDS
    // reads issued): one wait for all of them.
    auto qk_held = [&](f32x16 (&sacc)[NB], bf16x8 (&kf)[D / 16]) {
      asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");
#pragma unroll
      for (int sl = 0; sl < D / 16; ++sl) asm volatile("" : "+v"(kf[sl]));
#pragma unroll
      for (int nb = 0; nb < NB; ++nb) {
        sacc[nb] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(kf[0], qreg[nb][0], f32x16{}, 0, 0, 0);
#pragma unroll
        for (int sl = 1; sl < D / 16; ++sl)
          sacc[nb] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(kf[sl], qreg[nb][sl], sacc[nb], 0, 0, 0);
      }
    };
    // O^T += V^T P^T from V reads the caller has waited for, key half 0
    // first (it needs only the first eight exponentials of each lane).
    auto pv_held = [&](bf16x8 (&va)[D / 32][2], const bf16x8 (&pb)[NB][2]) {
#pragma unroll
      for (int k16 = 0; k16 < 2; ++k16)
#pragma unroll
        for (int db = 0; db < D / 32; ++db)
#pragma unroll
          for (int nb = 0; nb < NB; ++nb)
            oacc[db][nb] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(va[db][k16], pb[nb][k16], oacc[db][nb], 0, 0, 0);
    };

    // Raise the reference of every row whose lane sum l has passed 2^32 by
    // the integer part of log2 l (the same in both lanes of a row), with O and
    // l rescaled by that exact power of two; a non-finite l marks the query
    // tile for the exact path.
    // y (the shifted scores of the next tile) moves with the reference.
    auto raise_ref = [&](bool& bad, f32x16 (&ys)[NB]) {
#pragma unroll
      for (int nb = 0; nb < NB; ++nb) {
        const float lr = halves_max(l_part[nb]);
        const bool fin = lr < INFINITY;
        bad |= !fin;
        const int e = __builtin_amdgcn_frexp_expf(lr);  // lr = f * 2^e, f in [0.5, 1)
        const int dd = (fin && lr > kRaiseAt) ? e - 1 : 0;
        n_raise += (dd != 0 && g == 0) ? 1u : 0u;
        l_part[nb] = __builtin_ldexpf(l_part[nb], -dd);
#pragma unroll
        for (int db = 0; db < D / 32; ++db)
#pragma unroll
          for (int e2 = 0; e2 < 16; ++e2) oacc[db][nb][e2] = __builtin_ldexpf(oacc[db][nb][e2], -dd);
#pragma unroll
        for (int e2 = 0; e2 < 16; ++e2) ys[nb][e2] -= (float)dd;
        m_ref[nb] += (float)dd;
        neg_sub[nb] -= (float)dd;
      }
    };

    // The plain online softmax over every visible tile, one tile at a time
    // through LDS stage 0: exact tile max, rescale of O and l whenever it
    // rises.  Recomputes the query tile from scratch.
    f32x16 xa[NB], xb[NB];
    bf16x8 pb[NB][2], va[D / 32][2];
    float mt[NB], ls[NB];
    const uint32_t pairs_before = pairs_partial;
    auto exact_pass = [&]() {
      pairs_partial = pairs_before;
      ++n_exact;
      reset_state();
      for (int t = t0; t < t1; ++t) {
        Tile x;
        x.t = t;
        x.kt = 0;
        block_counts(x);
        if (x.vis > 0) block_addrs(x);
        for (int kt = 0; kt < x.vis; ++kt) {
          x.kt = kt;
          __syncthreads();  // every wave has finished reading stage 0
          issue_loads(Ic<0>{}, x);
          asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
          __syncthreads();
          qk(xa, Ic<0>{});
          if (kt >= x.full) mask(xa, x);
          row_max(xa, mt);
          shift(xa);
          rescale(mt, xa);
          exps(xa, pb, ls);
#pragma unroll
          for (int nb = 0; nb < NB; ++nb) l_part[nb] += ls[nb];
          v_reads(Ic<0>{}, va);
          pv(va, pb);
        }
      }
      __syncthreads();
    };

    // The first tile: loads of tiles 0 .. AHEAD-1, its scores, exact row max.
    Tile first;
    first.t = -1;
    first.kt = 0;
    first.vis = 0;
    first.full = 0;
    first.kb = first.vb = nullptr;
    int n_tiles;
    {
      int tot = lvis[0] + lvis[1];
#pragma unroll
      for (int off = 32; off > 0; off >>= 1) tot += __shfl_xor(tot, off);
      n_tiles = __builtin_amdgcn_readfirstlane(tot);
      const uint64_t m0 = __builtin_amdgcn_ballot_w64(lvis[0] > 0);
      const uint64_t m1 = __builtin_amdgcn_ballot_w64(lvis[1] > 0);
      if (m0 | m1) {
        first.t = m0 ? (int)__builtin_ctzll(m0) : 64 + (int)__builtin_ctzll(m1);
        block_counts(first);
        block_addrs(first);
      }
    }
    // Every row of the query tile sees key 0 of the first tile (so that the
    // first tile gives every row a finite reference) unless a causal mask
    // hides it from the tile's first row (positions ascend).
    const bool fast = n_tiles > 0 &&
                      (!p.causal || count_upto32(owner_of(first.t), pos_first, n_loc, p.c, p.split) >= 1);
    if (fast) {
      Tile ld = first;
      static_for<0, C::AHEAD>([&](auto I) {
        if (decltype(I)::value < n_tiles) issue_loads(I, ld);
        ld = advance(ld, Ic<1>{});
      });
      asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
      __syncthreads();

      bf16x8 kf[D / 16];  // K fragments of the next tile
      qk(xa, Ic<0>{});
      k_reads(Ic<1>{}, kf);
      if (first.kt >= first.full) mask(xa, first);
      row_max(xa, mt);
      shift(xa);
      rescale(mt, xa);  // first reference: the exact max (O and l are still zero)
      bool bad = false;

      // Step i at compile-time rotation position K: tiles i, i+1 and i+2 live
      // in stages K, K+1 and K+2 (mod NS); x holds tile i's shifted scores
      // (masked), y receives tile i+1's.  Control flow (mask, loads, barrier,
      // reference check) sits at the step boundaries only, so the body is one
      // straight-line block for the scheduler.  Returns false after the last
      // tile.
      int i = 0;
      Tile nx = advance(first, Ic<0>{});  // tile i+1
      auto step = [&](auto K) {
        constexpr int k = decltype(K)::value;
        auto& x = (k % 2 == 0) ? xa : xb;
        auto& y = (k % 2 == 0) ? xb : xa;
        if constexpr (k % G == 0) {
          // Tiles i+AHEAD .. i+AHEAD+G-1 refill the stages of tiles i-G ..
          // i-1, released by the barrier that closed step i-1.
          static_for<0, G>([&](auto J) {
            constexpr int jx = decltype(J)::value;
            if (__builtin_expect(i + C::AHEAD + jx < n_tiles, 1)) issue_loads(Ic<(k + C::AHEAD + jx) % NS>{}, ld);
            ld = advance(ld, Ic<1>{});
          });
          // Measurement mode: no overlap of the tile transfers with compute.
          if (p.sync_loads) asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
        }
        // ---- straight-line body ----
        qk_held(y, kf);  // scores of tile i+1 (harmless past the end)
        v_reads(Ic<k % NS>{}, va);
        exps(x, pb, ls);
#pragma unroll
        for (int nb = 0; nb < NB; ++nb) l_part[nb] += ls[nb];
        if constexpr (kPinP) {
          // P is complete beside the score products: the vector work of the
          // exponentials stays in the first half of the step.
#pragma unroll
          for (int nb = 0; nb < NB; ++nb) asm volatile("" : "+v"(pb[nb][0]), "+v"(pb[nb][1]));
          __builtin_amdgcn_sched_barrier(0);
        }
        asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");  // the V reads of tile i
#pragma unroll
        for (int db = 0; db < D / 32; ++db) asm volatile("" : "+v"(va[db][0]), "+v"(va[db][1]));
        k_reads(Ic<(k + 2) % NS>{}, kf);  // tile i+2 (harmless past the end)
        pv_held(va, pb);
        shift(y);
        if constexpr (kPinP) {
#pragma unroll
          for (int nb = 0; nb < NB; ++nb) asm volatile("" : "+v"(y[nb]));
        }
        // ---- step boundary ----
        if constexpr (k % G == G - 1) {
          // The tiles the next group reads must have landed; the last LATE
          // tiles loaded at the start of this group may stay in flight.
          // A bare s_barrier: a fenced one would wait for every load in
          // flight.  Every LDS read of a stage the next group refills was
          // awaited inside its step.
          // (vmcnt counts in issue order: the allowance holds only when this
          // group issued all G tiles' loads; near the end it issued fewer.)
          if (C::LATE > 0 && i + C::AHEAD < n_tiles) {
            asm volatile("s_waitcnt vmcnt(%0)" ::"n"(C::LATE * 2 * C::LOADS) : "memory");
          } else {
            asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
          }
          __builtin_amdgcn_s_barrier();
          // Reference check (wave-uniform branch, rarely taken).
          bool high = false;
#pragma unroll
          for (int nb = 0; nb < NB; ++nb) high |= l_part[nb] > kRaiseAt;
          if (__builtin_expect(__builtin_amdgcn_ballot_w64(high) != 0, 0)) raise_ref(bad, y);
        }
        if (__builtin_expect(++i >= n_tiles, 0)) return false;
        if (__builtin_expect(nx.kt >= nx.full, 0)) mask(y, nx);  // tile i (the next step's x)
        nx = advance(nx, Ic<0>{});
        return true;
      };
      // Stages rotate with period NS, the score buffers with period 2 and
      // the load groups with period G.
      constexpr int kUnroll = lcm3(NS, 2, G);
      while (i < n_tiles) {
        if (!unrolled_steps<0, kUnroll>(step)) break;
      }
      // The last K reads issued ahead are never consumed: wait for them while
      // their registers are still reserved.
      static_for<0, D / 16>([&kf](auto I) { asm volatile("s_waitcnt lgkmcnt(0)" : "+v"(kf[I])); });
      // A final barrier: the sequence may end between the group barriers.
      asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
      __syncthreads();

      // A row whose sum or output is not finite took an exponential past the
      // fp32 range: recompute the query tile by the exact path.
      float z = 0.f;
#pragma unroll
      for (int nb = 0; nb < NB; ++nb) {
        z = __builtin_fmaf(l_part[nb], 0.f, z);
#pragma unroll
        for (int db = 0; db < D / 32; ++db)
#pragma unroll
          for (int e2 = 0; e2 < 16; ++e2) z = __builtin_fmaf(oacc[db][nb][e2], 0.f, z);
      }
      bad |= !(z == 0.f);  // inf * 0 and NaN * 0 are NaN
      // Each wave's vote in a slot of the last K stage: its loads have all
      // landed (the barrier above), and the next query tile's first loads
      // fill the first AHEAD stages only, so every wave has read the votes
      // before anything is written there again.  (Inline assembly like every
      // other access to the ring, each access awaited in its own block.)
      const uint32_t votes = lds0 + (NS - 1) * C::TILEB;
      const uint32_t my_vote = __builtin_amdgcn_ballot_w64(bad) != 0 ? 1u : 0u;
      if (lane == 0)
        asm volatile("ds_write_b32 %0, %1\n\ts_waitcnt lgkmcnt(0)" ::"v"(votes + 4 * wave), "v"(my_vote) : "memory");
      __syncthreads();
      uint32_t redo = 0;
#pragma unroll
      for (int w = 0; w < NW; ++w) {
        uint32_t vw;
        asm volatile("ds_read_b32 %0, %1\n\ts_waitcnt lgkmcnt(0)" : "=v"(vw) : "v"(votes + 4 * w) : "memory");
        redo |= vw;
      }
      if (redo) exact_pass();
    } else if (n_tiles > 0) {
      exact_pass();
    }

    // Epilogue: out = O / l, lse = ln 2 * (m_ref + log2 l).
#pragma unroll
    for (int nb = 0; nb < NB; ++nb) {
      const float lt = halves_sum(l_part[nb]);
      const float inv = lt > 0.f ? 1.f / lt : 0.f;
      const int row = i0 + (wave * NB + nb) * 32 + lc;
      if (row < n_loc) {
        const int64_t ro = q_off + (p.qo_natural ? posq[nb] : row);
        OutT* op = out_base + ro * D;
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
        if (g == 0) lse_base[ro] = lt > 0.f ? (m_ref[nb] + __log2f(lt)) * kLn2 : -INFINITY;
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
      const int pos_first = token_pos32(rank, i0, n_loc, p.c, p.split);
      const int pos_last = token_pos32(rank, last_row, n_loc, p.c, p.split);
      for (int t = t0; t < t1; ++t) {
        const int j = owner_of(t);
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
    if (p.event_counts) {
      unsigned long long r = n_raise;
#pragma unroll
      for (int off = 32; off > 0; off >>= 1) r += __shfl_xor(r, off);
      if (lane == 0 && r) atomicAdd(p.stats + 4, r);
      if (tid == 0 && n_exact) atomicAdd(p.stats + 5, (unsigned long long)n_exact);
    }
    if (tid == 0) {
      atomicAdd(p.stats + 0, pairs_full);
      atomicAdd(p.stats + 1, t_full);
      atomicAdd(p.stats + 2, t_part);
      atomicAdd(p.stats + 3, t_skip);
    }
  }
}

// Per head_dim tile configuration (waves, 32-row blocks per wave).
template <int D>
struct TileCfg {
  static constexpr int NW = RA_FWD_NW, NB = 1;
};
template <>
struct TileCfg<64> {  // the d = 64 tiles are too small to split over more than 4 waves
  static constexpr int NW = 4, NB = 2;
};

template <int D, typename OutT>
hipError_t launch_one(FwdParams p, hipStream_t stream) {
  using T = TileCfg<D>;
  using C = Cfg<D, T::NW, T::NB>;
  p.n_qtiles = (int32_t)((p.n_loc + C::BQ - 1) / C::BQ);
  p.n_ktiles = (int32_t)((p.n_loc + C::BK - 1) / C::BK);
  p.n_pairs = (p.n_qtiles + 1) / 2;
  const int64_t per_split = (int64_t)p.batch * p.h_q * p.n_pairs;
  const int64_t grid = per_split * p.n_splits;
  if (grid > 0x7fffffff) return hipErrorInvalidConfiguration;
  p.grid_per_split = (int32_t)per_split;
  const int64_t per_rank = per_split * p.n_splits;
  if (p.all_ranks) {
    if (per_rank * p.c > 0x7fffffff) return hipErrorInvalidConfiguration;
    p.grid_per_rank = (int32_t)per_rank;
  }
  const int64_t grid_all = p.all_ranks ? per_rank * p.c : grid;
  hipLaunchKernelGGL((fwd_bf16_kernel<D, T::NW, T::NB, OutT>), dim3((unsigned)grid_all), dim3(C::NT), 0,
                     stream, p);
  return hipGetLastError();
}

}  // namespace

void tile_shape_bf16(int32_t head_dim, int32_t* tq, int32_t* tk) {
  if (head_dim == 64) {
    *tq = TileCfg<64>::NW * TileCfg<64>::NB * 32;
  } else {
    *tq = TileCfg<128>::NW * TileCfg<128>::NB * 32;
  }
  *tk = 32;
}

hipError_t launch_fwd_bf16(const FwdParams& p, int32_t head_dim, int32_t out_dtype,
                           hipStream_t stream) {
  if (head_dim == 128)
    return out_dtype == RA_F32 ? launch_one<128, float>(p, stream) : launch_one<128, __bf16>(p, stream);
  return out_dtype == RA_F32 ? launch_one<64, float>(p, stream) : launch_one<64, __bf16>(p, stream);
}

}  // namespace ra
