// fp32 shard forward: plain VALU kernel, one query row per four lanes.
//
// The online-softmax fold over ring-ordered key/value blocks ("Sequence /
// context parallelism" notes, section 4): per key tile, raise the running
// max m, rescale the running normaliser l and output accumulator by
// exp(m_old - m_new), add the tile's exp(s - m_new) terms, and divide by l at
// the end.  Everything stays in fp32 (no reduced-precision products), which
// is what a 1e-5 absolute bound against fp64 needs.
//
// Workgroup = KS wavefronts on the same 16 query rows of one (batch, head).
// In each wavefront a row is spread over 4 lanes (lanes l, l+16, l+32, l+48),
// each holding d/4 of its dimensions, and a score is the sum of the 4 partial
// dot products (two lane exchanges), so every lane of a row holds the whole
// score.  The visible key tiles of the ring-ordered blocks are dealt to the
// wavefronts in turn (tile g to wavefront g mod KS); each folds its tiles into
// its own (m, l, O) state, staging them in its own LDS buffer with the next
// one of its tiles loaded into registers meanwhile, and the KS states are
// merged through LDS at the end (the same fold, applied to partial states).
// Small shards so keep KS times more wavefronts in flight.  Tiles whose keys
// all follow the workgroup's last query are skipped without being read.
#include "ra_common.h"
#include "tile_common.h"

namespace ra {
namespace {

// Sum over lanes l and l ^ 16 (the 16-lane rows of each half-wave swapped):
// as with halves_sum, both lanes of a pair get the same value bit for bit.
__device__ inline float rows16_sum(float x) {
  auto r = __builtin_amdgcn_permlane16_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return __uint_as_float(r[0]) + __uint_as_float(r[1]);
}

constexpr int TK = 32;
constexpr int kLanesPerRow = 4;
constexpr int TQ = 64 / kLanesPerRow;  // query rows per wavefront
static_assert(kLanesPerRow == 4, "the score reduction pairs lanes l ^ 16 and l ^ 32");

// Wavefronts per workgroup (key-tile split): 4 x 32 KiB or 8 x 16 KiB of LDS tiles.
template <int D>
struct F32Cfg {
  static constexpr int KS = D == 64 ? 8 : 4;
};

template <int D, int KS>
__global__ __launch_bounds__(64 * KS) void fwd_f32_kernel(FwdParams p) {
  constexpr int DL = D / kLanesPerRow;  // dimensions held per lane
  constexpr int NL = TK * D / 4 / 64;  // 16-byte loads per lane per tile and tensor
  // One K and one V tile per wavefront (its own tiles only).
  __shared__ float ks[KS][TK][D];
  __shared__ float vs[KS][TK][D];
  static_assert(KS * TK * D >= KS * 64 * (2 + DL), "the merge reuses the K tiles");

  const int lane = threadIdx.x & 63;
  const int wv = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int w = blockIdx.x;
  const int qt = w % p.n_qtiles;
  const int h = (w / p.n_qtiles) % p.h_q;
  const int b = w / (p.n_qtiles * p.h_q);
  const int hk = h / p.group;
  const int64_t n_loc = p.n_loc;
  const int64_t kv_off = ((int64_t)b * p.h_kv + hk) * n_loc * D;

  const int part = lane / TQ;  // which quarter of the row's dimensions this lane holds
  const int d0 = part * DL;
  const int64_t i0 = (int64_t)qt * TQ;
  const int64_t row = i0 + lane % TQ;
  const bool row_ok = row < n_loc;
  const int64_t last_row = (i0 + TQ <= n_loc ? i0 + TQ : n_loc) - 1;
  const bool rows_full = i0 + TQ <= n_loc;
  const int64_t pos_q = row_ok ? token_pos(p.rank, row, n_loc, p.c, p.split) : -1;
  const int64_t pos_first = token_pos(p.rank, i0, n_loc, p.c, p.split);
  const int64_t pos_last = token_pos(p.rank, last_row, n_loc, p.c, p.split);

  const int64_t qrow = row_ok ? (p.qo_natural ? pos_q : row) : 0;  // q / out / lse row of this query
  const float* qp = (const float*)p.q + (((int64_t)b * p.h_q + h) * p.qo_rows + qrow) * D;
  float qv[DL], o[DL];
#pragma unroll
  for (int e = 0; e < DL; ++e) {
    qv[e] = row_ok ? qp[d0 + e] : 0.f;
    o[e] = 0.f;
  }
  float m = -INFINITY, l = 0.f;
  unsigned long long pairs = 0;

  // Cursor over the visible tiles of the block list: block t, tile kt, and
  // the block's visible / unmasked tile counts.  t == n_blocks: past the end.
  struct Cur {
    int t, kt, vis, full;
  };
  auto counts = [&](Cur& x) {
    const int j = p.owner[x.t];
    const int64_t c_last = p.causal ? count_upto(j, pos_last, n_loc, p.c, p.split) : n_loc;
    const int64_t c_first = p.causal ? count_upto(j, pos_first, n_loc, p.c, p.split) : n_loc;
    x.vis = (int)((c_last + TK - 1) / TK);
    x.full = rows_full ? (int)(c_first / TK) : 0;
  };
  auto advance = [&](Cur x, int n) {  // n visible tiles further on
    x.kt += n;
    while (x.t < p.n_blocks && x.kt >= x.vis) {
      x.kt -= x.vis;
      if (++x.t < p.n_blocks) counts(x);
    }
    return x;
  };

  // Tile x's K and V rows in registers; rows past the shard end read row 0
  // (always present) and are stored as zeros.
  float4 kx[NL], vx[NL];
  auto load = [&](const Cur& x) {
    const float* kp = (const float*)p.k[x.t] + kv_off;
    const float* vp = (const float*)p.v[x.t] + kv_off;
#pragma unroll
    for (int i = 0; i < NL; ++i) {
      const int idx = lane + 64 * i;
      const int kk = idx / (D / 4), e = (idx % (D / 4)) * 4;
      const int64_t key = (int64_t)x.kt * TK + kk;
      const int64_t kr = key < n_loc ? key : 0;
      kx[i] = *(const float4*)(kp + kr * D + e);
      vx[i] = *(const float4*)(vp + kr * D + e);
    }
  };
  // (A wavefront's LDS operations execute in order, so its own buffer needs no
  // barrier between the reads of one tile and the stores of the next.)
  auto store = [&](const Cur& x) {
#pragma unroll
    for (int i = 0; i < NL; ++i) {
      const int idx = lane + 64 * i;
      const int kk = idx / (D / 4), e = (idx % (D / 4)) * 4;
      const bool ok = (int64_t)x.kt * TK + kk < n_loc;
      *(float4*)&ks[wv][kk][e] =
          float4{ok ? kx[i].x : 0.f, ok ? kx[i].y : 0.f, ok ? kx[i].z : 0.f, ok ? kx[i].w : 0.f};
      *(float4*)&vs[wv][kk][e] =
          float4{ok ? vx[i].x : 0.f, ok ? vx[i].y : 0.f, ok ? vx[i].z : 0.f, ok ? vx[i].w : 0.f};
    }
  };

  Cur cur;
  cur.t = 0;
  cur.kt = 0;
  counts(cur);  // n_blocks >= 1
  cur = advance(cur, wv);  // this wavefront's first tile
  if (cur.t < p.n_blocks) load(cur);
  while (cur.t < p.n_blocks) {
    const Cur x = cur;
    store(x);
    cur = advance(cur, KS);
    if (cur.t < p.n_blocks) load(cur);  // in flight while tile x is computed

    const int j = p.owner[x.t];
    const int64_t key0 = (int64_t)x.kt * TK;
    const bool masked = x.kt >= x.full;
    float s[TK];
    float mt = -INFINITY;
#pragma unroll 4
    for (int kk = 0; kk < TK; ++kk) {
      float dot = 0.f;
#pragma unroll
      for (int e = 0; e < DL; ++e) dot = fmaf(qv[e], ks[wv][kk][d0 + e], dot);
      // Every lane of the row ends with the full score, bit for bit.
      dot = halves_sum(rows16_sum(dot));
      bool vis = true;
      if (masked) {
        const int64_t jj = key0 + kk;
        vis = row_ok && jj < n_loc && (!p.causal || token_pos(j, jj, n_loc, p.c, p.split) <= pos_q);
        pairs += (vis && part == 0) ? 1 : 0;
      }
      s[kk] = vis ? dot * p.scale : -INFINITY;
      mt = fmaxf(mt, s[kk]);
    }
    if (!masked && part == 0) pairs += TK;
    const float m_new = fmaxf(m, mt);
    if (m_new == -INFINITY) continue;  // nothing visible to this row yet
    const float alpha = expf(m - m_new);  // m = -inf gives 0
    l *= alpha;
#pragma unroll
    for (int e = 0; e < DL; ++e) o[e] *= alpha;
#pragma unroll 4
    for (int kk = 0; kk < TK; ++kk) {
      const float pk = expf(s[kk] - m_new);
      l += pk;
#pragma unroll
      for (int e = 0; e < DL; ++e) o[e] = fmaf(pk, vs[wv][kk][d0 + e], o[e]);
    }
    m = m_new;
  }

  // Merge the wavefronts' states: m* = max m_w, l* = sum l_w exp(m_w - m*),
  // O* = sum O_w exp(m_w - m*).
  __syncthreads();  // every wavefront is done with its tiles
  float* red = &ks[0][0][0];
  red[(wv * (2 + DL) + 0) * 64 + lane] = m;
  red[(wv * (2 + DL) + 1) * 64 + lane] = l;
#pragma unroll
  for (int e = 0; e < DL; ++e) red[(wv * (2 + DL) + 2 + e) * 64 + lane] = o[e];
  __syncthreads();
  if (wv == 0 && row_ok) {
    float mm = m;
#pragma unroll
    for (int u = 1; u < KS; ++u) mm = fmaxf(mm, red[(u * (2 + DL)) * 64 + lane]);
    float ll = 0.f;
    float oo[DL];
#pragma unroll
    for (int e = 0; e < DL; ++e) oo[e] = 0.f;
    if (mm != -INFINITY) {
#pragma unroll
      for (int u = 0; u < KS; ++u) {
        const float f = expf(red[(u * (2 + DL)) * 64 + lane] - mm);  // -inf state: 0
        ll = fmaf(red[(u * (2 + DL) + 1) * 64 + lane], f, ll);
#pragma unroll
        for (int e = 0; e < DL; ++e) oo[e] = fmaf(red[(u * (2 + DL) + 2 + e) * 64 + lane], f, oo[e]);
      }
    }
    const int64_t ro = ((int64_t)b * p.h_q + h) * p.qo_rows + qrow;
    float* op = (float*)p.out + ro * D;
    const float inv = ll > 0.f ? 1.f / ll : 0.f;
#pragma unroll
    for (int e = 0; e < DL; ++e) op[d0 + e] = oo[e] * inv;
    if (part == 0) p.lse[ro] = ll > 0.f ? mm + logf(ll) : -INFINITY;
  }

  if (p.stats) {
#pragma unroll
    for (int off = 32; off > 0; off >>= 1) pairs += __shfl_xor(pairs, off);
    if (lane == 0 && pairs) atomicAdd(p.stats + 0, pairs);
    if (threadIdx.x == 0) {
      // Tile classes per block, counted once per workgroup.
      unsigned long long t_full = 0, t_part = 0, t_skip = 0;
      for (int t = 0; t < p.n_blocks; ++t) {
        Cur x;
        x.t = t;
        counts(x);
        t_full += x.full;
        t_part += x.vis - x.full;
        t_skip += p.n_ktiles - x.vis;
      }
      atomicAdd(p.stats + 1, t_full);
      atomicAdd(p.stats + 2, t_part);
      atomicAdd(p.stats + 3, t_skip);
    }
  }
}

}  // namespace

void tile_shape_f32(int32_t /*head_dim*/, int32_t* tq, int32_t* tk) {
  *tq = TQ;
  *tk = TK;
}

hipError_t launch_fwd_f32(const FwdParams& p0, int32_t head_dim, hipStream_t stream) {
  FwdParams p = p0;
  p.n_qtiles = (int32_t)((p.n_loc + TQ - 1) / TQ);
  p.n_ktiles = (int32_t)((p.n_loc + TK - 1) / TK);
  p.n_pairs = p.n_qtiles;
  const int64_t grid = (int64_t)p.batch * p.h_q * p.n_qtiles;
  if (grid > 0x7fffffff) return hipErrorInvalidConfiguration;
  if (head_dim == 64)
    hipLaunchKernelGGL((fwd_f32_kernel<64, F32Cfg<64>::KS>), dim3((unsigned)grid), dim3(64 * F32Cfg<64>::KS), 0,
                       stream, p);
  else
    hipLaunchKernelGGL((fwd_f32_kernel<128, F32Cfg<128>::KS>), dim3((unsigned)grid), dim3(64 * F32Cfg<128>::KS), 0,
                       stream, p);
  return hipGetLastError();
}

}  // namespace ra
