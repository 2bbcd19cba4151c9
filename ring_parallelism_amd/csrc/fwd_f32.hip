// fp32 shard forward: plain VALU kernel, one query row per four lanes.
//
// The online-softmax fold over ring-ordered key/value blocks ("Sequence /
// context parallelism" notes, section 4): per key tile, raise the running
// max m, rescale the running normaliser l and output accumulator by
// exp(m_old - m_new), add the tile's exp(s - m_new) terms, and divide by l at
// the end.  Everything stays in fp32 (no reduced-precision products), which
// is what a 1e-5 absolute bound against fp64 needs.
//
// Workgroup = one wavefront = 16 query rows of one (batch, head); each row
// is spread over 4 lanes (lanes l, l+16, l+32, l+48), each holding d/4 of its
// dimensions, and a score is the sum of the 4 partial dot products (two lane
// exchanges), so every lane of a row holds the whole score.  Small rows per
// wave keep many workgroups in flight on small shards.  Key/value tiles of TK
// rows are staged in LDS (two buffers: the next tile's loads are in flight
// while a tile is computed) and read as broadcasts.  Tiles whose keys all
// follow the workgroup's last query are skipped without being read.
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

template <int D>
__global__ __launch_bounds__(64) void fwd_f32_kernel(FwdParams p) {
  constexpr int DL = D / kLanesPerRow;  // dimensions held per lane
  constexpr int NL = TK * D / 4 / 64;  // 16-byte loads per lane per tile and tensor
  // Two LDS buffers: tile kt+1 is loaded into registers while tile kt is
  // computed, then stored into the other buffer.
  __shared__ float ks[2][TK][D];
  __shared__ float vs[2][TK][D];

  const int lane = threadIdx.x;
  const int w = blockIdx.x;
  const int qt = w % p.n_qtiles;
  const int h = (w / p.n_qtiles) % p.h_q;
  const int b = w / (p.n_qtiles * p.h_q);
  const int hk = h / p.group;
  const int64_t n_loc = p.n_loc;

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
  unsigned long long pairs = 0, t_full = 0, t_part = 0, t_skip = 0;

  for (int t = 0; t < p.n_blocks; ++t) {
    const int j = p.owner[t];
    const int64_t kv_off = ((int64_t)b * p.h_kv + hk) * n_loc * D;
    const float* kp = (const float*)p.k[t] + kv_off;
    const float* vp = (const float*)p.v[t] + kv_off;
    const int64_t c_last = p.causal ? count_upto(j, pos_last, n_loc, p.c, p.split) : n_loc;
    const int64_t c_first = p.causal ? count_upto(j, pos_first, n_loc, p.c, p.split) : n_loc;
    const int n_vis = (int)((c_last + TK - 1) / TK);
    const int n_full = rows_full ? (int)(c_first / TK) : 0;
    t_full += n_full;
    t_part += n_vis - n_full;
    t_skip += p.n_ktiles - n_vis;

    // Tile kt's K and V rows in registers; rows past the shard end read row 0
    // (always present) and are stored as zeros.
    float4 kx[NL], vx[NL];
    auto load = [&](int kt) {
#pragma unroll
      for (int i = 0; i < NL; ++i) {
        const int idx = lane + 64 * i;
        const int kk = idx / (D / 4), e = (idx % (D / 4)) * 4;
        const int64_t key = (int64_t)kt * TK + kk;
        const int64_t kr = key < n_loc ? key : 0;
        kx[i] = *(const float4*)(kp + kr * D + e);
        vx[i] = *(const float4*)(vp + kr * D + e);
      }
    };
    auto store = [&](int kt, int buf) {
#pragma unroll
      for (int i = 0; i < NL; ++i) {
        const int idx = lane + 64 * i;
        const int kk = idx / (D / 4), e = (idx % (D / 4)) * 4;
        const bool ok = (int64_t)kt * TK + kk < n_loc;
        *(float4*)&ks[buf][kk][e] =
            float4{ok ? kx[i].x : 0.f, ok ? kx[i].y : 0.f, ok ? kx[i].z : 0.f, ok ? kx[i].w : 0.f};
        *(float4*)&vs[buf][kk][e] =
            float4{ok ? vx[i].x : 0.f, ok ? vx[i].y : 0.f, ok ? vx[i].z : 0.f, ok ? vx[i].w : 0.f};
      }
    };
    if (n_vis > 0) load(0);

    for (int kt = 0; kt < n_vis; ++kt) {
      const int64_t key0 = (int64_t)kt * TK;
      const int buf = kt & 1;
      // Buffer `buf` was last read by tile kt-2 (or by the previous block's
      // tiles), whose reads ended before an earlier barrier: the one after
      // tile kt-1 was stored, or for tile 0 the one here.
      if (kt == 0) __syncthreads();
      store(kt, buf);
      __syncthreads();  // tile kt visible to every lane
      if (kt + 1 < n_vis) load(kt + 1);  // in flight while tile kt is computed

      const bool masked = kt >= n_full;
      float s[TK];
      float mt = -INFINITY;
#pragma unroll 4
      for (int kk = 0; kk < TK; ++kk) {
        float dot = 0.f;
#pragma unroll
        for (int e = 0; e < DL; ++e) dot = fmaf(qv[e], ks[buf][kk][d0 + e], dot);
        // Every lane of the row ends with the full score, bit for bit.
        dot = halves_sum(rows16_sum(dot));
        bool vis = true;
        if (masked) {
          const int64_t jj = key0 + kk;
          vis = row_ok && jj < n_loc &&
                (!p.causal || token_pos(j, jj, n_loc, p.c, p.split) <= pos_q);
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
        for (int e = 0; e < DL; ++e) o[e] = fmaf(pk, vs[buf][kk][d0 + e], o[e]);
      }
      m = m_new;
    }
  }

  if (row_ok) {
    const int64_t ro = ((int64_t)b * p.h_q + h) * p.qo_rows + qrow;
    float* op = (float*)p.out + ro * D;
    const float inv = l > 0.f ? 1.f / l : 0.f;
#pragma unroll
    for (int e = 0; e < DL; ++e) op[d0 + e] = o[e] * inv;
    if (part == 0) p.lse[ro] = l > 0.f ? m + logf(l) : -INFINITY;
  }

  if (p.stats) {
#pragma unroll
    for (int off = 32; off > 0; off >>= 1) pairs += __shfl_xor(pairs, off);
    if (lane == 0) {
      atomicAdd(p.stats + 0, pairs);
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
    hipLaunchKernelGGL(fwd_f32_kernel<64>, dim3((unsigned)grid), dim3(64), 0, stream, p);
  else
    hipLaunchKernelGGL(fwd_f32_kernel<128>, dim3((unsigned)grid), dim3(64), 0, stream, p);
  return hipGetLastError();
}

}  // namespace ra
