// C ABI of the ring-attention shard library: argument validation, ring-order
// resolution and kernel dispatch.  Every check runs before any launch, so a
// rejected call leaves the stream untouched.
#include <cmath>
#include <cstdarg>
#include <cstdio>
#include <cstring>

#include "ra_common.h"

namespace {

thread_local char g_err[512] = "";

ra_status fail(ra_status code, const char* fmt, ...) {
  va_list ap;
  va_start(ap, fmt);
  vsnprintf(g_err, sizeof g_err, fmt, ap);
  va_end(ap);
  return code;
}

ra_status ok() {
  g_err[0] = '\0';
  return RA_OK;
}

}  // namespace

namespace ra {
ra_status set_error(ra_status code, const char* fmt, ...) {
  va_list ap;
  va_start(ap, fmt);
  vsnprintf(g_err, sizeof g_err, fmt, ap);
  va_end(ap);
  return code;
}
}  // namespace ra

namespace {

bool aligned(const void* p, uintptr_t a) { return ((uintptr_t)p % a) == 0; }

ra_status check_split(int64_t S, int32_t c, int32_t split) {
  if (S < 1) return fail(RA_EINVAL, "seq_len must be >= 1 (got %lld)", (long long)S);
  if (S > ((int64_t)1 << 40)) return fail(RA_EINVAL, "seq_len too large (%lld)", (long long)S);
  if (c < 1) return fail(RA_EINVAL, "n_shards must be >= 1 (got %d)", c);
  if (split != RA_SPLIT_CONTIGUOUS && split != RA_SPLIT_ZIGZAG && split != RA_SPLIT_STRIPED)
    return fail(RA_EINVAL, "unknown split %d", split);
  if (split == RA_SPLIT_ZIGZAG && S % (2 * (int64_t)c) != 0)
    return fail(RA_EINVAL, "zig-zag split needs seq_len %% (2*n_shards) == 0 (S=%lld, c=%d)",
                (long long)S, c);
  if (S % c != 0)
    return fail(RA_EINVAL, "seq_len %% n_shards != 0 (S=%lld, c=%d)", (long long)S, c);
  return RA_OK;
}

// a * b, or INT64_MAX where that overflows (size checks must not wrap).
int64_t mul_sat(int64_t a, int64_t b) {
  int64_t r;
  return __builtin_mul_overflow(a, b, &r) ? INT64_MAX : r;
}

ra_status check_desc(const ra_attn_desc* d) {
  if (!d) return fail(RA_EINVAL, "desc is NULL");
  ra_status st = check_split(d->seq_len, d->n_shards, d->split);
  if (st != RA_OK) return st;
  if (d->batch < 1) return fail(RA_EINVAL, "batch must be >= 1 (got %d)", d->batch);
  if (d->h_q < 1 || d->h_kv < 1) return fail(RA_EINVAL, "h_q and h_kv must be >= 1");
  if (d->h_q % d->h_kv != 0)
    return fail(RA_EINVAL, "h_q %% h_kv != 0 (h_q=%d, h_kv=%d)", d->h_q, d->h_kv);
  if (d->in_dtype != RA_F32 && d->in_dtype != RA_BF16)
    return fail(RA_EINVAL, "unknown in_dtype %d", d->in_dtype);
  if (d->out_dtype != RA_F32 && d->out_dtype != RA_BF16)
    return fail(RA_EINVAL, "unknown out_dtype %d", d->out_dtype);
  if (d->causal != 0 && d->causal != 1) return fail(RA_EINVAL, "causal must be 0 or 1");
  if (!std::isfinite(d->scale) || !(d->scale > 0.f))
    return fail(RA_EINVAL, "scale must be finite and > 0");
  if (d->head_dim != 64 && d->head_dim != 128)
    return fail(RA_EUNSUPPORTED, "head_dim %d not supported (64 or 128)", d->head_dim);
  if (d->in_dtype == RA_F32 && d->out_dtype == RA_BF16)
    return fail(RA_EUNSUPPORTED, "fp32 inputs with bf16 output are not supported");
  if ((d->flags & ~(RA_FLAG_SYNC_LOADS | RA_FLAG_NATURAL_QO | RA_FLAG_EVENT_COUNTS)) != 0)
    return fail(RA_EINVAL, "unknown flags 0x%x", d->flags);
  if ((d->flags & RA_FLAG_SYNC_LOADS) && d->in_dtype != RA_BF16)
    return fail(RA_EUNSUPPORTED, "RA_FLAG_SYNC_LOADS applies to bf16 inputs only");
  if (d->seq_len >= ((int64_t)1 << 31) - 1)
    return fail(RA_EUNSUPPORTED, "seq_len must be < 2^31 - 1 for attention");
  const int64_t n_loc = d->seq_len / d->n_shards;
  if (n_loc * d->head_dim >= ((int64_t)1 << 31))
    return fail(RA_EUNSUPPORTED, "seq_len/n_shards * head_dim must be < 2^31");
  if (mul_sat(mul_sat(d->batch, d->h_q), n_loc) >= ((int64_t)1 << 40))
    return fail(RA_EUNSUPPORTED, "batch * h_q * seq_len/n_shards too large");
  return RA_OK;
}

}  // namespace

extern "C" {

int32_t ring_attn_abi_version(void) { return RA_ABI_VERSION; }

const char* ring_attn_last_error(void) { return g_err; }

static ra_status partition_common(int64_t S, int32_t c, int32_t split, int64_t* perm,
                                  const void* src, void* dst, int64_t outer, int64_t inner_bytes,
                                  void* stream, bool inverse) {
  ra_status st = check_split(S, c, split);
  if (st != RA_OK) return st;
  if ((src == nullptr) != (dst == nullptr)) return fail(RA_EINVAL, "src and dst must both be set or both NULL");
  if (!perm && !src) return fail(RA_EINVAL, "nothing to do: perm, src and dst are NULL");
  if (perm && !aligned(perm, 8)) return fail(RA_EINVAL, "perm must be 8-byte aligned");
  if (src) {
    if (outer < 1 || inner_bytes < 1)
      return fail(RA_EINVAL, "outer and inner_bytes must be >= 1 (got %lld, %lld)",
                  (long long)outer, (long long)inner_bytes);
    const int64_t total = outer * S;
    if (total / S != outer || total > ((int64_t)1 << 46) / inner_bytes)
      return fail(RA_EINVAL, "outer * seq_len * inner_bytes too large");
    const char* s0 = (const char*)src;
    const char* d0 = (const char*)dst;
    const int64_t bytes = total * inner_bytes;
    if (s0 < d0 + bytes && d0 < s0 + bytes) return fail(RA_EINVAL, "src and dst overlap");
  }
  hipError_t e = ra::launch_partition(S, c, split, perm, src, dst, outer, inner_bytes, inverse,
                                      (hipStream_t)stream);
  if (e != hipSuccess) return fail(RA_EHIP, "partition launch failed: %s", hipGetErrorString(e));
  return ok();
}

ra_status zigzag_partition(int64_t seq_len, int32_t n_shards, int32_t split, int64_t* perm,
                           const void* src, void* dst, int64_t outer, int64_t inner_bytes,
                           void* stream) {
  return partition_common(seq_len, n_shards, split, perm, src, dst, outer, inner_bytes, stream,
                          false);
}

ra_status zigzag_unpartition(int64_t seq_len, int32_t n_shards, int32_t split, const void* src,
                             void* dst, int64_t outer, int64_t inner_bytes, void* stream) {
  if (!src || !dst) return fail(RA_EINVAL, "src and dst must be set");
  return partition_common(seq_len, n_shards, split, nullptr, src, dst, outer, inner_bytes, stream,
                          true);
}

ra_status ring_attn_tile_shape(const ra_attn_desc* desc, int32_t* tile_q, int32_t* tile_k) {
  ra_status st = check_desc(desc);
  if (st != RA_OK) return st;
  if (!tile_q || !tile_k) return fail(RA_EINVAL, "tile_q and tile_k must be set");
  if (desc->in_dtype == RA_F32)
    ra::tile_shape_f32(desc->head_dim, tile_q, tile_k);
  else
    ra::tile_shape_bf16(desc->head_dim, tile_q, tile_k);
  return ok();
}

// Validates the arguments shared by the two shard entry points and fills p.
static ra_status shard_params(const ra_attn_desc* desc, int32_t rank, const void* q, int32_t n_blocks,
                              const int32_t* block_owner, const void* const* k_blocks,
                              const void* const* v_blocks, void* out, float* lse, int64_t* stats,
                              ra::FwdParams& p) {
  ra_status st = check_desc(desc);
  if (st != RA_OK) return st;
  const int32_t c = desc->n_shards;
  if (rank < 0 || rank >= c) return fail(RA_EINVAL, "rank %d not in [0, %d)", rank, c);
  if (n_blocks < 1 || n_blocks > c)
    return fail(RA_EINVAL, "n_blocks %d not in [1, n_shards=%d]", n_blocks, c);
  if (n_blocks > RA_MAX_BLOCKS)
    return fail(RA_EUNSUPPORTED, "n_blocks %d exceeds RA_MAX_BLOCKS (%d)", n_blocks, RA_MAX_BLOCKS);
  if (!q || !out || !lse) return fail(RA_EINVAL, "q, out and lse must be set");
  if (!aligned(q, 16) || !aligned(out, 16)) return fail(RA_EINVAL, "q and out must be 16-byte aligned");
  if (!aligned(lse, 4)) return fail(RA_EINVAL, "lse must be 4-byte aligned");
  if (stats && !aligned(stats, 8)) return fail(RA_EINVAL, "stats must be 8-byte aligned");
  if (!k_blocks || !v_blocks) return fail(RA_EINVAL, "k_blocks and v_blocks must be set");

  std::memset(&p, 0, sizeof p);
  for (int t = 0; t < n_blocks; ++t) {
    const int32_t j = block_owner ? block_owner[t] : (int32_t)(((int64_t)rank - t % c + c) % c);
    if (j < 0 || j >= c) return fail(RA_EINVAL, "block_owner[%d] = %d not in [0, %d)", t, j, c);
    for (int u = 0; u < t; ++u)
      if (p.owner[u] == j) return fail(RA_EINVAL, "block_owner[%d] = %d repeats an earlier block", t, j);
    if (!k_blocks[t] || !v_blocks[t]) return fail(RA_EINVAL, "k_blocks[%d] / v_blocks[%d] is NULL", t, t);
    if (!aligned(k_blocks[t], 16) || !aligned(v_blocks[t], 16))
      return fail(RA_EINVAL, "k_blocks[%d] / v_blocks[%d] must be 16-byte aligned", t, t);
    p.owner[t] = j;
    p.k[t] = k_blocks[t];
    p.v[t] = v_blocks[t];
  }

  p.q = q;
  p.out = out;
  p.lse = lse;
  p.stats = (unsigned long long*)stats;
  p.n_loc = desc->seq_len / c;
  p.c = c;
  p.split = desc->split;
  p.rank = rank;
  p.n_blocks = n_blocks;
  p.batch = desc->batch;
  p.h_q = desc->h_q;
  p.h_kv = desc->h_kv;
  p.group = desc->h_q / desc->h_kv;
  p.causal = desc->causal;
  p.scale = desc->scale;
  p.scale_log2 = (float)((double)desc->scale * 1.4426950408889634);
  p.sync_loads = (desc->flags & RA_FLAG_SYNC_LOADS) ? 1 : 0;
  p.qo_natural = (desc->flags & RA_FLAG_NATURAL_QO) ? 1 : 0;
  p.event_counts = (desc->flags & RA_FLAG_EVENT_COUNTS) ? 1 : 0;
  p.qo_rows = p.qo_natural ? desc->seq_len : p.n_loc;
  p.n_splits = 1;
  return RA_OK;
}

ra_status ring_attn_shard_fwd(const ra_attn_desc* desc, int32_t rank, const void* q,
                              int32_t n_blocks, const int32_t* block_owner,
                              const void* const* k_blocks, const void* const* v_blocks, void* out,
                              float* lse, int64_t* stats, void* stream) {
  ra::FwdParams p;
  ra_status st = shard_params(desc, rank, q, n_blocks, block_owner, k_blocks, v_blocks, out, lse, stats, p);
  if (st != RA_OK) return st;
  hipError_t e = desc->in_dtype == RA_F32
                     ? ra::launch_fwd_f32(p, desc->head_dim, (hipStream_t)stream)
                     : ra::launch_fwd_bf16(p, desc->head_dim, desc->out_dtype, (hipStream_t)stream);
  if (e != hipSuccess) return fail(RA_EHIP, "shard_fwd launch failed: %s", hipGetErrorString(e));
  return ok();
}

ra_status ring_attn_all_shards_fwd(const ra_attn_desc* desc, const void* q_shards, const void* const* k_blocks,
                                   const void* const* v_blocks, void* out_shards, float* lse_shards,
                                   int64_t* stats, void* stream) {
  ra_status st = check_desc(desc);
  if (st != RA_OK) return st;
  const int32_t c = desc->n_shards;
  if (c > RA_MAX_BLOCKS) return fail(RA_EUNSUPPORTED, "n_shards %d exceeds RA_MAX_BLOCKS (%d)", c, RA_MAX_BLOCKS);
  const bool natural = (desc->flags & RA_FLAG_NATURAL_QO) != 0;
  const int64_t n_loc = desc->seq_len / c;
  const int64_t rows = (int64_t)desc->batch * desc->h_q * n_loc;  // per rank
  const int64_t q_stride = natural ? 0 : rows * desc->head_dim;
  const int64_t lse_stride = natural ? 0 : rows;
  const size_t in_sz = desc->in_dtype == RA_F32 ? 4 : 2, out_sz = desc->out_dtype == RA_F32 ? 4 : 2;
  if (!k_blocks || !v_blocks) return fail(RA_EINVAL, "k_blocks and v_blocks must be set");
  int32_t ident[RA_MAX_BLOCKS];
  for (int32_t j = 0; j < c; ++j) ident[j] = j;
  if (desc->in_dtype == RA_F32) {
    // fp32 inputs: one launch per rank (the parity path).
    const void* kb[RA_MAX_BLOCKS];
    const void* vb[RA_MAX_BLOCKS];
    for (int32_t r = 0; r < c; ++r) {
      for (int32_t t = 0; t < c; ++t) {
        const int32_t j = (r - t + c) % c;
        kb[t] = k_blocks[j];
        vb[t] = v_blocks[j];
      }
      ra::FwdParams p;
      st = shard_params(desc, r, q_shards ? (const char*)q_shards + r * q_stride * in_sz : nullptr, c, nullptr,
                        kb, vb, out_shards ? (char*)out_shards + r * q_stride * out_sz : nullptr,
                        lse_shards ? lse_shards + r * lse_stride : nullptr, stats, p);
      if (st != RA_OK) return st;
      hipError_t e = ra::launch_fwd_f32(p, desc->head_dim, (hipStream_t)stream);
      if (e != hipSuccess) return fail(RA_EHIP, "shard_fwd launch failed: %s", hipGetErrorString(e));
    }
    return ok();
  }
  ra::FwdParams p;
  st = shard_params(desc, 0, q_shards, c, ident, k_blocks, v_blocks, out_shards, lse_shards, stats, p);
  if (st != RA_OK) return st;
  p.all_ranks = 1;
  p.rank_stride_q = q_stride;
  p.rank_stride_out = q_stride;
  p.rank_stride_lse = lse_stride;
  hipError_t e = ra::launch_fwd_bf16(p, desc->head_dim, desc->out_dtype, (hipStream_t)stream);
  if (e != hipSuccess) return fail(RA_EHIP, "all-shards launch failed: %s", hipGetErrorString(e));
  return ok();
}

ra_status ring_attn_shard_fwd_split(const ra_attn_desc* desc, int32_t rank, const void* q, int32_t n_blocks,
                                    const int32_t* block_owner, const void* const* k_blocks,
                                    const void* const* v_blocks, int32_t n_splits, float* work_out,
                                    float* work_lse, void* out, float* lse, int64_t* stats, void* stream) {
  if (desc && desc->in_dtype != RA_BF16)
    return fail(RA_EUNSUPPORTED, "the split pass takes bf16 inputs");
  if (desc && (desc->flags & RA_FLAG_NATURAL_QO))
    return fail(RA_EUNSUPPORTED, "the split pass writes shard-layout results (no RA_FLAG_NATURAL_QO)");
  ra::FwdParams p;
  ra_status st = shard_params(desc, rank, q, n_blocks, block_owner, k_blocks, v_blocks, out, lse, stats, p);
  if (st != RA_OK) return st;
  if (n_splits < 1 || n_splits > n_blocks)
    return fail(RA_EINVAL, "n_splits %d not in [1, n_blocks=%d]", n_splits, n_blocks);
  if (!work_out || !work_lse) return fail(RA_EINVAL, "work_out and work_lse must be set");
  if (!aligned(work_out, 16) || !aligned(work_lse, 4))
    return fail(RA_EINVAL, "work_out must be 16-byte aligned, work_lse 4-byte");
  const int64_t rows = (int64_t)desc->batch * desc->h_q * p.n_loc;
  const int64_t part = rows * desc->head_dim;
  // The workspace must not overlap the result.
  const char* w0 = (const char*)work_out;
  const char* w1 = w0 + n_splits * part * 4;
  const char* o0 = (const char*)out;
  const char* o1 = o0 + part * (desc->out_dtype == RA_F32 ? 4 : 2);
  if (o0 < w1 && o1 > w0) return fail(RA_EINVAL, "out overlaps work_out");
  if ((const char*)lse < (const char*)(work_lse + n_splits * rows) && (const char*)(lse + rows) > (const char*)work_lse)
    return fail(RA_EINVAL, "lse overlaps work_lse");
  p.out = work_out;
  p.lse = work_lse;
  p.n_splits = n_splits;
  p.part_stride_out = part;
  p.part_stride_lse = rows;
  hipError_t e = ra::launch_fwd_bf16(p, desc->head_dim, RA_F32, (hipStream_t)stream);
  if (e != hipSuccess) return fail(RA_EHIP, "split shard pass launch failed: %s", hipGetErrorString(e));
  ra::MergeParams m;
  std::memset(&m, 0, sizeof m);
  m.strided = 1;
  m.outs_base = work_out;
  m.lses_base = work_lse;
  m.out_stride = part;
  m.lse_stride = rows;
  m.out = out;
  m.lse = lse;
  m.n_rows = rows;
  m.head_dim = desc->head_dim;
  m.n_parts = n_splits;
  e = ra::launch_merge(m, RA_F32, desc->out_dtype, (hipStream_t)stream);
  if (e != hipSuccess) return fail(RA_EHIP, "merge launch failed: %s", hipGetErrorString(e));
  return ok();
}

ra_status ring_attn_merge(int32_t batch, int32_t heads, int64_t rows, int32_t head_dim,
                          int32_t n_parts, const void* const* outs, int32_t parts_dtype,
                          const float* const* lses, void* out, int32_t out_dtype, float* lse,
                          void* stream) {
  if (batch < 1 || heads < 1 || rows < 1 || head_dim < 1)
    return fail(RA_EINVAL, "batch, heads, rows and head_dim must be >= 1");
  if (n_parts < 1 || n_parts > RA_MAX_PARTS)
    return fail(RA_EINVAL, "n_parts %d not in [1, %d]", n_parts, RA_MAX_PARTS);
  if ((parts_dtype != RA_F32 && parts_dtype != RA_BF16) || (out_dtype != RA_F32 && out_dtype != RA_BF16))
    return fail(RA_EINVAL, "unknown dtype");
  if (head_dim % 4 != 0 || 256 % head_dim != 0)
    return fail(RA_EUNSUPPORTED, "head_dim %d must be a multiple of 4 dividing 256", head_dim);
  const int64_t n_rows = mul_sat(mul_sat(batch, heads), rows);
  if (n_rows > ((int64_t)1 << 40)) return fail(RA_EINVAL, "batch * heads * rows too large");
  if (!outs || !lses || !out || !lse) return fail(RA_EINVAL, "outs, lses, out and lse must be set");
  const uintptr_t oa = parts_dtype == RA_F32 ? 16 : 8;
  const uintptr_t wa = out_dtype == RA_F32 ? 16 : 8;
  if (!aligned(out, wa) || !aligned(lse, 4)) return fail(RA_EINVAL, "out / lse misaligned");
  ra::MergeParams p;
  std::memset(&p, 0, sizeof p);
  for (int k = 0; k < n_parts; ++k) {
    if (!outs[k] || !lses[k]) return fail(RA_EINVAL, "outs[%d] / lses[%d] is NULL", k, k);
    if (!aligned(outs[k], oa) || !aligned(lses[k], 4))
      return fail(RA_EINVAL, "outs[%d] / lses[%d] misaligned", k, k);
    if (k > 0 && (outs[k] == out || lses[k] == lse))
      return fail(RA_EINVAL, "only part 0 may alias the output");
    p.outs[k] = outs[k];
    p.lses[k] = lses[k];
  }
  if (outs[0] == out && parts_dtype != out_dtype)
    return fail(RA_EINVAL, "in-place merge needs parts_dtype == out_dtype");
  p.out = out;
  p.lse = lse;
  p.n_rows = n_rows;
  p.head_dim = head_dim;
  p.n_parts = n_parts;
  hipError_t e = ra::launch_merge(p, parts_dtype, out_dtype, (hipStream_t)stream);
  if (e != hipSuccess) return fail(RA_EHIP, "merge launch failed: %s", hipGetErrorString(e));
  return ok();
}



ra_status ring_attn_merge_strided(int32_t batch, int32_t heads, int64_t rows, int32_t head_dim,
                                  int32_t n_parts, const void* outs, int64_t out_stride, int32_t parts_dtype,
                                  const float* lses, int64_t lse_stride, void* out, int32_t out_dtype,
                                  float* lse, void* stream) {
  if (batch < 1 || heads < 1 || rows < 1 || head_dim < 1)
    return fail(RA_EINVAL, "batch, heads, rows and head_dim must be >= 1");
  if (n_parts < 1) return fail(RA_EINVAL, "n_parts must be >= 1");
  if ((parts_dtype != RA_F32 && parts_dtype != RA_BF16) || (out_dtype != RA_F32 && out_dtype != RA_BF16))
    return fail(RA_EINVAL, "unknown dtype");
  if (head_dim % 4 != 0 || 256 % head_dim != 0)
    return fail(RA_EUNSUPPORTED, "head_dim %d must be a multiple of 4 dividing 256", head_dim);
  const int64_t n_rows = mul_sat(mul_sat(batch, heads), rows);
  if (n_rows > ((int64_t)1 << 40)) return fail(RA_EINVAL, "batch * heads * rows too large");
  if (!outs || !lses || !out || !lse) return fail(RA_EINVAL, "outs, lses, out and lse must be set");
  if (out_stride < n_rows * head_dim || lse_stride < n_rows)
    return fail(RA_EINVAL, "strides must be at least one part (%lld elements / %lld lse values)",
                (long long)(n_rows * head_dim), (long long)n_rows);
  if (out_stride > ((int64_t)1 << 46) / n_parts || lse_stride > ((int64_t)1 << 46) / n_parts)
    return fail(RA_EINVAL, "part strides too large");
  const int64_t pes = parts_dtype == RA_F32 ? 4 : 2, oes = out_dtype == RA_F32 ? 4 : 2;
  if (!aligned(outs, 4 * pes) || (out_stride * pes) % (4 * pes) != 0 || !aligned(lses, 4))
    return fail(RA_EINVAL, "parts misaligned (outs and out_stride must keep 4-element groups aligned)");
  if (!aligned(out, 4 * oes) || !aligned(lse, 4)) return fail(RA_EINVAL, "out / lse misaligned");
  // The output may be part 0 exactly; it must not overlap any other part.
  const char* p0 = (const char*)outs;
  const char* pend = p0 + (n_parts - 1) * out_stride * pes + n_rows * head_dim * pes;
  const char* o0 = (const char*)out;
  const char* oend = o0 + n_rows * head_dim * oes;
  if (o0 != p0 && o0 < pend && oend > p0) return fail(RA_EINVAL, "out overlaps the parts other than part 0");
  const char* l0 = (const char*)lses;
  const char* lend = l0 + ((n_parts - 1) * lse_stride + n_rows) * 4;
  if ((const char*)lse != l0 && (const char*)lse < lend && (const char*)(lse + n_rows) > l0)
    return fail(RA_EINVAL, "lse overlaps the parts other than part 0");
  if (o0 == p0 && parts_dtype != out_dtype) return fail(RA_EINVAL, "in-place merge needs parts_dtype == out_dtype");
  ra::MergeParams p;
  std::memset(&p, 0, sizeof p);
  p.strided = 1;
  p.outs_base = outs;
  p.lses_base = lses;
  p.out_stride = out_stride;
  p.lse_stride = lse_stride;
  p.out = out;
  p.lse = lse;
  p.n_rows = n_rows;
  p.head_dim = head_dim;
  p.n_parts = n_parts;
  hipError_t e = ra::launch_merge(p, parts_dtype, out_dtype, (hipStream_t)stream);
  if (e != hipSuccess) return fail(RA_EHIP, "merge launch failed: %s", hipGetErrorString(e));
  return ok();
}

ra_status ring_attn_decode(const ra_attn_desc* desc, const void* q, int32_t n_blocks,
                           const void* const* k_blocks, const void* const* v_blocks, int32_t n_splits,
                           float* out_parts, float* lse_parts, void* stream) {
  ra_status st = check_desc(desc);
  if (st != RA_OK) return st;
  if (desc->in_dtype != RA_BF16) return fail(RA_EUNSUPPORTED, "decode takes bf16 inputs");
  if (desc->out_dtype != RA_F32) return fail(RA_EUNSUPPORTED, "decode partials are fp32 (out_dtype RA_F32)");
  if (desc->flags != 0) return fail(RA_EINVAL, "decode takes no flags");
  const int32_t group = desc->h_q / desc->h_kv;
  if (group > 32) return fail(RA_EUNSUPPORTED, "h_q / h_kv = %d > 32 query heads per kv head", group);
  const int32_t c = desc->n_shards;
  if (n_blocks < 1 || n_blocks > c || n_blocks > RA_MAX_BLOCKS)
    return fail(RA_EINVAL, "n_blocks %d not in [1, min(n_shards, %d)]", n_blocks, RA_MAX_BLOCKS);
  const int64_t n_loc = desc->seq_len / c;
  if (n_splits < 1 || n_splits > n_loc) return fail(RA_EINVAL, "n_splits %d not in [1, %lld]", n_splits, (long long)n_loc);
  if (!q || !k_blocks || !v_blocks || !out_parts || !lse_parts)
    return fail(RA_EINVAL, "q, k_blocks, v_blocks, out_parts and lse_parts must be set");
  if (!aligned(q, 16) || !aligned(out_parts, 16) || !aligned(lse_parts, 4))
    return fail(RA_EINVAL, "q / out_parts must be 16-byte aligned, lse_parts 4-byte");
  const int64_t items = mul_sat(mul_sat(mul_sat(n_blocks, n_splits), desc->batch), desc->h_kv);
  if (items >= ((int64_t)1 << 31)) return fail(RA_EUNSUPPORTED, "too many (block, range, batch, kv head) items");
  ra::DecodeParams p;
  std::memset(&p, 0, sizeof p);
  for (int t = 0; t < n_blocks; ++t) {
    if (!k_blocks[t] || !v_blocks[t]) return fail(RA_EINVAL, "k_blocks[%d] / v_blocks[%d] is NULL", t, t);
    if (!aligned(k_blocks[t], 16) || !aligned(v_blocks[t], 16))
      return fail(RA_EINVAL, "k_blocks[%d] / v_blocks[%d] must be 16-byte aligned", t, t);
    p.k[t] = k_blocks[t];
    p.v[t] = v_blocks[t];
  }
  p.q = q;
  p.out_parts = out_parts;
  p.lse_parts = lse_parts;
  p.n_loc = n_loc;
  p.n_blocks = n_blocks;
  p.n_splits = n_splits;
  p.batch = desc->batch;
  p.h_q = desc->h_q;
  p.h_kv = desc->h_kv;
  p.group = group;
  p.n_items = (int32_t)items;
  p.scale_log2 = (float)((double)desc->scale * 1.4426950408889634);
  hipError_t e = ra::launch_decode_bf16(p, desc->head_dim, (hipStream_t)stream);
  if (e != hipSuccess) return fail(RA_EHIP, "decode launch failed: %s", hipGetErrorString(e));
  return ok();
}

}  // extern "C"
