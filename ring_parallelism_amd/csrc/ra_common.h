// Internal definitions shared by the library's kernels and host code.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "../../include/ring_attn.h"

namespace ra {

// Global position of local token t of shard r (n_loc = S/c tokens per
// shard).  Positions ascend with t for every split, which the kernels use to
// classify a tile from its first and last row alone.
//   contiguous: r*n_loc + t
//   zig-zag:    chunk r then chunk 2c-1-r of n = n_loc/2 tokens each
//   striped:    t*c + r
__host__ __device__ inline int64_t token_pos(int64_t r, int64_t t, int64_t n_loc, int32_t c,
                                             int32_t split) {
  if (split == RA_SPLIT_ZIGZAG) {
    const int64_t n = n_loc >> 1;
    return t < n ? r * n + t : (2 * (int64_t)c - 1 - r) * n + (t - n);
  }
  if (split == RA_SPLIT_STRIPED) return t * c + r;
  return r * n_loc + t;
}

__host__ __device__ inline int64_t clamp64(int64_t x, int64_t lo, int64_t hi) {
  return x < lo ? lo : (x > hi ? hi : x);
}

// Number of local keys of block j whose global position is <= p.  Because
// positions ascend within a block, these keys are the block's first
// count_upto() rows.
__host__ __device__ inline int64_t count_upto(int64_t j, int64_t p, int64_t n_loc, int32_t c,
                                              int32_t split) {
  if (p < 0) return 0;
  if (split == RA_SPLIT_ZIGZAG) {
    const int64_t n = n_loc >> 1;
    return clamp64(p - j * n + 1, 0, n) + clamp64(p - (2 * (int64_t)c - 1 - j) * n + 1, 0, n);
  }
  if (split == RA_SPLIT_STRIPED) return p < j ? 0 : clamp64((p - j) / c + 1, 0, n_loc);
  return clamp64(p - j * n_loc + 1, 0, n_loc);
}

// 32-bit forms for the attention kernels (global positions < 2^31 there).
__device__ inline int token_pos32(int r, int t, int n_loc, int c, int split) {
  if (split == RA_SPLIT_ZIGZAG) {
    const int n = n_loc >> 1;
    return t < n ? r * n + t : (2 * c - 1 - r) * n + (t - n);
  }
  if (split == RA_SPLIT_STRIPED) return t * c + r;
  return r * n_loc + t;
}

__device__ inline int clamp32(int x, int lo, int hi) { return x < lo ? lo : (x > hi ? hi : x); }

__device__ inline int count_upto32(int j, int p, int n_loc, int c, int split) {
  if (p < 0) return 0;
  if (split == RA_SPLIT_ZIGZAG) {
    const int n = n_loc >> 1;
    return clamp32(p - j * n + 1, 0, n) + clamp32(p - (2 * c - 1 - j) * n + 1, 0, n);
  }
  if (split == RA_SPLIT_STRIPED) return p < j ? 0 : clamp32((p - j) / c + 1, 0, n_loc);
  return clamp32(p - j * n_loc + 1, 0, n_loc);
}

struct FwdParams {
  const void* q;
  void* out;
  float* lse;
  unsigned long long* stats;
  int64_t n_loc;       // S / c
  int32_t c, split, rank, n_blocks;
  int32_t batch, h_q, h_kv, group;  // group = h_q / h_kv
  int32_t causal;
  int32_t n_qtiles;    // ceil(n_loc / tile_q)
  int32_t n_pairs;     // ceil(n_qtiles / 2): each workgroup takes q-tiles p and n_qtiles-1-p
  int32_t n_ktiles;    // ceil(n_loc / tile_k)
  float scale;         // softmax scale
  float scale_log2;    // scale * log2(e)
  int32_t sync_loads;  // wait for each batch of tile loads right after issuing it
  int32_t qo_natural;  // q / out / lse rows are global positions of [B, h_q, S, d] tensors
  int32_t event_counts;  // stats has slots 4 and 5 (reference raises, exact recomputations)
  int64_t qo_rows;     // rows per (batch, head) of q / out / lse: S/c, or S when qo_natural
  // Split over the block list: n_splits groups of consecutive blocks, each
  // written as a partial to out / lse + split * part_stride (1: no split).
  int32_t n_splits, grid_per_split;
  int64_t part_stride_out, part_stride_lse;
  // Every rank in one launch (all_ranks != 0): rank r's q / out / lse start
  // r * rank_stride_* elements in, its blocks follow the ring order and
  // k[] / v[] are indexed by owner.
  int32_t all_ranks, grid_per_rank;
  int64_t rank_stride_q, rank_stride_out, rank_stride_lse;
  int32_t owner[RA_MAX_BLOCKS];
  const void* k[RA_MAX_BLOCKS];
  const void* v[RA_MAX_BLOCKS];
};

struct MergeParams {
  const void* outs[RA_MAX_PARTS];
  const float* lses[RA_MAX_PARTS];
  // Strided form (strided != 0): part k at outs_base + k * out_stride elements
  // and lses_base + k * lse_stride, for any number of parts.
  const void* outs_base;
  const float* lses_base;
  int64_t out_stride, lse_stride;
  int32_t strided;
  void* out;
  float* lse;
  int64_t n_rows;     // batch * heads * rows
  int32_t head_dim;
  int32_t n_parts;
};

// Split-KV decode: one query token per (batch, query head) against key ranges
// of the blocks; one wave per (part, batch, kv head), part = block * n_splits + range.
struct DecodeParams {
  const void* q;          // [B, h_q, d] bf16
  float* out_parts;       // [n_parts, B, h_q, d]
  float* lse_parts;       // [n_parts, B, h_q]
  int64_t n_loc;          // keys per block
  int32_t n_blocks, n_splits, batch, h_q, h_kv, group;
  int32_t n_items;        // n_blocks * n_splits * batch * h_kv
  float scale_log2;       // scale * log2(e)
  const void* k[RA_MAX_BLOCKS];
  const void* v[RA_MAX_BLOCKS];
};

// Records the thread's last-error message; returns code.
ra_status set_error(ra_status code, const char* fmt, ...);

// Launchers (defined in the kernel translation units).
hipError_t launch_partition(int64_t S, int32_t c, int32_t split, int64_t* perm, const void* src,
                            void* dst, int64_t outer, int64_t inner_bytes, bool inverse,
                            hipStream_t stream);
hipError_t launch_fwd_f32(const FwdParams& p, int32_t head_dim, hipStream_t stream);
hipError_t launch_fwd_bf16(const FwdParams& p, int32_t head_dim, int32_t out_dtype,
                           hipStream_t stream);
hipError_t launch_merge(const MergeParams& p, int32_t parts_dtype, int32_t out_dtype,
                        hipStream_t stream);
void tile_shape_f32(int32_t head_dim, int32_t* tq, int32_t* tk);
void tile_shape_bf16(int32_t head_dim, int32_t* tq, int32_t* tk);
hipError_t launch_decode_bf16(const DecodeParams& p, int32_t head_dim, hipStream_t stream);

}  // namespace ra
