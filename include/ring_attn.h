/* ring_attn.h -- C ABI of the MI355X (gfx950) ring-attention shard library.
 *
 * One device's share of exact causal blockwise ring attention.  Each device
 * holds the queries of its own tokens and sees the key/value blocks of every
 * device in ring order; each block's partial result is folded in with an
 * online softmax (running max m, normaliser l, output rescaled when the max
 * rises) and the output is divided by l at the end ("Sequence / context
 * parallelism" notes, section 4 "Ring Attention -- the core algorithm";
 * "Splitting the Sequence", intro).  On one GPU the blocks that would arrive
 * from the ring neighbours are read from HBM in ring order.
 *
 * Conventions shared by every entry point
 *   - Every function returns ra_status; RA_OK (0) on success.  On failure
 *     nothing was launched and ring_attn_last_error() describes the cause.
 *   - Device buffers are owned by the caller; the library allocates no
 *     device memory and is thread-safe.  Its only device state is the static
 *     scratch of ring_attn_shard_fwd_split_noalloc (see there).  Host arrays
 *     passed in (block_owner, k_blocks, v_blocks, outs, lses) are read during
 *     the call only.
 *   - `stream` is a hipStream_t (NULL = the default stream).  Work is enqueued
 *     on it and the call returns at once; faults surface at the caller's next
 *     synchronisation.
 *   - Tensors are dense and row-major with the last dimension contiguous;
 *     device pointers must be 16-byte aligned (lse and stats: 4 / 8 bytes).
 *   - No C++ exception crosses this interface.
 */
#ifndef RING_ATTN_H
#define RING_ATTN_H

#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef int32_t ra_status;
enum {
  RA_OK = 0,
  RA_EINVAL = 1,        /* invalid argument (null, divisibility, range, alignment) */
  RA_EUNSUPPORTED = 2,  /* valid but not implemented (head_dim, dtype pairing, too many blocks) */
  RA_EHIP = 3           /* the HIP runtime refused a launch */
};

/* Token placement of the shards.
 *   CONTIGUOUS: shard r holds tokens [r*S/c, (r+1)*S/c) ("Sequence / context
 *               parallelism" notes, section 1 diagram).
 *   ZIGZAG:     the sequence is cut into 2c chunks of n = S/(2c) tokens and
 *               shard r holds chunks r and 2c-1-r, in that order
 *               ("Splitting the Sequence", intro and Terms: zig-zag split).
 *   STRIPED:    round-robin; shard r holds tokens r, r+c, r+2c, ... (notes,
 *               section 5 "Striped / zigzag attention": interleaved pattern).
 * Within a shard the tokens keep ascending global position. */
enum { RA_SPLIT_CONTIGUOUS = 0, RA_SPLIT_ZIGZAG = 1, RA_SPLIT_STRIPED = 2 };

enum { RA_F32 = 0, RA_BF16 = 1 };

#define RA_MAX_BLOCKS 128  /* ring blocks per ring_attn_shard_fwd call */
#define RA_MAX_PARTS 64    /* partial results per ring_attn_merge call */
#define RA_ABI_VERSION 3

typedef struct {
  int64_t seq_len;   /* S, global tokens; S % c == 0 (S % 2c == 0 for ZIGZAG) */
  int32_t n_shards;  /* c >= 1 */
  int32_t split;     /* RA_SPLIT_*: fixes the global position of every shard-local token */
  int32_t batch;     /* B >= 1 */
  int32_t h_q;       /* query heads */
  int32_t h_kv;      /* key/value heads; h_q % h_kv == 0 and query head h reads
                        key/value head h / (h_q / h_kv) (grouped-query attention,
                        "Splitting the Sequence", intro: 8 KV against 128 query heads) */
  int32_t head_dim;  /* d: 64 or 128 */
  int32_t in_dtype;  /* RA_F32 or RA_BF16, the dtype of Q, K and V */
  int32_t out_dtype; /* RA_F32 or RA_BF16; bf16 inputs may write fp32 out */
  int32_t causal;    /* 1: key position <= query position (global positions); 0: all keys */
  float scale;       /* softmax scale applied to q.k: finite and > 0 (e.g. 1/sqrt(d)) */
  uint32_t flags;    /* RA_FLAG_* bits; 0 for normal use */
} ra_attn_desc;

/* Measurement switch for timing the pass with its block transfers hidden
 * behind the arithmetic and without ("Sequence / context parallelism" notes,
 * section 10, exercise C): the key/value tiles are still prefetched into the
 * LDS ring, but every wave waits for each batch of tile loads right after
 * issuing it, so no transfer runs beside the attention arithmetic.  Results
 * are bitwise the same.  bf16 inputs only (RA_EUNSUPPORTED with fp32
 * inputs). */
#define RA_FLAG_SYNC_LOADS 1u

/* q, out and lse are the natural-order, full-sequence tensors [B, h_q, S, d]
 * and [B, h_q, S] instead of shard tensors: the call reads the queries of
 * shard `rank` at their global positions and writes its outputs there, so
 * the gather of Q and the scatter of out back to natural order happen inside
 * the kernel and no shard copy of Q or out exists ("Splitting the Sequence",
 * intro: device k holds chunks k and 2c-1-k; the notes, section 5).  After
 * the calls for every rank, out and lse hold the whole sequence's result.
 * K and V blocks stay in shard layout (the blocks that travel the ring). */
#define RA_FLAG_NATURAL_QO 2u

/* stats (when not NULL) holds RA_STATS_EVENTS_LEN int64 instead of 4: slot 4
 * counts the mid-pass raises of a row's softmax reference -- the online
 * softmax rescaling its earlier partial sums because a later block holds a
 * larger score ("Sequence Parallelism and Ring Attention Quiz", Q3 and Q7) --
 * summed over rows, batch and heads; slot 5 the query tiles that were recomputed by the plain
 * per-tile online softmax (an exponential left the fp32 range between two
 * reference checks, or a row of the first tile sees no key).  Both depend on
 * the data and on the tile order, not only on the shapes.  bf16 inputs; with
 * fp32 inputs slots 4 and 5 stay 0. */
#define RA_FLAG_EVENT_COUNTS 4u
#define RA_STATS_EVENTS_LEN 6

/* Shard placement and optional gather into shard-major order: which
 * tokens each device of the ring holds ("Splitting the Sequence", intro and
 * Terms: the zig-zag split of 2c chunks; "Sequence / context parallelism"
 * notes, section 1 for contiguous shards and section 5 for the interleaved
 * and zig-zag placements that balance the causal work).
 *
 * perm (device int64[S], may be NULL): perm[r*(S/c) + t] = global position
 *   of shard r's t-th token under `split`.
 * src, dst (device, both NULL or both set): src viewed as
 *   [outer][S][inner_bytes] in natural token order, dst as
 *   [c][outer][S/c][inner_bytes]; dst[r][o][t] = src[o][perm[r*(S/c)+t]].
 *   With a [B, H, S, d] tensor: outer = B*H, inner_bytes = d * element size,
 *   and dst[r] is shard r's [B, H, S/c, d] tensor.  src and dst must not
 *   overlap.
 * Errors: RA_EINVAL for S < 1, c < 1, S not divisible as `split` needs,
 *   unknown split, perm == src == NULL, outer < 1 or inner_bytes < 1 with a
 *   gather, or misaligned pointers. */
ra_status zigzag_partition(int64_t seq_len, int32_t n_shards, int32_t split, int64_t* perm,
                           const void* src, void* dst, int64_t outer, int64_t inner_bytes,
                           void* stream);

/* The inverse placement: scatter shard-major rows back to natural order
 * (the output of a sequence-parallel layer returned to token order; same
 * passages as zigzag_partition).
 * src viewed as [c][outer][S/c][inner_bytes], dst as [outer][S][inner_bytes];
 * dst[o][perm[r*(S/c)+t]] = src[r][o][t].  Same errors as zigzag_partition. */
ra_status zigzag_unpartition(int64_t seq_len, int32_t n_shards, int32_t split,
                             const void* src, void* dst, int64_t outer, int64_t inner_bytes,
                             void* stream);

/* One shard's queries against a sequence of key/value blocks: the ring
 * pass of one device, its queries kept in place while the blocks arrive in
 * ring order, each folded in by the online softmax ("Sequence / context
 * parallelism" notes, section 4 "Ring Attention -- the core algorithm";
 * "Splitting the Sequence", intro; "Sequence Parallelism and Ring Attention
 * Quiz", Q2-Q4 and Q7).
 *
 * rank         : the shard r in [0, c) whose queries q holds.
 * q            : device [B, h_q, S/c, d] in_dtype, shard r's tokens in shard order
 *                ([B, h_q, S, d] in natural order with RA_FLAG_NATURAL_QO).
 * n_blocks     : number of blocks to fold, 1..min(c, RA_MAX_BLOCKS).
 * block_owner  : host int32[n_blocks], the shard each block belongs to, in
 *                visiting order; distinct values in [0, c).  NULL = ring
 *                order owner[t] = (r - t) mod c, t = 0..n_blocks-1 (at step t
 *                a device holds the block that started t hops upstream).
 * k_blocks,
 * v_blocks     : host arrays of n_blocks device pointers; block t is shard
 *                block_owner[t]'s keys / values, [B, h_kv, S/c, d] in_dtype.
 * out          : device [B, h_q, S/c, d] out_dtype ([B, h_q, S, d] with
 *                RA_FLAG_NATURAL_QO: only shard r's rows are written).  With all c blocks it is
 *                the exact attention output of the shard's queries; with a
 *                subset, the partial result over those keys only.
 * lse          : device fp32 [B, h_q, S/c] ([B, h_q, S] with
 *                RA_FLAG_NATURAL_QO): natural log of the sum of
 *                exp(scale * q.k) over the visible keys of the folded
 *                blocks; -inf (with out = 0) for a row that sees none.
 * stats        : device int64[4] or NULL; atomically ADDED to:
 *                [0] visible (query, key) pairs summed over batch and query
 *                    heads, [1] full tiles, [2] partially masked tiles,
 *                [3] skipped (fully masked) tiles; tiles are
 *                ring_attn_tile_shape() query rows x key rows of one block,
 *                counted per (batch, query head).
 * Errors: RA_EINVAL for a bad descriptor (see ra_attn_desc), rank or
 *   n_blocks out of range, owners out of range or repeated, null or
 *   misaligned pointers; RA_EUNSUPPORTED for head_dim not 64/128, f32 inputs
 *   with bf16 output, S >= 2^31 - 1 or S/c * d >= 2^31; RA_EHIP on launch
 *   failure. */
ra_status ring_attn_shard_fwd(const ra_attn_desc* desc, int32_t rank, const void* q,
                              int32_t n_blocks, const int32_t* block_owner,
                              const void* const* k_blocks, const void* const* v_blocks,
                              void* out, float* lse, int64_t* stats, void* stream);

/* Every shard's ring pass at once: on one GPU, the work all c devices of the
 * ring do in one layer ("Splitting the Sequence", "One sequence, sixteen
 * devices": each device's queries against every block; the notes, section
 * 4).  Equivalent to ring_attn_shard_fwd for every rank r in [0, c) with the
 * ring order, bitwise; with bf16 inputs it is a single launch, so shards too
 * small to fill the device on their own (few query tiles per rank) still do.
 *
 * q_shards     : device [c, B, h_q, S/c, d] in_dtype, shard r at index r (the
 *                layout zigzag_partition's gather writes); with
 *                RA_FLAG_NATURAL_QO the natural-order [B, h_q, S, d].
 * k_blocks,
 * v_blocks     : host arrays of c device pointers; entry j is shard j's keys /
 *                values [B, h_kv, S/c, d] (indexed by owner, not by step).
 * out_shards   : device [c, B, h_q, S/c, d] out_dtype (natural order with the
 *                flag: every row is written once).
 * lse_shards   : device fp32 [c, B, h_q, S/c] (or [B, h_q, S]).
 * stats        : as ring_attn_shard_fwd, summed over the ranks.
 * Errors: as ring_attn_shard_fwd; RA_EUNSUPPORTED for c > RA_MAX_BLOCKS.
 * fp32 inputs run one launch per rank. */
ra_status ring_attn_all_shards_fwd(const ra_attn_desc* desc, const void* q_shards,
                                   const void* const* k_blocks, const void* const* v_blocks,
                                   void* out_shards, float* lse_shards, int64_t* stats, void* stream);

/* Tile shape (query rows, keys) that ring_attn_shard_fwd uses for `desc`,
 * i.e. the unit its stats count (the work accounting behind the balance
 * comparison of causal placements: "Splitting the Sequence", "One sequence,
 * sixteen devices", the busiest device's share of the work under the
 * contiguous split).  Errors as for the descriptor checks. */
ra_status ring_attn_tile_shape(const ra_attn_desc* desc, int32_t* tile_q, int32_t* tile_k);

/* n-way merge of partial results over disjoint key sets.
 *
 * For each of batch*heads*rows rows: LSE = log sum_k exp(lse_k) and
 * out = sum_k exp(lse_k - LSE) * out_k; parts with lse_k = -inf carry no
 * keys, and a row whose parts are all -inf gives (0, -inf).  This is the fold
 * each ring step applies ("Sequence / context parallelism" notes, section 4).
 *
 * outs  : host array of n_parts device pointers, each [batch, heads, rows,
 *         head_dim] of parts_dtype.
 * lses  : host array of n_parts device pointers, each fp32 [batch, heads, rows].
 * out   : device [batch, heads, rows, head_dim] out_dtype; lse: device fp32
 *         [batch, heads, rows].  out may be outs[0] and lse may be lses[0]
 *         (in-place accumulation); no other overlap is allowed.
 * Errors: RA_EINVAL for n_parts not in 1..RA_MAX_PARTS, any size < 1, null or
 *   misaligned pointers, unknown dtypes; RA_EUNSUPPORTED for head_dim that is
 *   not a multiple of 4 dividing 256 (every row is then covered by whole
 *   4-element groups, and each group is written only by the thread that read
 *   it, which is what makes the in-place aliasing safe); RA_EHIP on launch
 *   failure. */
ra_status ring_attn_merge(int32_t batch, int32_t heads, int64_t rows, int32_t head_dim,
                          int32_t n_parts, const void* const* outs, int32_t parts_dtype,
                          const float* const* lses, void* out, int32_t out_dtype, float* lse,
                          void* stream);

/* ring_attn_shard_fwd for shards too small to fill the device: the block
 * list is cut into n_splits groups of consecutive blocks (1 <= n_splits <=
 * n_blocks), the groups run concurrently, each writing a partial result
 * (the online-softmax fold over its blocks, "Sequence / context parallelism"
 * notes, section 4) to the caller's workspace, and the partials are folded
 * into out / lse by the merge of ring_attn_merge.  The result equals
 * ring_attn_shard_fwd's up to rounding; stats count the same tiles.
 *
 * work_out: device fp32 [n_splits, B, h_q, S/c, d]; work_lse: device fp32
 * [n_splits, B, h_q, S/c]; both caller-owned scratch, overwritten, and must
 * not overlap out / lse.  bf16 inputs only, no RA_FLAG_NATURAL_QO
 * (RA_EUNSUPPORTED).  Other arguments and errors as ring_attn_shard_fwd. */
ra_status ring_attn_shard_fwd_split(const ra_attn_desc* desc, int32_t rank, const void* q, int32_t n_blocks,
                                    const int32_t* block_owner, const void* const* k_blocks,
                                    const void* const* v_blocks, int32_t n_splits, float* work_out,
                                    float* work_lse, void* out, float* lse, int64_t* stats, void* stream);

/* ring_attn_shard_fwd_split without a workspace, for callers that cannot
 * allocate device memory (code under HIP graph capture, tight serving loops,
 * harnesses that forbid hipMalloc).  The partial results live in a static
 * device array of the library -- RA_NOALLOC_MAX_PARTIAL_FLOATS floats for the
 * partial outputs and RA_NOALLOC_MAX_LSE_FLOATS for their lse, 64.5 MiB that
 * each GPU the library runs on holds until the process ends -- so the call
 * allocates nothing.  n_splits * B * h_q * S/c * head_dim beyond the first
 * limit (or n_splits * B * h_q * S/c beyond the second) is RA_EINVAL with a
 * message; 4 splits of the 8 192-token (32 / 8 heads) and 32 768-token
 * (16 / 1 heads) shards fit exactly.  All calls on one GPU share its array:
 * calls that may overlap on one GPU (other streams, other host threads) race
 * and must be serialised by the caller.  Other arguments, results and errors
 * as ring_attn_shard_fwd_split. */
#define RA_NOALLOC_MAX_PARTIAL_FLOATS (1 << 24)
#define RA_NOALLOC_MAX_LSE_FLOATS (1 << 17)
ra_status ring_attn_shard_fwd_split_noalloc(const ra_attn_desc* desc, int32_t rank, const void* q,
                                            int32_t n_blocks, const int32_t* block_owner,
                                            const void* const* k_blocks, const void* const* v_blocks,
                                            int32_t n_splits, void* out, float* lse, int64_t* stats,
                                            void* stream);

/* ring_attn_merge with the parts in one buffer (the same fold, "Sequence /
 * context parallelism" notes, section 4; also the gather of decode partials,
 * section 7): part k's out starts
 * out_stride elements after part k-1's (parts_dtype elements, out_stride >=
 * batch*heads*rows*head_dim) and its lse lse_stride values after part k-1's
 * (lse_stride >= batch*heads*rows).  Any n_parts >= 1.  out / lse may be part
 * 0 exactly and must not overlap any other part.  Same formula, alignment
 * (outs and out_stride keep 4-element groups aligned) and errors as
 * ring_attn_merge. */
ra_status ring_attn_merge_strided(int32_t batch, int32_t heads, int64_t rows, int32_t head_dim,
                                  int32_t n_parts, const void* outs, int64_t out_stride, int32_t parts_dtype,
                                  const float* lses, int64_t lse_stride, void* out, int32_t out_dtype,
                                  float* lse, void* stream);

/* Split-KV decode ("Sequence / context parallelism" notes, section 7: decode
 * has one query, and attention over a key/value cache spread across devices
 * is a split-K with a gather of partial results; section 9, pitfalls: decode
 * gains less from sequence parallelism than prefill).
 *
 * q: [B, h_q, d] bf16, one new token per (sequence, query head), placed after
 *   every cached key, so every key is visible (desc->causal changes nothing).
 * k_blocks / v_blocks: host arrays of n_blocks device pointers (1 <= n_blocks
 *   <= min(n_shards, RA_MAX_BLOCKS)), each a cache block [B, h_kv, S/c, d]
 *   bf16 -- on a ring, the blocks a device holds.
 * n_splits: each block's S/c keys are cut into n_splits ranges of
 *   floor/ceil((S/c)/n_splits) keys (1 <= n_splits <= S/c).
 * out_parts: [n_blocks * n_splits, B, h_q, d] fp32 and lse_parts:
 *   [n_blocks * n_splits, B, h_q] fp32 (natural log) receive one partial per
 *   (block t, range s) at index t * n_splits + s: the attention of the query
 *   over that range's keys alone.  Fold them with ring_attn_merge_strided
 *   (out_stride = B*h_q*d, lse_stride = B*h_q) into the full result.
 * desc: in_dtype RA_BF16, out_dtype RA_F32 (the partials), flags 0,
 *   h_q / h_kv <= 32 (RA_EUNSUPPORTED otherwise); split is not used. */
ra_status ring_attn_decode(const ra_attn_desc* desc, const void* q, int32_t n_blocks,
                           const void* const* k_blocks, const void* const* v_blocks, int32_t n_splits,
                           float* out_parts, float* lse_parts, void* stream);

/* Message for the last non-OK status returned on this thread (interface
 * plumbing; no passage of the method). */
const char* ring_attn_last_error(void);

/* RA_ABI_VERSION of the loaded library (interface plumbing). */
int32_t ring_attn_abi_version(void);

#ifdef __cplusplus
}
#endif

#endif /* RING_ATTN_H */
