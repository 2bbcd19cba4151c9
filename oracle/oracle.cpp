// Reference oracle for ring-attention shard results: plain fp64 CPU attention.
//
// TEST INFRASTRUCTURE ONLY.  Nothing on the product path may include, link or
// call this file; it shares no code, header or constant with the HIP library.
// It is slow on purpose: every result is the textbook definition written out,
// one query row at a time, with no blocking, fusion or reordering.
//
// What it computes.  Ring attention is exact: combining the per-block partial
// results with the online softmax gives precisely full softmax attention
// ("Sequence Parallelism and Ring Attention Quiz", Q3 and Q7; "Sequence /
// context parallelism" notes, section 4 "Ring Attention -- the core
// algorithm", and section 10 exercise A, "matches single-GPU attention").  So
// the oracle is full softmax attention over the whole (natural-order)
// sequence, with
//   * a causal mask over global token positions: query i sees key j iff
//     j <= i ("Splitting the Sequence", intro: attention needs every earlier
//     key; self included so that the first token has a defined output),
//   * grouped-query attention: query head h reads key/value head h / (Hq/Hkv)
//     ("Splitting the Sequence", intro: 8 KV heads against 128 query heads),
//   * the log-sum-exp of the scaled scores (natural log) returned beside the
//     output, the state a partial result carries forward,
//   * optionally a restriction of the keys to a given set of positions: this
//     is the partial result of one ring step (the keys of one block).
// A query row that sees no key gets out = 0, lse = -inf.
//
// Inputs are read in their stored type (fp32, raw bf16 bits or fp64) and
// widened exactly to double before any arithmetic.

#include <cmath>
#include <cstdint>
#ifdef _OPENMP
#include <omp.h>
#endif
#include <cstring>
#include <limits>
#include <vector>

namespace {

enum { DT_F32 = 0, DT_BF16 = 1, DT_F64 = 2 };

inline double load(const void* base, int dtype, int64_t idx) {
  if (dtype == DT_F32) return static_cast<double>(static_cast<const float*>(base)[idx]);
  if (dtype == DT_F64) return static_cast<const double*>(base)[idx];
  // bf16: the 16 stored bits are the top half of an fp32 pattern.
  uint32_t bits = static_cast<uint32_t>(static_cast<const uint16_t*>(base)[idx]) << 16;
  float f;
  std::memcpy(&f, &bits, sizeof f);
  return static_cast<double>(f);
}

}  // namespace

extern "C" {

// Full (or key-restricted) softmax attention in fp64.
//
//   q     : [B, Hq, Sq, d]  query rows; row t of q has global position q_pos[t]
//   k, v  : [B, Hkv, S, d]  keys / values in natural order (position = index)
//   q_pos : [Sq] global positions of the q rows
//   rows  : [n_rows] indices into the q rows to evaluate (NULL = all Sq)
//   heads : [n_heads] query heads to evaluate (NULL = all Hq)
//   keys  : [n_keys] key positions allowed (NULL = all S); the causal test is
//           applied on top of this set
//   out   : [B, n_heads, n_rows, d]   lse : [B, n_heads, n_rows]
// Returns 0, or -1 on invalid sizes.
int oracle_attention(const void* q, const void* k, const void* v, int dtype,
                     int64_t B, int64_t Hq, int64_t Hkv, int64_t Sq, int64_t S, int64_t d,
                     const int64_t* q_pos, double scale, int causal,
                     const int64_t* rows, int64_t n_rows,
                     const int64_t* heads, int64_t n_heads,
                     const int64_t* keys, int64_t n_keys,
                     double* out, double* lse) {
  if (B < 1 || Hq < 1 || Hkv < 1 || Hq % Hkv != 0 || Sq < 0 || S < 1 || d < 1) return -1;
  if (!rows) n_rows = Sq;
  if (!heads) n_heads = Hq;
  if (!keys) n_keys = S;
  const int64_t group = Hq / Hkv;
  const int64_t n_items = B * n_heads * n_rows;

#pragma omp parallel
  {
    std::vector<double> qrow(d), score(n_keys), acc(d);
    std::vector<int64_t> vis(n_keys);
#pragma omp for schedule(dynamic, 4)
    for (int64_t item = 0; item < n_items; ++item) {
      const int64_t b = item / (n_heads * n_rows);
      const int64_t hi = (item / n_rows) % n_heads;
      const int64_t ri = item % n_rows;
      const int64_t h = heads ? heads[hi] : hi;
      const int64_t row = rows ? rows[ri] : ri;
      const int64_t pos = q_pos[row];
      const int64_t hk = h / group;

      for (int64_t e = 0; e < d; ++e) qrow[e] = load(q, dtype, ((b * Hq + h) * Sq + row) * d + e);

      // Visible keys: the allowed set, minus later positions when causal.
      int64_t nv = 0;
      for (int64_t t = 0; t < n_keys; ++t) {
        const int64_t j = keys ? keys[t] : t;
        if (!causal || j <= pos) vis[nv++] = j;
      }

      double* o = out + item * d;
      if (nv == 0) {
        for (int64_t e = 0; e < d; ++e) o[e] = 0.0;
        lse[item] = -std::numeric_limits<double>::infinity();
        continue;
      }

      // s_j = scale * <q_i, k_j>
      double mx = -std::numeric_limits<double>::infinity();
      for (int64_t t = 0; t < nv; ++t) {
        const int64_t kbase = ((b * Hkv + hk) * S + vis[t]) * d;
        double dot = 0.0;
        for (int64_t e = 0; e < d; ++e) dot += qrow[e] * load(k, dtype, kbase + e);
        score[t] = scale * dot;
        if (score[t] > mx) mx = score[t];
      }
      // softmax weights exp(s_j - M) / Z applied to v_j
      double z = 0.0;
      for (int64_t e = 0; e < d; ++e) acc[e] = 0.0;
      for (int64_t t = 0; t < nv; ++t) {
        const double w = std::exp(score[t] - mx);
        z += w;
        const int64_t vbase = ((b * Hkv + hk) * S + vis[t]) * d;
        for (int64_t e = 0; e < d; ++e) acc[e] += w * load(v, dtype, vbase + e);
      }
      for (int64_t e = 0; e < d; ++e) o[e] = acc[e] / z;
      lse[item] = mx + std::log(z);
    }
  }
  return 0;
}

int oracle_threads(void) {
#ifdef _OPENMP
  return omp_get_max_threads();
#else
  return 1;
#endif
}

}  // extern "C"
