"""Cost model behind the pages' modelled figures (memory, ring traffic, compute).

TEST INFRASTRUCTURE ONLY, like the rest of ``oracle/``: imported by ``tests/``,
never by the product package.  Nothing here is on the attention path; it
restates, as plain arithmetic, the model of the "Splitting the Sequence" plate
(section "Workshop") and the KV-memory column of the "Sequence / context
parallelism" notes (section 7, "Performance"), so that the figures those pages
print can be reproduced and the same model evaluated for other links and
compute rates (how the shard pass would overlap a real ring).

Readings where the pages leave a quantity unstated (each is pinned by a
printed figure in ``tests/test_cost_model.py``):

* GB means 10**9 bytes; "1M tokens" means 10**6 tokens.
* Activation memory per layer is the Korthikanti et al. estimate with
  FlashAttention, i.e. without the stored score matrix: 34 bytes times
  tokens times hidden size, divided by the tensor-parallel degree t (their
  sequence-parallel form) and by the context-parallel degree c; a pipeline
  stage holds layers / p of the layers.
* Per layer, the ring moves the bf16 keys and values of the device's own
  n_kv / t heads over the whole sequence; the fraction (c - 1)/c of those
  bytes leaves the device, over one link of the stated rate.
* The attention arithmetic of a layer on one device is the causal forward
  work of the busiest device (all equal under the zig-zag split): 4 * d FLOP
  per visible (query, key) pair and query head, run at a fraction of the
  peak.
* The H100 peak is the dense bf16 figure of the SXM part, 989.4 TFLOP/s.
"""
from __future__ import annotations

from dataclasses import dataclass

from . import SPLIT_ZIGZAG, pair_counts

BF16_BYTES = 2
H100_BF16_DENSE_FLOPS = 989.4e12


@dataclass(frozen=True)
class Model:
    layers: int
    hidden: int
    n_q_heads: int
    n_kv_heads: int
    head_dim: int


# Shapes of the two models the pages use (published architecture figures).
LLAMA3_405B = Model(layers=126, hidden=16384, n_q_heads=128, n_kv_heads=8, head_dim=128)
LLAMA3_8B = Model(layers=32, hidden=4096, n_q_heads=32, n_kv_heads=8, head_dim=128)


def gbit_per_s(gbit: float) -> float:
    """A network rate in Gb/s as bytes per second."""
    return gbit * 1e9 / 8


def heads_per_device(n_heads: int, tp: int) -> int:
    """Heads one tensor-parallel rank holds (at least one; KV heads are
    replicated when t exceeds their number)."""
    return max(1, n_heads // tp)


def activation_bytes_per_device(m: Model, seq_len: int, tp: int, pp: int, cp: int = 1) -> float:
    """Activations of one sequence held by one device ("Splitting the
    Sequence", Workshop): 34 * s * h / (t * c) bytes per layer, times the
    layers of one pipeline stage."""
    per_layer = 34.0 * seq_len * m.hidden / (tp * cp)
    return per_layer * m.layers / pp


def ring_bytes_per_layer(m: Model, seq_len: int, tp: int, cp: int, elem_bytes: int = BF16_BYTES) -> float:
    """Bytes one device sends round the ring per layer ("Splitting the
    Sequence", Workshop): its share of K and V over the sequence, (c-1)/c of it."""
    share = 2.0 * seq_len * heads_per_device(m.n_kv_heads, tp) * m.head_dim * elem_bytes
    return share * (cp - 1) / cp


def attention_flop_per_layer(m: Model, seq_len: int, tp: int, cp: int, split: int = SPLIT_ZIGZAG) -> float:
    """Causal forward attention FLOP of the busiest device for one layer:
    4 * d per visible (query, key) pair, per query head on this device."""
    busiest = int(pair_counts(seq_len, cp, split, causal=True).max())
    return 4.0 * m.head_dim * heads_per_device(m.n_q_heads, tp) * busiest


def transfer_over_compute(m: Model, seq_len: int, tp: int, cp: int, link_bytes_per_s: float,
                          flops_per_s: float) -> dict:
    """Ring transfer time against attention time, per layer per device."""
    nbytes = ring_bytes_per_layer(m, seq_len, tp, cp)
    flop = attention_flop_per_layer(m, seq_len, tp, cp)
    t_x, t_c = nbytes / link_bytes_per_s, flop / flops_per_s
    return {"bytes": nbytes, "flop": flop, "transfer_s": t_x, "compute_s": t_c, "ratio": t_x / t_c}


def kv_cache_bytes(m: Model, tokens: float, tp: int = 1, sp: int = 1, elem_bytes: int = BF16_BYTES) -> float:
    """K and V of every layer for ``tokens`` tokens ("Sequence / context
    parallelism" notes, section 7), split over t ranks by heads and over
    sp ranks by tokens."""
    per_token = m.layers * 2 * m.n_kv_heads * m.head_dim * elem_bytes
    return per_token * tokens / (tp * sp)
