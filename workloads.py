"""Seeded synthetic inputs and workload shapes for the ring-attention shard.

This module is shared by the tests, the benchmark and the oracle harness.  It
holds no attention arithmetic: only the workload shapes, a seeded Gaussian
draw and the fp32 -> bf16 input quantisation (round to nearest even), so
that both the HIP path and the fp64 oracle receive identical bits.

Draws are counter-addressed: the values of tensor ``t`` at batch ``b``, head
``h`` and natural token positions ``[u*UNIT, (u+1)*UNIT)`` come from their own
PCG64 stream seeded by ``SeedSequence([seed, t, b, h, u])``.  Any subset of
rows can therefore be regenerated without drawing the rest.

Workload shapes follow the pages' setting (Llama 3 405B attention layer: one
tensor-parallel slice of 128 query / 8 key-value heads, head_dim 128, at
131 072 tokens over c = 16 devices; "Splitting the Sequence", Workshop and
"One sequence, sixteen devices").  Values are i.i.d. N(0, sigma^2): the
pages name no dataset, so synthetic Gaussians stand in for activations.
"""
from __future__ import annotations

import concurrent.futures
import dataclasses
import os

import numpy as np

UNIT = 1024          # positions per independently seeded draw unit
TENSOR_Q, TENSOR_K, TENSOR_V = 0, 1, 2

SPLIT_CONTIGUOUS = 0
SPLIT_ZIGZAG = 1
SPLIT_STRIPED = 2


@dataclasses.dataclass(frozen=True)
class Workload:
    name: str
    seq_len: int
    n_shards: int
    split: int
    batch: int
    h_q: int
    h_kv: int
    head_dim: int
    dtype: str          # "f32" or "bf16": dtype of Q, K, V as handed to the GPU
    sigma: float
    causal: bool
    seed: int

    @property
    def n_loc(self) -> int:
        return self.seq_len // self.n_shards

    @property
    def scale(self) -> float:
        return 1.0 / float(np.sqrt(self.head_dim))


# The five workloads (sizes as stated for the ring-attention shard benchmark).
WORKLOADS = [
    Workload("s1k_c4_contig_f32_d64", 1024, 4, SPLIT_CONTIGUOUS, 1, 4, 1, 64, "f32", 1.0, True, 1001),
    Workload("s8k_c8_zigzag_gqa32x8", 8192, 8, SPLIT_ZIGZAG, 1, 32, 8, 128, "bf16", 1.0, True, 1002),
    Workload("s32k_c16_contig_16x1", 32768, 16, SPLIT_CONTIGUOUS, 1, 16, 1, 128, "bf16", 1.0, True, 1003),
    Workload("s32k_c16_zigzag_16x1", 32768, 16, SPLIT_ZIGZAG, 1, 16, 1, 128, "bf16", 1.0, True, 1003),
    Workload("s128k_c16_zigzag_16x1", 131072, 16, SPLIT_ZIGZAG, 1, 16, 1, 128, "bf16", 1.0, True, 1004),
    Workload("s256k_c32_zigzag_64x8", 262144, 32, SPLIT_ZIGZAG, 1, 64, 8, 128, "bf16", 0.5, True, 1005),
]
WORKLOAD_BY_NAME = {w.name: w for w in WORKLOADS}


def f32_to_bf16_bits(x: np.ndarray) -> np.ndarray:
    """Round float32 values to bfloat16 (round to nearest, ties to even).

    Returns the raw 16-bit patterns as uint16.  Inputs are finite draws.
    """
    x = np.ascontiguousarray(x, dtype=np.float32)
    flat = x.reshape(-1).view(np.uint32)
    res = np.empty(flat.shape, dtype=np.uint16)
    step = 1 << 20

    def chunk(lo):
        u = flat[lo:lo + step].copy()
        if np.any((u & np.uint32(0x7F800000)) == np.uint32(0x7F800000)):
            raise ValueError("bf16 rounding expects finite values")
        # Finite patterns are <= 0xFF7FFFFF, so the sum cannot wrap in 32 bits.
        t = u >> np.uint32(16)
        t &= np.uint32(1)
        t += np.uint32(0x7FFF)
        u += t
        u >>= np.uint32(16)
        res[lo:lo + step] = u

    with concurrent.futures.ThreadPoolExecutor(max_workers=min(8, os.cpu_count() or 1)) as ex:
        list(ex.map(chunk, range(0, flat.size, step)))
    return res.reshape(x.shape)


def bf16_bits_to_f32(b: np.ndarray) -> np.ndarray:
    """Exact widening of bfloat16 bit patterns to float32."""
    b = np.ascontiguousarray(b, dtype=np.uint16)
    return (b.astype(np.uint32) << np.uint32(16)).view(np.float32)


def _unit_draw(seed: int, tensor: int, b: int, h: int, u: int, n: int, d: int) -> np.ndarray:
    ss = np.random.SeedSequence([seed, tensor, b, h, u])
    g = np.random.Generator(np.random.PCG64(ss))
    return g.standard_normal((n, d), dtype=np.float32)


def draw(seed: int, tensor: int, batch: int, heads: int, seq_len: int, head_dim: int,
         sigma: float = 1.0, dtype: str = "f32", positions: np.ndarray | None = None) -> np.ndarray:
    """Natural-order tensor ``[batch, heads, len(positions) or seq_len, head_dim]``.

    ``dtype="f32"`` gives float32 values; ``dtype="bf16"`` gives uint16 bf16
    bit patterns of the same draws rounded to nearest even.
    """
    if positions is None:
        out = np.empty((batch, heads, seq_len, head_dim), dtype=np.float32)
        jobs = [(b, h, u) for b in range(batch) for h in range(heads) for u in range(-(-seq_len // UNIT))]

        def fill(job):
            b, h, u = job
            lo = u * UNIT
            n = min(UNIT, seq_len - lo)
            out[b, h, lo:lo + n] = _unit_draw(seed, tensor, b, h, u, n, head_dim)

        with concurrent.futures.ThreadPoolExecutor(max_workers=min(8, os.cpu_count() or 1)) as ex:
            list(ex.map(fill, jobs))
        return _finish(out, sigma, dtype)
    positions = np.asarray(positions, dtype=np.int64)
    if positions.size and (positions.min() < 0 or positions.max() >= seq_len):
        raise ValueError("position out of range")
    out = np.empty((batch, heads, positions.size, head_dim), dtype=np.float32)
    units = positions // UNIT
    for b in range(batch):
        for h in range(heads):
            for u in np.unique(units):
                lo = int(u) * UNIT
                n = min(UNIT, seq_len - lo)
                vals = _unit_draw(seed, tensor, b, h, int(u), n, head_dim)
                sel = np.nonzero(units == u)[0]
                out[b, h, sel, :] = vals[positions[sel] - lo]
    return _finish(out, sigma, dtype)


def _finish(out: np.ndarray, sigma: float, dtype: str) -> np.ndarray:
    if sigma != 1.0:
        out *= np.float32(sigma)
    if dtype == "f32":
        return out
    if dtype == "bf16":
        return f32_to_bf16_bits(out)
    raise ValueError(f"unknown dtype {dtype}")


def draw_qkv(w: Workload, positions: np.ndarray | None = None):
    """Q, K, V of a workload in natural token order (Q restricted to ``positions``)."""
    q = draw(w.seed, TENSOR_Q, w.batch, w.h_q, w.seq_len, w.head_dim, w.sigma, w.dtype, positions)
    k = draw(w.seed, TENSOR_K, w.batch, w.h_kv, w.seq_len, w.head_dim, w.sigma, w.dtype)
    v = draw(w.seed, TENSOR_V, w.batch, w.h_kv, w.seq_len, w.head_dim, w.sigma, w.dtype)
    return q, k, v


def sample_rows(n_loc: int, chunk: int, n_random: int, seed: int) -> np.ndarray:
    """Shard-local row sample: first and last 4 rows of every chunk plus uniform draws."""
    rows = set()
    for start in range(0, n_loc, chunk):
        end = min(start + chunk, n_loc)
        rows.update(range(start, min(start + 4, end)))
        rows.update(range(max(end - 4, start), end))
    g = np.random.default_rng(seed)
    rows.update(int(x) for x in g.integers(0, n_loc, size=n_random))
    return np.array(sorted(rows), dtype=np.int64)
