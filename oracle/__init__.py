"""fp64 CPU oracle for the ring-attention shard path.

TEST INFRASTRUCTURE ONLY: imported by ``tests/``, by ``__graft_entry__.smoke()``
and by the ``cpu_baseline`` leg of ``bench.py``, never by the product package.
It shares no code with the HIP library and never reads a value produced by it.

Contents (each is the plain definition from the pages, see the docstrings):

* :func:`attention` -- full (or key-restricted) softmax attention in fp64,
  via the C++ core in ``oracle.cpp`` (OpenMP over query rows).
* :func:`partition_perm` -- the token placement of each shard.
* :func:`pair_counts`, :func:`tile_counts` -- causal work per shard.
* :func:`merge` -- combining partial (out, lse) pairs.
* :func:`blockwise_online` -- the online-softmax recurrence over key blocks,
  used only to show that blockwise evaluation equals full attention.
"""
from __future__ import annotations

import ctypes
import math
import os
import subprocess

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SO = os.path.join(_HERE, "liboracle.so")
_SRC = os.path.join(_HERE, "oracle.cpp")

SPLIT_CONTIGUOUS = 0
SPLIT_ZIGZAG = 1
SPLIT_STRIPED = 2

_DT = {np.dtype(np.float32): 0, np.dtype(np.uint16): 1, np.dtype(np.float64): 2}


def build(out: str = _SO, src: str = _SRC, extra: tuple = ()) -> str:
    """Compile the C++ core with g++ (portable x86-64 code, OpenMP)."""
    cmd = ["g++", "-O2", "-std=c++17", "-fopenmp", "-shared", "-fPIC", *extra, "-o", out, src]
    subprocess.run(cmd, check=True)
    return out


_lib = None


def load_lib(path: str | None = None):
    global _lib
    if path is None and _lib is not None:
        return _lib
    so = path or _SO
    if not os.path.exists(so):
        build(so)
    lib = ctypes.CDLL(so)
    p = ctypes.c_void_p
    i64 = ctypes.c_int64
    lib.oracle_attention.argtypes = [p, p, p, ctypes.c_int, i64, i64, i64, i64, i64, i64,
                                     p, ctypes.c_double, ctypes.c_int, p, i64, p, i64, p, i64, p, p]
    lib.oracle_attention.restype = ctypes.c_int
    lib.oracle_threads.restype = ctypes.c_int
    if path is None:
        _lib = lib
    return lib


def threads() -> int:
    return int(load_lib().oracle_threads())


def _ptr(a):
    return None if a is None else a.ctypes.data_as(ctypes.c_void_p)


def attention(q, k, v, scale, causal, q_pos=None, rows=None, heads=None, keys=None, lib=None):
    """Softmax attention in fp64 (the plain definition).

    q: [B, Hq, Sq, d]; k, v: [B, Hkv, S, d] in natural token order, all of one
    dtype: float32, float64, or uint16 holding bf16 bits (widened exactly).
    q_pos: global position of each q row (default: 0..Sq-1).  rows / heads
    select which q rows / query heads to evaluate; keys restricts the key
    positions (one ring block's keys -> that block's partial result).

    Query head h reads key/value head h // (Hq // Hkv); with ``causal`` a
    query at position i sees key positions j <= i.  Returns (out, lse):
    out [B, n_heads, n_rows, d], lse [B, n_heads, n_rows] (natural log of the
    sum of exp(scaled score)); a row with no visible key gives (0, -inf).
    """
    q = np.ascontiguousarray(q)
    k = np.ascontiguousarray(k)
    v = np.ascontiguousarray(v)
    if not (q.dtype == k.dtype == v.dtype) or q.dtype not in _DT:
        raise TypeError("q, k, v must share one dtype: float32, float64 or uint16 (bf16 bits)")
    B, Hq, Sq, d = q.shape
    _, Hkv, S, _ = k.shape
    if q_pos is None:
        q_pos = np.arange(Sq, dtype=np.int64)
    q_pos = np.ascontiguousarray(q_pos, dtype=np.int64)
    rows = None if rows is None else np.ascontiguousarray(rows, dtype=np.int64)
    heads = None if heads is None else np.ascontiguousarray(heads, dtype=np.int64)
    keys = None if keys is None else np.ascontiguousarray(keys, dtype=np.int64)
    n_rows = Sq if rows is None else rows.size
    n_heads = Hq if heads is None else heads.size
    out = np.empty((B, n_heads, n_rows, d), dtype=np.float64)
    lse = np.empty((B, n_heads, n_rows), dtype=np.float64)
    lib = lib or load_lib()
    rc = lib.oracle_attention(_ptr(q), _ptr(k), _ptr(v), _DT[q.dtype], B, Hq, Hkv, Sq, S, d,
                              _ptr(q_pos), float(scale), int(bool(causal)),
                              _ptr(rows), 0 if rows is None else rows.size,
                              _ptr(heads), 0 if heads is None else heads.size,
                              _ptr(keys), 0 if keys is None else keys.size,
                              _ptr(out), _ptr(lse))
    if rc != 0:
        raise ValueError("oracle_attention: invalid sizes")
    return out, lse


# ---------------------------------------------------------------------------
# Token placement.  Contiguous: device k holds the k-th run of S/c tokens
# ("Sequence / context parallelism" notes, section 1 diagram).  Zig-zag: the
# sequence is cut into 2c chunks and device k holds chunks k and 2c-1-k
# ("Splitting the Sequence", second intro paragraph and Terms).  Within a
# shard the tokens are kept in ascending position (chunk k first).  Striped:
# tokens are dealt round-robin, device k holding positions k, k+c, k+2c, ...
# (notes, section 5 "Striped / zigzag attention": an interleaved pattern).
# ---------------------------------------------------------------------------

def partition_perm(seq_len: int, n_shards: int, split: int) -> np.ndarray:
    """perm[r*(S/c) + t] = global position of shard r's t-th token (int64[S])."""
    S, c = int(seq_len), int(n_shards)
    if c < 1 or S < 1:
        raise ValueError("need S >= 1 and c >= 1")
    if split == SPLIT_ZIGZAG:
        if S % (2 * c):
            raise ValueError("zig-zag needs S divisible by 2c")
        n = S // (2 * c)
        out = []
        for r in range(c):
            out.extend(range(r * n, (r + 1) * n))
            out.extend(range((2 * c - 1 - r) * n, (2 * c - r) * n))
        return np.array(out, dtype=np.int64)
    if S % c:
        raise ValueError("S must be divisible by c")
    n_loc = S // c
    if split == SPLIT_CONTIGUOUS:
        return np.arange(S, dtype=np.int64)
    if split == SPLIT_STRIPED:
        return np.array([t * c + r for r in range(c) for t in range(n_loc)], dtype=np.int64)
    raise ValueError("unknown split")


def shard_positions(seq_len: int, n_shards: int, split: int, rank: int) -> np.ndarray:
    n_loc = seq_len // n_shards
    return partition_perm(seq_len, n_shards, split)[rank * n_loc:(rank + 1) * n_loc]


# ---------------------------------------------------------------------------
# Work accounting.  Under the causal mask a query at position i sees i+1 keys
# ("Sequence Parallelism and Ring Attention Quiz", Q6 and Q8: the later a
# token stands, the more keys it sees), so the work of a shard is the number of visible
# (query, key) pairs of its tokens ("Splitting the Sequence", "One sequence,
# sixteen devices": busiest device versus the average).
# ---------------------------------------------------------------------------

def pair_counts(seq_len: int, n_shards: int, split: int, causal: bool = True) -> np.ndarray:
    """Visible (query, key) pairs per shard, per query head (int64[c])."""
    perm = partition_perm(seq_len, n_shards, split)
    n_loc = seq_len // n_shards
    if not causal:
        return np.full(n_shards, n_loc * seq_len, dtype=np.int64)
    return (perm + 1).reshape(n_shards, n_loc).sum(axis=1).astype(np.int64)


def pair_counts_brute(seq_len: int, n_shards: int, split: int, causal: bool = True) -> list:
    """Same as :func:`pair_counts`, by enumerating every (query, key) pair."""
    perm = partition_perm(seq_len, n_shards, split)
    n_loc = seq_len // n_shards
    res = []
    for r in range(n_shards):
        cnt = 0
        for t in range(n_loc):
            i = int(perm[r * n_loc + t])
            for j in range(seq_len):
                if (not causal) or j <= i:
                    cnt += 1
        res.append(cnt)
    return res


def block_pair_counts(seq_len: int, n_shards: int, split: int, causal: bool = True) -> np.ndarray:
    """Per shard, the number of ring blocks holding at least one visible key."""
    perm = partition_perm(seq_len, n_shards, split)
    n_loc = seq_len // n_shards
    res = np.zeros(n_shards, dtype=np.int64)
    for r in range(n_shards):
        qmax = perm[r * n_loc:(r + 1) * n_loc].max()
        for j in range(n_shards):
            kmin = perm[j * n_loc:(j + 1) * n_loc].min()
            if (not causal) or kmin <= qmax:
                res[r] += 1
    return res


def tile_counts(seq_len: int, n_shards: int, split: int, causal: bool, rank: int,
                tile_q: int, tile_k: int, owners=None) -> dict:
    """Classify every (query tile, key tile) of one shard's pass.

    Query tiles are runs of ``tile_q`` shard-local rows, key tiles runs of
    ``tile_k`` local keys of each visited block.  A tile's nominal area is
    tile_q x tile_k; rows or keys past the shard end count as not visible.
    full: every nominal pair visible; skipped: none; partial: the rest.
    Returns dict(pairs, full, partial, skipped) summed over the visited blocks.
    """
    perm = partition_perm(seq_len, n_shards, split)
    n_loc = seq_len // n_shards
    if owners is None:
        owners = [(rank - t) % n_shards for t in range(n_shards)]
    qpos = perm[rank * n_loc:(rank + 1) * n_loc]
    nqt = -(-n_loc // tile_q)
    nkt = -(-n_loc // tile_k)
    pad_q = np.full(nqt * tile_q, -1, dtype=np.int64)
    pad_q[:n_loc] = qpos
    res = dict(pairs=0, full=0, partial=0, skipped=0)
    for j in owners:
        kpos = np.full(nkt * tile_k, np.iinfo(np.int64).max, dtype=np.int64)
        kpos[:n_loc] = perm[j * n_loc:(j + 1) * n_loc]
        qv = pad_q[:, None]
        kv = kpos[None, :]
        valid = (qv >= 0) & (kv != np.iinfo(np.int64).max)
        vis = valid & ((kv <= qv) if causal else True)
        for a in range(nqt):
            for b in range(nkt):
                cnt = int(vis[a * tile_q:(a + 1) * tile_q, b * tile_k:(b + 1) * tile_k].sum())
                res["pairs"] += cnt
                if cnt == tile_q * tile_k:
                    res["full"] += 1
                elif cnt == 0:
                    res["skipped"] += 1
                else:
                    res["partial"] += 1
    return res


# ---------------------------------------------------------------------------
# Combining partial results.  A partial (out_k, lse_k) is attention over a
# subset of keys; the full result over the union is the softmax-weighted mix
# of the parts: LSE = log sum_k exp(lse_k), out = sum_k exp(lse_k - LSE) out_k.
# This is the fold ring attention applies at every step ("Sequence / context
# parallelism" notes, section 4; "Splitting the Sequence", intro: results
# combined with the online softmax).  Parts with lse = -inf carry no keys.
# ---------------------------------------------------------------------------

def merge(outs, lses):
    """fp64 merge of partial results: outs [n, ..., d], lses [n, ...]."""
    outs = np.asarray(outs, dtype=np.float64)
    lses = np.asarray(lses, dtype=np.float64)
    m = lses.max(axis=0)
    m_safe = np.where(np.isneginf(m), 0.0, m)
    w = np.exp(lses - m_safe[None])          # exp(-inf) = 0 for empty parts
    z = w.sum(axis=0)
    with np.errstate(divide="ignore", invalid="ignore"):
        lse = np.where(z > 0, m_safe + np.log(z), -np.inf)
        out = np.where((z > 0)[..., None], (w[..., None] * outs).sum(axis=0) / z[..., None], 0.0)
    return out, lse


# ---------------------------------------------------------------------------
# Online softmax over key blocks (running max m, normaliser l, output
# rescaled when the max rises): the per-step update of the ring loop
# ("Sequence / context parallelism" notes, section 4; quiz Q3 and Q7).  The
# equations themselves are not printed on the pages; this follows the
# published online-normaliser recurrence of Milakov and Gimelshein (2018),
# extended with the output accumulator.  Used only for invariant tests.
# ---------------------------------------------------------------------------

def blockwise_online(q, k, v, scale, causal, q_pos, block_keys):
    """q [Sq, d], k/v [S, d] float64; block_keys: list of key-position arrays
    visited in order.  Returns (out [Sq, d], lse [Sq])."""
    q = np.asarray(q, dtype=np.float64)
    k = np.asarray(k, dtype=np.float64)
    v = np.asarray(v, dtype=np.float64)
    Sq, d = q.shape
    out = np.zeros((Sq, d))
    lse = np.empty(Sq)
    for i in range(Sq):
        m = -math.inf
        l = 0.0
        o = np.zeros(d)
        for keys in block_keys:
            keys = np.asarray(keys, dtype=np.int64)
            if causal:
                keys = keys[keys <= q_pos[i]]
            if keys.size == 0:
                continue
            s = scale * (k[keys] @ q[i])
            m_new = max(m, float(s.max()))
            alpha = math.exp(m - m_new) if m != -math.inf else 0.0
            p = np.exp(s - m_new)
            l = alpha * l + p.sum()
            o = alpha * o + p @ v[keys]
            m = m_new
        if l == 0.0:
            out[i] = 0.0
            lse[i] = -math.inf
        else:
            out[i] = o / l
            lse[i] = m + math.log(l)
    return out, lse


def widen(a: np.ndarray, dtype: str) -> np.ndarray:
    """Stored input values as float64 (bf16 bits are widened exactly)."""
    if dtype == "bf16":
        return (np.asarray(a, dtype=np.uint16).astype(np.uint32) << np.uint32(16)).view(np.float32).astype(np.float64)
    return np.asarray(a).astype(np.float64)
