"""Python binding of the MI355X ring-attention shard library.

Argument marshalling only: every function forwards to the C ABI declared in
``include/ring_attn.h`` (``libring_attn.so`` next to this file), passing
device pointers and the current HIP stream of PyTorch.  PyTorch supplies
device memory and streams; all computation runs in the library's HIP
kernels.  There is no fallback: if the library is missing, importing the
binding's functions raises.
"""
from __future__ import annotations

import ctypes
import os

SPLIT_CONTIGUOUS = 0
SPLIT_ZIGZAG = 1
SPLIT_STRIPED = 2
F32 = 0
BF16 = 1
FLAG_SYNC_LOADS = 1
FLAG_NATURAL_QO = 2
FLAG_EVENT_COUNTS = 4
STATS_EVENTS_LEN = 6
OK, EINVAL, EUNSUPPORTED, EHIP = 0, 1, 2, 3
MAX_BLOCKS = 128
NOALLOC_MAX_PARTIAL_FLOATS = 1 << 24  # static scratch of ring_attn_shard_fwd_split_noalloc
NOALLOC_MAX_LSE_FLOATS = 1 << 17
MAX_PARTS = 64

# RING_ATTN_LIB may name another build of the same library (tuning variants).
LIB_PATH = os.environ.get("RING_ATTN_LIB") or os.path.join(os.path.dirname(os.path.abspath(__file__)),
                                                           "libring_attn.so")

EXPORTS = ("zigzag_partition", "zigzag_unpartition", "ring_attn_shard_fwd", "ring_attn_tile_shape",
           "ring_attn_merge", "ring_attn_last_error", "ring_attn_abi_version", "ring_attn_all_shards_fwd",
           "ring_attn_shard_fwd_split_noalloc",
           "ring_attn_merge_strided", "ring_attn_decode", "ring_attn_shard_fwd_split")


class RingAttnError(RuntimeError):
    def __init__(self, status: int, message: str):
        super().__init__(f"[status {status}] {message}")
        self.status = status


class AttnDesc(ctypes.Structure):
    _fields_ = [
        ("seq_len", ctypes.c_int64),
        ("n_shards", ctypes.c_int32),
        ("split", ctypes.c_int32),
        ("batch", ctypes.c_int32),
        ("h_q", ctypes.c_int32),
        ("h_kv", ctypes.c_int32),
        ("head_dim", ctypes.c_int32),
        ("in_dtype", ctypes.c_int32),
        ("out_dtype", ctypes.c_int32),
        ("causal", ctypes.c_int32),
        ("scale", ctypes.c_float),
        ("flags", ctypes.c_uint32),
    ]


_lib = None


def lib():
    """The loaded C library (raises if it has not been built)."""
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(LIB_PATH):
        raise ImportError(f"{LIB_PATH} is missing: build it with __graft_entry__.build() "
                          "(hipcc for gfx950); there is no fallback")
    L = ctypes.CDLL(LIB_PATH)
    vp, i32, i64 = ctypes.c_void_p, ctypes.c_int32, ctypes.c_int64
    L.zigzag_partition.argtypes = [i64, i32, i32, vp, vp, vp, i64, i64, vp]
    L.zigzag_unpartition.argtypes = [i64, i32, i32, vp, vp, i64, i64, vp]
    L.ring_attn_shard_fwd.argtypes = [ctypes.POINTER(AttnDesc), i32, vp, i32, vp, vp, vp, vp, vp, vp, vp]
    L.ring_attn_tile_shape.argtypes = [ctypes.POINTER(AttnDesc), ctypes.POINTER(i32), ctypes.POINTER(i32)]
    L.ring_attn_merge.argtypes = [i32, i32, i64, i32, i32, vp, i32, vp, vp, i32, vp, vp]
    L.ring_attn_all_shards_fwd.argtypes = [ctypes.POINTER(AttnDesc), vp, vp, vp, vp, vp, vp, vp]
    L.ring_attn_shard_fwd_split_noalloc.argtypes = [ctypes.POINTER(AttnDesc), i32, vp, i32, vp, vp, vp, i32, vp, vp,
                                                    vp, vp]
    L.ring_attn_merge_strided.argtypes = [i32, i32, i64, i32, i32, vp, i64, i32, vp, i64, vp, i32, vp, vp]
    L.ring_attn_decode.argtypes = [ctypes.POINTER(AttnDesc), vp, i32, vp, vp, i32, vp, vp, vp]
    L.ring_attn_shard_fwd_split.argtypes = [ctypes.POINTER(AttnDesc), i32, vp, i32, vp, vp, vp, i32, vp, vp, vp,
                                            vp, vp, vp]
    for name in ("zigzag_partition", "zigzag_unpartition", "ring_attn_shard_fwd",
                 "ring_attn_tile_shape", "ring_attn_merge", "ring_attn_all_shards_fwd",
                 "ring_attn_merge_strided", "ring_attn_decode", "ring_attn_shard_fwd_split",
                 "ring_attn_shard_fwd_split_noalloc"):
        getattr(L, name).restype = i32
    L.ring_attn_last_error.restype = ctypes.c_char_p
    L.ring_attn_abi_version.restype = i32
    _lib = L
    return L


def _check(status: int):
    if status != OK:
        raise RingAttnError(status, lib().ring_attn_last_error().decode())


def _ptr(x):
    """Device pointer of a tensor, or an integer address, or None."""
    if x is None:
        return None
    if isinstance(x, int):
        return x
    return x.data_ptr()


def _stream(stream, *tensors):
    if stream is not None:
        return stream if isinstance(stream, int) else stream.cuda_stream
    import torch
    for t in tensors:
        if t is not None and not isinstance(t, int) and t.is_cuda:
            return torch.cuda.current_stream(t.device).cuda_stream
    return None


def abi_version() -> int:
    return int(lib().ring_attn_abi_version())


def make_desc(seq_len, n_shards, split, batch, h_q, h_kv, head_dim, in_dtype, out_dtype,
              causal=True, scale=None, flags=0) -> AttnDesc:
    if scale is None:
        scale = head_dim ** -0.5
    return AttnDesc(int(seq_len), int(n_shards), int(split), int(batch), int(h_q), int(h_kv),
                    int(head_dim), int(in_dtype), int(out_dtype), int(bool(causal)), float(scale),
                    int(flags))


def zigzag_partition(seq_len, n_shards, split, perm=None, src=None, dst=None, outer=0,
                     inner_bytes=0, stream=None):
    """Write shard placement ``perm`` and/or gather ``src`` rows into shard-major ``dst``."""
    _check(lib().zigzag_partition(int(seq_len), int(n_shards), int(split), _ptr(perm), _ptr(src),
                                  _ptr(dst), int(outer), int(inner_bytes),
                                  _stream(stream, perm, src, dst)))


def zigzag_unpartition(seq_len, n_shards, split, src, dst, outer, inner_bytes, stream=None):
    """Scatter shard-major ``src`` rows back to natural order in ``dst``."""
    _check(lib().zigzag_unpartition(int(seq_len), int(n_shards), int(split), _ptr(src), _ptr(dst),
                                    int(outer), int(inner_bytes), _stream(stream, src, dst)))


def ring_attn_tile_shape(desc: AttnDesc):
    tq, tk = ctypes.c_int32(), ctypes.c_int32()
    _check(lib().ring_attn_tile_shape(ctypes.byref(desc), ctypes.byref(tq), ctypes.byref(tk)))
    return tq.value, tk.value


def ring_attn_shard_fwd(desc: AttnDesc, rank, q, k_blocks, v_blocks, out, lse, block_owner=None,
                        stats=None, stream=None):
    """Shard ``rank``'s queries against the given key/value blocks (ring order by default)."""
    n = len(k_blocks)
    if len(v_blocks) != n:
        raise ValueError("k_blocks and v_blocks differ in length")
    kp = (ctypes.c_void_p * max(n, 1))(*[_ptr(t) for t in k_blocks])
    vp = (ctypes.c_void_p * max(n, 1))(*[_ptr(t) for t in v_blocks])
    owners = None
    if block_owner is not None:
        if len(block_owner) != n:
            raise ValueError("block_owner and k_blocks differ in length")
        owners = (ctypes.c_int32 * n)(*[int(x) for x in block_owner])
    _check(lib().ring_attn_shard_fwd(ctypes.byref(desc), int(rank), _ptr(q), n, owners, kp, vp,
                                     _ptr(out), _ptr(lse), _ptr(stats), _stream(stream, q, out)))


def ring_attn_all_shards_fwd(desc: AttnDesc, q_shards, k_blocks, v_blocks, out_shards, lse_shards, stats=None,
                             stream=None):
    """Every shard's ring pass at once: ``q_shards`` [c, B, h_q, S/c, d], block
    ``j`` of ``k_blocks`` / ``v_blocks`` = shard j's keys / values, results in
    ``out_shards`` [c, B, h_q, S/c, d] and ``lse_shards`` [c, B, h_q, S/c]."""
    n = len(k_blocks)
    if len(v_blocks) != n or n != desc.n_shards:
        raise ValueError("k_blocks and v_blocks must hold one block per shard")
    kp = (ctypes.c_void_p * n)(*[_ptr(t) for t in k_blocks])
    vp = (ctypes.c_void_p * n)(*[_ptr(t) for t in v_blocks])
    _check(lib().ring_attn_all_shards_fwd(ctypes.byref(desc), _ptr(q_shards), kp, vp, _ptr(out_shards),
                                          _ptr(lse_shards), _ptr(stats), _stream(stream, q_shards, out_shards)))


def ring_attn_shard_fwd_split(desc, rank, q, k_blocks, v_blocks, n_splits, work_out, work_lse, out, lse,
                              block_owner=None, stats=None, stream=None):
    """ring_attn_shard_fwd with the block list cut into ``n_splits`` concurrent
    groups (partials in the fp32 workspace ``work_out`` [n_splits, B, h_q, S/c, d]
    and ``work_lse`` [n_splits, B, h_q, S/c]), folded into ``out`` / ``lse``."""
    n = len(k_blocks)
    if len(v_blocks) != n:
        raise ValueError("k_blocks and v_blocks differ in length")
    kp = (ctypes.c_void_p * max(n, 1))(*[_ptr(t) for t in k_blocks])
    vp = (ctypes.c_void_p * max(n, 1))(*[_ptr(t) for t in v_blocks])
    owners = None
    if block_owner is not None:
        if len(block_owner) != n:
            raise ValueError("block_owner and k_blocks differ in length")
        owners = (ctypes.c_int32 * n)(*[int(x) for x in block_owner])
    _check(lib().ring_attn_shard_fwd_split(ctypes.byref(desc), int(rank), _ptr(q), n, owners, kp, vp, int(n_splits),
                                           _ptr(work_out), _ptr(work_lse), _ptr(out), _ptr(lse), _ptr(stats),
                                           _stream(stream, q, out)))


def ring_attn_shard_fwd_split_noalloc(desc, rank, q, k_blocks, v_blocks, n_splits, out, lse, block_owner=None,
                                      stats=None, stream=None):
    """ring_attn_shard_fwd_split with the partials in the library's static
    device scratch (no workspace, no allocation; overlapping calls on one GPU
    race)."""
    n = len(k_blocks)
    if len(v_blocks) != n:
        raise ValueError("k_blocks and v_blocks differ in length")
    kp = (ctypes.c_void_p * max(n, 1))(*[_ptr(t) for t in k_blocks])
    vp = (ctypes.c_void_p * max(n, 1))(*[_ptr(t) for t in v_blocks])
    owners = None
    if block_owner is not None:
        if len(block_owner) != n:
            raise ValueError("block_owner and k_blocks differ in length")
        owners = (ctypes.c_int32 * n)(*[int(x) for x in block_owner])
    _check(lib().ring_attn_shard_fwd_split_noalloc(ctypes.byref(desc), int(rank), _ptr(q), n, owners, kp, vp,
                                                   int(n_splits), _ptr(out), _ptr(lse), _ptr(stats),
                                                   _stream(stream, q, out)))


def ring_attn_merge(batch, heads, rows, head_dim, outs, parts_dtype, lses, out, out_dtype, lse,
                    stream=None):
    """Fold partial (out, lse) results; ``out``/``lse`` may be ``outs[0]``/``lses[0]``."""
    n = len(outs)
    if len(lses) != n:
        raise ValueError("outs and lses differ in length")
    op = (ctypes.c_void_p * max(n, 1))(*[_ptr(t) for t in outs])
    lp = (ctypes.c_void_p * max(n, 1))(*[_ptr(t) for t in lses])
    _check(lib().ring_attn_merge(int(batch), int(heads), int(rows), int(head_dim), n, op,
                                 int(parts_dtype), lp, _ptr(out), int(out_dtype), _ptr(lse),
                                 _stream(stream, out, lse)))


def ring_attn_merge_strided(batch, heads, rows, head_dim, outs, parts_dtype, lses, out, out_dtype, lse,
                            n_parts=None, out_stride=None, lse_stride=None, stream=None):
    """Fold the parts stacked along the first dimension of ``outs`` / ``lses``
    (strides default to one part's size); ``out``/``lse`` may be part 0."""
    n = int(outs.shape[0]) if n_parts is None else int(n_parts)
    os_ = batch * heads * rows * head_dim if out_stride is None else out_stride
    ls_ = batch * heads * rows if lse_stride is None else lse_stride
    _check(lib().ring_attn_merge_strided(int(batch), int(heads), int(rows), int(head_dim), n, _ptr(outs),
                                         int(os_), int(parts_dtype), _ptr(lses), int(ls_), _ptr(out),
                                         int(out_dtype), _ptr(lse), _stream(stream, out, lse)))


def ring_attn_decode(desc, q, k_blocks, v_blocks, n_splits, out_parts, lse_parts, stream=None):
    """Split-KV decode partials: one per (block, key range), at index block * n_splits + range."""
    n = len(k_blocks)
    if len(v_blocks) != n:
        raise ValueError("k_blocks and v_blocks differ in length")
    kp = (ctypes.c_void_p * max(n, 1))(*[_ptr(t) for t in k_blocks])
    vp = (ctypes.c_void_p * max(n, 1))(*[_ptr(t) for t in v_blocks])
    _check(lib().ring_attn_decode(ctypes.byref(desc), _ptr(q), n, kp, vp, int(n_splits), _ptr(out_parts),
                                  _ptr(lse_parts), _stream(stream, q, out_parts)))


def shard_tensor(x, n_shards, split, stream=None):
    """Gather a natural-order ``[B, H, S, d]`` device tensor into ``[c, B, H, S/c, d]``.

    Allocates the result with torch and fills it with one zigzag_partition call.
    """
    import torch
    B, H, S, d = x.shape
    out = torch.empty((n_shards, B, H, S // n_shards, d), dtype=x.dtype, device=x.device)
    zigzag_partition(S, n_shards, split, None, x, out, B * H, d * x.element_size(), stream)
    return out


def unshard_tensor(xs, seq_len, split, stream=None):
    """Scatter ``[c, B, H, S/c, d]`` shard tensors back to natural order ``[B, H, S, d]``."""
    import torch
    c, B, H, n_loc, d = xs.shape
    out = torch.empty((B, H, seq_len, d), dtype=xs.dtype, device=xs.device)
    zigzag_unpartition(seq_len, c, split, xs, out, B * H, d * xs.element_size(), stream)
    return out
