"""Helpers for the GPU parity tests: seeded problems on the device, shard
passes through the C ABI, and comparisons against the fp64 oracle."""
from __future__ import annotations

import sys

import numpy as np
import torch

import oracle
import ring_parallelism_amd as ra
import workloads

DEV = torch.device("cuda:0")
SPLITS = {ra.SPLIT_CONTIGUOUS: "contiguous", ra.SPLIT_ZIGZAG: "zigzag", ra.SPLIT_STRIPED: "striped"}

# Tolerances against the fp64 oracle.  fp32 path: 1e-5 on out and lse.  bf16
# inputs: max |err| <= 1e-2 and mean |err| <= 1e-3 on out, 1e-3 on lse.
TOL = {"f32": (1e-5, 1e-5, 1e-5), "bf16": (1e-2, 1e-3, 1e-3)}


def say(msg):
    print(msg, flush=True)
    sys.stdout.flush()


def up(arr, dtype):
    arr = np.ascontiguousarray(arr)
    if dtype == "bf16":
        return torch.from_numpy(arr.view(np.int16)).view(torch.bfloat16).to(DEV)
    return torch.from_numpy(arr).to(DEV)


class Problem:
    """Natural-order host Q/K/V plus their device shards ``[c, B, H, S/c, d]``."""

    def __init__(self, S, c, split, B, Hq, Hkv, d, dtype, sigma=1.0, seed=0, q_positions=None, arrays=None):
        self.S, self.c, self.split, self.B, self.Hq, self.Hkv, self.d = S, c, split, B, Hq, Hkv, d
        self.dtype, self.n_loc, self.scale = dtype, S // c, d ** -0.5
        if arrays is None:
            self.q = workloads.draw(seed, workloads.TENSOR_Q, B, Hq, S, d, sigma, dtype)
            self.k = workloads.draw(seed, workloads.TENSOR_K, B, Hkv, S, d, sigma, dtype)
            self.v = workloads.draw(seed, workloads.TENSOR_V, B, Hkv, S, d, sigma, dtype)
        else:
            # Given natural-order fp32 values, quantised like the workloads' draws.
            conv = workloads.f32_to_bf16_bits if dtype == "bf16" else (lambda a: np.ascontiguousarray(a, np.float32))
            self.q, self.k, self.v = (conv(a) for a in arrays)
        self.perm = oracle.partition_perm(S, c, split)
        self.qs = ra.shard_tensor(up(self.q, dtype), c, split)
        self.ks = ra.shard_tensor(up(self.k, dtype), c, split)
        self.vs = ra.shard_tensor(up(self.v, dtype), c, split)
        torch.cuda.synchronize()

    @classmethod
    def from_workload(cls, w):
        return cls(w.seq_len, w.n_shards, w.split, w.batch, w.h_q, w.h_kv, w.head_dim, w.dtype, w.sigma, w.seed)

    def desc(self, out_dtype=ra.F32, causal=True, flags=0):
        in_dt = ra.BF16 if self.dtype == "bf16" else ra.F32
        return ra.make_desc(self.S, self.c, self.split, self.B, self.Hq, self.Hkv, self.d, in_dt,
                            out_dtype, causal, self.scale, flags)

    def ring_owners(self, rank):
        return [(rank - t) % self.c for t in range(self.c)]

    def run(self, rank, out_dtype=ra.F32, causal=True, owners=None, with_stats=True, fill=float("nan"), flags=0):
        owners = self.ring_owners(rank) if owners is None else list(owners)
        odt = torch.float32 if out_dtype == ra.F32 else torch.bfloat16
        out = torch.full((self.B, self.Hq, self.n_loc, self.d), fill, dtype=odt, device=DEV)
        lse = torch.full((self.B, self.Hq, self.n_loc), fill, dtype=torch.float32, device=DEV)
        n_stats = ra.STATS_EVENTS_LEN if flags & ra.FLAG_EVENT_COUNTS else 4
        stats = torch.zeros(n_stats, dtype=torch.int64, device=DEV) if with_stats else None
        ra.ring_attn_shard_fwd(self.desc(out_dtype, causal, flags), rank, self.qs[rank],
                               [self.ks[j] for j in owners], [self.vs[j] for j in owners],
                               out, lse, block_owner=owners, stats=stats)
        torch.cuda.synchronize()
        return out, lse, stats

    def reference(self, rank, rows=None, heads=None, causal=True, owners=None):
        """Oracle (out, lse) for shard-local ``rows`` of ``rank``: [B, nh, nr, d], [B, nh, nr]."""
        if rows is None:
            rows = np.arange(self.n_loc)
        pos = self.perm[rank * self.n_loc + np.asarray(rows)]
        keys = None
        if owners is not None:
            keys = np.sort(np.concatenate([self.perm[j * self.n_loc:(j + 1) * self.n_loc] for j in owners]))
        return oracle.attention(self.q, self.k, self.v, self.scale, causal, rows=pos, heads=heads, keys=keys)


def compare(out, lse, ref_o, ref_l, rows=None, heads=None, tol=(1e-2, 1e-3, 1e-3), bf16_out=False):
    """Element-by-element comparison on the selected rows / heads; returns (max, mean, lse max)."""
    o = out.float().cpu().numpy()
    l = lse.cpu().numpy()
    if heads is not None:
        o, l = o[:, heads], l[:, heads]
    if rows is not None:
        o, l = o[:, :, rows], l[:, :, rows]
    assert o.shape == ref_o.shape, (o.shape, ref_o.shape)
    assert np.all(np.isfinite(o)), "non-finite output"
    err = np.abs(o - ref_o)
    tol_max, tol_mean, tol_lse = tol
    if bf16_out:
        # bf16 output adds one rounding of at most half a bf16 ulp of the value.
        allow = tol_max + np.abs(ref_o) * 2.0 ** -8
        assert np.all(err <= allow), f"max out err {err.max():.3e} beyond bf16-output bound"
        over = int((err > tol_max).sum())
        if over:
            say(f"  bf16 output: {over} of {err.size} elements use the half-ulp allowance "
                f"(max |ref| among them {np.abs(ref_o)[err > tol_max].max():.2f})")
    else:
        assert err.max() <= tol_max, f"max out err {err.max():.3e} > {tol_max}"
    assert err.mean() <= tol_mean, f"mean out err {err.mean():.3e} > {tol_mean}"
    inf_ref = np.isneginf(ref_l)
    assert np.array_equal(np.isneginf(l), inf_ref), "lse -inf pattern differs"
    lerr = np.abs(l[~inf_ref] - ref_l[~inf_ref]) if (~inf_ref).any() else np.zeros(1)
    assert lerr.max() <= tol_lse, f"max lse err {lerr.max():.3e} > {tol_lse}"
    if inf_ref.any():
        assert np.all(o[np.broadcast_to(inf_ref[..., None], o.shape)] == 0.0), "empty rows must give out = 0"
    return float(err.max()), float(err.mean()), float(lerr.max())


def expected_stats(p: Problem, rank, tile_q, tile_k, causal=True, owners=None):
    owners = p.ring_owners(rank) if owners is None else owners
    t = oracle.tile_counts(p.S, p.c, p.split, causal, rank, tile_q, tile_k, owners)
    f = p.B * p.Hq
    return [t["pairs"] * f, t["full"] * f, t["partial"] * f, t["skipped"] * f]
