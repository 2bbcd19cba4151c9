"""Pins of the fp64 oracle against facts that do not come from the oracle.

Each ``pin_*`` function takes the oracle's compiled core (a ctypes library,
so the same checks can run against deliberately broken builds) and raises
AssertionError when the oracle disagrees with:

* a pure-Python brute force on tiny inputs (``oracle/tiny.py``),
* closed forms of special inputs,
* PyTorch's CPU fp64 scaled-dot-product attention (an independent library),
* the invariant that attention over a union of key blocks equals the
  online-softmax / merge fold of the blocks' partial results.
"""
from __future__ import annotations

import math

import numpy as np

import oracle
from oracle import tiny


def _rng(seed):
    return np.random.default_rng(seed)


def pin_tiny_bruteforce(lib, seeds=(0, 1, 2), tol=1e-13):
    for seed in seeds:
        for (B, Hq, Hkv, S, d, causal) in [(1, 2, 1, 7, 4, True), (2, 4, 2, 16, 8, False),
                                          (1, 3, 3, 11, 5, True), (1, 4, 1, 16, 8, True)]:
            g = _rng(100 + seed)
            q = g.standard_normal((B, Hq, S, d))
            k = g.standard_normal((B, Hkv, S, d))
            v = g.standard_normal((B, Hkv, S, d))
            scale = 1.0 / math.sqrt(d)
            out, lse = oracle.attention(q, k, v, scale, causal, lib=lib)
            t_out, t_lse = tiny.attention(q.tolist(), k.tolist(), v.tolist(), scale, causal)
            assert np.max(np.abs(out - np.array(t_out))) <= tol, "out vs brute force"
            assert np.max(np.abs(lse - np.array(t_lse))) <= tol, "lse vs brute force"


def pin_closed_forms(lib):
    g = _rng(7)
    d = 8
    # S = 1: the only key gets weight 1.
    q = g.standard_normal((1, 1, 1, d)); k = g.standard_normal((1, 1, 1, d)); v = g.standard_normal((1, 1, 1, d))
    out, lse = oracle.attention(q, k, v, 0.3, True, lib=lib)
    assert np.allclose(out[0, 0, 0], v[0, 0, 0], rtol=0, atol=1e-15)
    assert abs(lse[0, 0, 0] - 0.3 * float(q[0, 0, 0] @ k[0, 0, 0])) <= 1e-14
    # q = 0: every visible key gets equal weight.
    S = 37
    q = np.zeros((1, 2, S, d)); k = g.standard_normal((1, 1, S, d)); v = g.standard_normal((1, 1, S, d))
    out, lse = oracle.attention(q, k, v, 0.125, True, lib=lib)
    for i in range(S):
        assert np.max(np.abs(out[0, 1, i] - v[0, 0, :i + 1].mean(axis=0))) <= 1e-14
        assert abs(lse[0, 1, i] - math.log(i + 1)) <= 1e-14
    out, lse = oracle.attention(q, k, v, 0.125, False, lib=lib)
    assert np.max(np.abs(out[0, 0] - v[0, 0].mean(axis=0)[None])) <= 1e-14
    assert np.max(np.abs(lse - math.log(S))) <= 1e-14
    # One key scoring 50 above the others takes (almost) all the weight.
    S = 9
    q = np.zeros((1, 1, S, d)); q[0, 0, :, 0] = 1.0
    k = np.zeros((1, 1, S, d)); k[0, 0, 3, 0] = 50.0
    v = g.standard_normal((1, 1, S, d))
    out, lse = oracle.attention(q, k, v, 1.0, False, lib=lib)
    assert np.max(np.abs(out[0, 0, :] - v[0, 0, 3][None])) <= 1e-19 + 1e-15 * np.abs(v).max() * 9
    assert np.max(np.abs(lse[0, 0] - (50.0 + math.log(1 + 8 * math.exp(-50.0))))) <= 1e-13
    # A row that sees no key (key set restricted to later positions): (0, -inf).
    q = g.standard_normal((1, 1, 4, d)); k = g.standard_normal((1, 1, 8, d)); v = g.standard_normal((1, 1, 8, d))
    out, lse = oracle.attention(q, k, v, 1.0, True, keys=np.arange(4, 8), lib=lib)
    assert np.all(out == 0.0) and np.all(np.isneginf(lse))


def pin_torch_sdpa(lib, shapes=((1, 4, 1, 256, 64), (1, 8, 2, 192, 128), (2, 6, 3, 96, 32))):
    import torch
    import torch.nn.functional as F
    for idx, (B, Hq, Hkv, S, d) in enumerate(shapes):
        g = _rng(20 + idx)
        q = g.standard_normal((B, Hq, S, d)); k = g.standard_normal((B, Hkv, S, d)); v = g.standard_normal((B, Hkv, S, d))
        scale = 1.0 / math.sqrt(d)
        for causal in (True, False):
            out, lse = oracle.attention(q, k, v, scale, causal, lib=lib)
            tq = torch.from_numpy(q)
            tk = torch.from_numpy(k).repeat_interleave(Hq // Hkv, dim=1)
            tv = torch.from_numpy(v).repeat_interleave(Hq // Hkv, dim=1)
            ref = F.scaled_dot_product_attention(tq, tk, tv, is_causal=causal, scale=scale)
            s = (tq @ tk.transpose(-1, -2)) * scale
            if causal:
                s = s.masked_fill(torch.ones(S, S, dtype=torch.bool).triu(1), float("-inf"))
            ref_lse = torch.logsumexp(s, dim=-1)
            assert np.max(np.abs(out - ref.numpy())) <= 1e-12, "out vs torch sdpa"
            assert np.max(np.abs(lse - ref_lse.numpy())) <= 1e-12, "lse vs torch logsumexp"


def pin_partial_merge(lib, S=96, c=4, seed=5):
    """Partials over ring blocks merge to the full result; blockwise online too."""
    g = _rng(seed)
    B, Hq, Hkv, d = 1, 4, 2, 16
    q = g.standard_normal((B, Hq, S, d)); k = g.standard_normal((B, Hkv, S, d)); v = g.standard_normal((B, Hkv, S, d))
    scale = 0.25
    for split in (oracle.SPLIT_CONTIGUOUS, oracle.SPLIT_ZIGZAG, oracle.SPLIT_STRIPED):
        perm = oracle.partition_perm(S, c, split)
        n_loc = S // c
        for causal in (True, False):
            full_o, full_l = oracle.attention(q, k, v, scale, causal, lib=lib)
            outs, lses = [], []
            for j in range(c):
                o, l = oracle.attention(q, k, v, scale, causal, keys=perm[j * n_loc:(j + 1) * n_loc], lib=lib)
                outs.append(o); lses.append(l)
            mo, ml = oracle.merge(outs, lses)
            assert np.max(np.abs(mo - full_o)) <= 1e-12, "merged partials vs full"
            assert np.max(np.abs(ml - full_l)) <= 1e-12, "merged lse vs full"
            # Merge is order-free: reversed and pairwise-tree folds agree.
            ro, rl = oracle.merge(outs[::-1], lses[::-1])
            ao, al = oracle.merge([oracle.merge(outs[:2], lses[:2])[0], oracle.merge(outs[2:], lses[2:])[0]],
                                  [oracle.merge(outs[:2], lses[:2])[1], oracle.merge(outs[2:], lses[2:])[1]])
            assert np.max(np.abs(ro - mo)) <= 1e-12 and np.max(np.abs(ao - mo)) <= 1e-12
            assert np.max(np.abs(rl - ml)) <= 1e-12 and np.max(np.abs(al - ml)) <= 1e-12
            # The online-softmax recurrence over ring-ordered blocks, for the
            # queries of shard r, equals full attention (any visit order).
            for r in (0, c - 1):
                rows = perm[r * n_loc:(r + 1) * n_loc]
                blocks = [perm[((r - t) % c) * n_loc:(((r - t) % c) + 1) * n_loc] for t in range(c)]
                for order in (blocks, blocks[::-1]):
                    bo, bl = oracle.blockwise_online(q[0, 1][rows], k[0, 0], v[0, 0], scale, causal, rows, order)
                    assert np.max(np.abs(bo - full_o[0, 1][rows])) <= 1e-12
                    assert np.max(np.abs(bl - full_l[0, 1][rows])) <= 1e-12


def pin_restricted_keys_subarray(lib, seed=9):
    """Restricting keys to a set equals attention over that sub-array of keys."""
    g = _rng(seed)
    S, d = 40, 8
    q = g.standard_normal((1, 2, S, d)); k = g.standard_normal((1, 1, S, d)); v = g.standard_normal((1, 1, S, d))
    keys = np.array([3, 5, 6, 17, 30, 31, 39])
    o, l = oracle.attention(q, k, v, 0.5, False, keys=keys, lib=lib)
    o2, l2 = oracle.attention(q, np.ascontiguousarray(k[:, :, keys]), np.ascontiguousarray(v[:, :, keys]), 0.5, False, lib=lib)
    assert np.max(np.abs(o - o2)) <= 1e-14 and np.max(np.abs(l - l2)) <= 1e-14


def pin_rows_heads_positions(lib, seed=11):
    """Row / head selection and explicit q positions pick the same numbers."""
    g = _rng(seed)
    S, d = 32, 8
    q = g.standard_normal((1, 4, S, d)); k = g.standard_normal((1, 2, S, d)); v = g.standard_normal((1, 2, S, d))
    full_o, full_l = oracle.attention(q, k, v, 0.5, True, lib=lib)
    perm = oracle.partition_perm(S, 2, oracle.SPLIT_ZIGZAG)
    rows = np.array([0, 5, 9, 15])
    o, l = oracle.attention(np.ascontiguousarray(q[:, :, perm]), k, v, 0.5, True, q_pos=perm, rows=rows,
                           heads=np.array([3, 1]), lib=lib)
    assert np.array_equal(o[0, 0], full_o[0, 3][perm[rows]]) and np.array_equal(o[0, 1], full_o[0, 1][perm[rows]])
    assert np.array_equal(l[0, 0], full_l[0, 3][perm[rows]])


def pin_dtypes(lib, seed=13):
    """bf16 and fp32 inputs are widened exactly: same result as fp64 of the values."""
    import workloads
    g = _rng(seed)
    x = g.standard_normal((3, 1, 2, 24, 8)).astype(np.float32)
    bf = workloads.f32_to_bf16_bits(x)
    for arr, dt in ((x, "f32"), (bf, "bf16")):
        o, l = oracle.attention(arr[0], arr[1][:, :1], arr[2][:, :1], 0.3, True, lib=lib)
        w = oracle.widen(arr, dt)
        o2, l2 = oracle.attention(w[0], w[1][:, :1], w[2][:, :1], 0.3, True, lib=lib)
        assert np.array_equal(o, o2) and np.array_equal(l, l2)


ALL_PINS = [pin_tiny_bruteforce, pin_closed_forms, pin_torch_sdpa, pin_partial_merge,
            pin_restricted_keys_subarray, pin_rows_heads_positions, pin_dtypes]
