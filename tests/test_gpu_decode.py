"""Split-KV decode through the C ABI against the fp64 oracle: every partial
(one per block and key range) against attention over that range's keys alone,
and the merged result against attention over the whole cache (a query token
placed after every cached key)."""
import numpy as np
import pytest
import torch

import oracle
import ring_parallelism_amd as ra
import workloads
from gpu_util import DEV, TOL, compare, say, up

pytestmark = pytest.mark.gpu


class Decode:
    def __init__(self, S, c, split, B, Hq, Hkv, d, seed, sigma=1.0):
        self.S, self.c, self.split, self.B, self.Hq, self.Hkv, self.d = S, c, split, B, Hq, Hkv, d
        self.n, self.scale = S // c, d ** -0.5
        self.k = workloads.draw(seed, workloads.TENSOR_K, B, Hkv, S, d, sigma, "bf16")
        self.v = workloads.draw(seed, workloads.TENSOR_V, B, Hkv, S, d, sigma, "bf16")
        # The new token sits at position S, after every cached key.
        self.q = workloads.draw(seed, workloads.TENSOR_Q, B, Hq, S + 1, d, sigma, "bf16", positions=np.array([S]))
        self.perm = oracle.partition_perm(S, c, split)
        self.ks = ra.shard_tensor(up(self.k, "bf16"), c, split)
        self.vs = ra.shard_tensor(up(self.v, "bf16"), c, split)
        self.qd = up(np.ascontiguousarray(self.q[:, :, 0]), "bf16")  # [B, Hq, d]

    def desc(self):
        return ra.make_desc(self.S, self.c, self.split, self.B, self.Hq, self.Hkv, self.d, ra.BF16, ra.F32,
                            True, self.scale)

    def run(self, blocks, n_splits):
        n_parts = len(blocks) * n_splits
        outs = torch.full((n_parts, self.B, self.Hq, self.d), float("nan"), dtype=torch.float32, device=DEV)
        lses = torch.full((n_parts, self.B, self.Hq), float("nan"), dtype=torch.float32, device=DEV)
        ra.ring_attn_decode(self.desc(), self.qd, [self.ks[t] for t in blocks], [self.vs[t] for t in blocks],
                            n_splits, outs, lses)
        torch.cuda.synchronize()
        return outs, lses

    def merged(self, outs, lses):
        out = torch.empty((self.B, self.Hq, self.d), dtype=torch.float32, device=DEV)
        lse = torch.empty((self.B, self.Hq), dtype=torch.float32, device=DEV)
        ra.ring_attn_merge_strided(self.B, self.Hq, 1, self.d, outs, ra.F32, lses, out, ra.F32, lse)
        torch.cuda.synchronize()
        return out, lse

    def ref(self, keys=None, heads=None):
        return oracle.attention(self.q, self.k, self.v, self.scale, True, q_pos=np.array([self.S]), keys=keys,
                                heads=heads)

    def range_keys(self, t, s, n_splits):
        k0, k1 = s * self.n // n_splits, (s + 1) * self.n // n_splits
        return self.perm[t * self.n + k0: t * self.n + k1]


def check_parts(p, blocks, n_splits, outs, lses):
    for ti, t in enumerate(blocks):
        for s in range(n_splits):
            ref_o, ref_l = p.ref(keys=p.range_keys(t, s, n_splits))
            part = ti * n_splits + s
            compare(outs[part][:, :, None], lses[part][:, :, None], ref_o, ref_l, tol=TOL["bf16"])


@pytest.mark.parametrize("S,c,split,B,Hq,Hkv,d,n_splits", [
    (4096, 4, ra.SPLIT_ZIGZAG, 2, 8, 2, 128, 3),       # ragged ranges (341/341/342 keys)
    (4096, 4, ra.SPLIT_CONTIGUOUS, 1, 32, 1, 128, 1),  # a full group of 32 heads, one range per block
    (2048, 2, ra.SPLIT_STRIPED, 2, 4, 4, 64, 5),       # one head per kv head, d = 64
    (1024, 4, ra.SPLIT_ZIGZAG, 1, 16, 2, 128, 256),    # one key per range
])
def test_decode_parts_and_merge(S, c, split, B, Hq, Hkv, d, n_splits):
    p = Decode(S, c, split, B, Hq, Hkv, d, seed=31)
    blocks = list(range(c))
    say(f"decode S={S} c={c} split={split} {Hq}x{Hkv} d={d} splits={n_splits}")
    outs, lses = p.run(blocks, n_splits)
    if n_splits <= 5:
        check_parts(p, blocks, n_splits, outs, lses)
    out, lse = p.merged(outs, lses)
    ref_o, ref_l = p.ref()
    compare(out[:, :, None], lse[:, :, None], ref_o, ref_l, tol=TOL["bf16"])


@pytest.mark.parametrize("d", [64, 128])
@pytest.mark.parametrize("n_splits", [1, 3])
def test_decode_ragged_block_end_before_nan_guard(d, n_splits):
    """Blocks of 250 keys (the last 32-key tile of a block is 26 rows long),
    each the start of a buffer whose following rows are NaN: the last tile of
    every range that ends at the block end reads past it, and those rows must
    read as zeros (the buffer range check), so every partial and the merge
    stay finite and match the oracle."""
    S, c, split, B, Hq, Hkv = 1000, 4, ra.SPLIT_CONTIGUOUS, 1, 4, 1
    p = Decode(S, c, split, B, Hq, Hkv, d, seed=41)
    guarded = {}
    for name, src in (("k", p.ks), ("v", p.vs)):
        guarded[name] = []
        for t in range(c):
            buf = torch.full((B, Hkv, p.n + 64, d), float("nan"), dtype=torch.bfloat16, device=DEV)
            buf[:, :, :p.n] = src[t]
            blk = buf.reshape(-1)[: B * Hkv * p.n * d].view(B, Hkv, p.n, d)  # B = Hkv = 1: block, then NaN rows
            guarded[name].append((blk, buf))
    torch.cuda.synchronize()
    say(f"decode NaN guard d={d} splits={n_splits}")
    n_parts = c * n_splits
    outs = torch.full((n_parts, B, Hq, d), float("nan"), dtype=torch.float32, device=DEV)
    lses = torch.full((n_parts, B, Hq), float("nan"), dtype=torch.float32, device=DEV)
    ra.ring_attn_decode(p.desc(), p.qd, [kb for kb, _ in guarded["k"]], [vb for vb, _ in guarded["v"]],
                        n_splits, outs, lses)
    torch.cuda.synchronize()
    assert torch.isfinite(outs).all() and torch.isfinite(lses).all()
    check_parts(p, list(range(c)), n_splits, outs, lses)
    out, lse = p.merged(outs, lses)
    ref_o, ref_l = p.ref()
    compare(out[:, :, None], lse[:, :, None], ref_o, ref_l, tol=TOL["bf16"])


def test_decode_maximum_block_count():
    p = Decode(8192, 128, ra.SPLIT_ZIGZAG, 1, 8, 1, 128, seed=9)
    outs, lses = p.run(list(range(128)), 2)
    out, lse = p.merged(outs, lses)
    ref_o, ref_l = p.ref()
    compare(out[:, :, None], lse[:, :, None], ref_o, ref_l, tol=TOL["bf16"])


def test_decode_block_subset_in_given_order():
    """A device holding some blocks: parts follow the blocks in the order given."""
    p = Decode(4096, 8, ra.SPLIT_ZIGZAG, 1, 8, 2, 128, seed=5)
    blocks = [5, 2, 7]
    outs, lses = p.run(blocks, 2)
    check_parts(p, blocks, 2, outs, lses)
    out, lse = p.merged(outs, lses)
    keys = np.concatenate([p.perm[t * p.n:(t + 1) * p.n] for t in blocks])
    ref_o, ref_l = p.ref(keys=keys)
    compare(out[:, :, None], lse[:, :, None], ref_o, ref_l, tol=TOL["bf16"])


def test_decode_262k_cache_64x8_heads():
    """The 262 144-token, c = 32, 64/8-head shape: all 32 blocks in 4 ranges each,
    128 partials merged in one strided call, every head against the oracle."""
    w = workloads.WORKLOAD_BY_NAME["s256k_c32_zigzag_64x8"]
    p = Decode(w.seq_len, w.n_shards, w.split, w.batch, w.h_q, w.h_kv, w.head_dim, seed=w.seed, sigma=w.sigma)
    say("decode 262k")
    outs, lses = p.run(list(range(w.n_shards)), 4)
    out, lse = p.merged(outs, lses)
    ref_o, ref_l = p.ref()
    compare(out[:, :, None], lse[:, :, None], ref_o, ref_l, tol=TOL["bf16"])
    # Two partials spot-checked against their own key ranges.
    for t, s in ((0, 0), (31, 3)):
        ref_o, ref_l = p.ref(keys=p.range_keys(t, s, 4))
        compare(outs[t * 4 + s][:, :, None], lses[t * 4 + s][:, :, None], ref_o, ref_l, tol=TOL["bf16"])


def test_strided_merge_in_place_matches_pointer_merge():
    g = torch.Generator(device=DEV).manual_seed(3)
    n_parts, B, H, R, d = 5, 2, 3, 17, 64
    outs = torch.randn((n_parts, B, H, R, d), generator=g, device=DEV)
    lses = torch.randn((n_parts, B, H, R), generator=g, device=DEV) * 4
    lses[1, 0, 0, :3] = float("-inf")
    lses[:, 1, 2, 5] = float("-inf")  # a row with no keys in any part
    out = torch.empty((B, H, R, d), device=DEV)
    lse = torch.empty((B, H, R), device=DEV)
    ra.ring_attn_merge(B, H, R, d, list(outs), ra.F32, list(lses), out, ra.F32, lse)
    o2, l2 = outs.clone(), lses.clone()
    ra.ring_attn_merge_strided(B, H, R, d, o2, ra.F32, l2, o2[0], ra.F32, l2[0])
    torch.cuda.synchronize()
    assert torch.equal(out, o2[0]) and torch.equal(lse, l2[0])
    ref_o, ref_l = oracle.merge([x.cpu().numpy().astype(np.float64) for x in outs],
                                [x.cpu().numpy().astype(np.float64) for x in lses])
    assert np.abs(out.cpu().numpy() - ref_o).max() < 1e-5
    fin = np.isfinite(ref_l)
    assert np.abs(lse.cpu().numpy()[fin] - ref_l[fin]).max() < 1e-5
    assert np.all(np.isneginf(lse.cpu().numpy()[~fin]))


@pytest.mark.parametrize("n_parts,in_place", [(40, False), (40, True), (19, False)])
def test_many_part_merge_vs_oracle(n_parts, in_place):
    """Many parts over few rows (the split-KV shape: the library spreads each
    group's parts over several threads unless lse is written over part 0's)."""
    g = torch.Generator(device=DEV).manual_seed(n_parts)
    B, H, R, d = 1, 6, 3, 128
    outs = torch.randn((n_parts, B, H, R, d), generator=g, device=DEV)
    lses = torch.randn((n_parts, B, H, R), generator=g, device=DEV) * 6
    lses[::3, 0, 1, 0] = float("-inf")   # parts without keys for one row
    lses[:, 0, 4, 2] = float("-inf")     # a row with no keys in any part
    ref_o, ref_l = oracle.merge([x.cpu().numpy().astype(np.float64) for x in outs],
                                [x.cpu().numpy().astype(np.float64) for x in lses])
    if in_place:
        ra.ring_attn_merge_strided(B, H, R, d, outs, ra.F32, lses, outs[0], ra.F32, lses[0])
        out, lse = outs[0], lses[0]
    else:
        out = torch.empty((B, H, R, d), device=DEV)
        lse = torch.empty((B, H, R), device=DEV)
        ra.ring_attn_merge_strided(B, H, R, d, outs, ra.F32, lses, out, ra.F32, lse)
    torch.cuda.synchronize()
    assert np.abs(out.cpu().numpy() - ref_o).max() < 1e-5
    fin = np.isfinite(ref_l)
    assert np.abs(lse.cpu().numpy()[fin] - ref_l[fin]).max() < 1e-5
    assert np.all(np.isneginf(lse.cpu().numpy()[~fin]))
    assert np.all(out.cpu().numpy()[0, 4, 2] == 0)
