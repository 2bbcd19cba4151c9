"""GPU parity of ring_attn_all_shards_fwd: every shard's ring pass in one
launch.  It must equal the per-rank ring_attn_shard_fwd calls bit for bit
(same tiles, same order of operations), count the same work summed over the
ranks, and match the oracle -- at small sizes on every row, on the 8 192-token
workload on every row of heads covering every key/value group, and on the
32 768-token workloads on sampled rows."""
import numpy as np
import pytest
import torch

import oracle
import ring_parallelism_amd as ra
import workloads
from gpu_util import DEV, TOL, Problem, compare, expected_stats, say, up

pytestmark = pytest.mark.gpu

CASES = [
    # (S, c, split, B, Hq, Hkv, d, dtype, causal)
    (1024, 4, ra.SPLIT_ZIGZAG, 1, 4, 2, 128, "bf16", True),
    (1000, 4, ra.SPLIT_CONTIGUOUS, 2, 3, 1, 128, "bf16", True),   # ragged tiles, batch 2
    (1024, 8, ra.SPLIT_STRIPED, 1, 2, 1, 128, "bf16", True),
    (1040, 4, ra.SPLIT_ZIGZAG, 1, 4, 1, 128, "bf16", False),      # bidirectional
    (512, 4, ra.SPLIT_ZIGZAG, 1, 6, 3, 64, "bf16", True),         # d = 64
    (8, 2, ra.SPLIT_ZIGZAG, 1, 2, 1, 128, "bf16", True),          # 2-token chunks
    (1024, 4, ra.SPLIT_CONTIGUOUS, 1, 4, 1, 64, "f32", True),     # fp32: per-rank launches
    # 16 work items per rank: each XCD takes a slice of every rank (heaviest
    # rank first) rather than whole ranks.
    (4096, 4, ra.SPLIT_CONTIGUOUS, 1, 8, 2, 128, "bf16", True),
    (4096, 4, ra.SPLIT_ZIGZAG, 2, 4, 4, 128, "bf16", True),
    # More than 64 ranks: blocks 64 and up take the second lane register of
    # the kernel's per-block count table.
    (12800, 100, ra.SPLIT_CONTIGUOUS, 1, 2, 1, 128, "bf16", True),
    (12800, 100, ra.SPLIT_STRIPED, 1, 2, 1, 64, "bf16", True),
]


def _all_shards(p, out_dtype=ra.F32, causal=True, flags=0, natural=False):
    odt = torch.float32 if out_dtype == ra.F32 else torch.bfloat16
    if natural:
        out = torch.full((p.B, p.Hq, p.S, p.d), float("nan"), dtype=odt, device=DEV)
        lse = torch.full((p.B, p.Hq, p.S), float("nan"), dtype=torch.float32, device=DEV)
        q = up(p.q, p.dtype)
    else:
        out = torch.full((p.c, p.B, p.Hq, p.n_loc, p.d), float("nan"), dtype=odt, device=DEV)
        lse = torch.full((p.c, p.B, p.Hq, p.n_loc), float("nan"), dtype=torch.float32, device=DEV)
        q = p.qs
    stats = torch.zeros(4, dtype=torch.int64, device=DEV)
    ra.ring_attn_all_shards_fwd(p.desc(out_dtype, causal, flags | (ra.FLAG_NATURAL_QO if natural else 0)), q,
                                list(p.ks), list(p.vs), out, lse, stats=stats)
    torch.cuda.synchronize()
    return out, lse, stats


@pytest.mark.parametrize("case", CASES, ids=lambda c: f"S{c[0]}_c{c[1]}_sp{c[2]}_B{c[3]}_h{c[4]}x{c[5]}_d{c[6]}_{c[7]}_"
                                                      f"{'causal' if c[8] else 'full'}")
def test_all_shards_equals_per_rank_passes_and_oracle(case):
    S, c, split, B, Hq, Hkv, d, dtype, causal = case
    p = Problem(S, c, split, B, Hq, Hkv, d, dtype, seed=S + 17 * c)
    tq, tk = ra.ring_attn_tile_shape(p.desc(causal=causal))
    say(f"all shards {case}")
    out, lse, stats = _all_shards(p, causal=causal)
    want = [0, 0, 0, 0]
    for r in range(c):
        o, l, st = p.run(r, causal=causal)
        assert torch.equal(out[r], o) and torch.equal(lse[r], l), f"rank {r} differs from its own pass"
        ref_o, ref_l = p.reference(r, causal=causal)
        compare(out[r], lse[r], ref_o, ref_l, tol=TOL[dtype])
        want = [a + b for a, b in zip(want, expected_stats(p, r, tq, tk, causal))]
    assert stats.cpu().tolist() == want


@pytest.mark.parametrize("case", [CASES[i] for i in (0, 2, 4)], ids=lambda c: f"S{c[0]}_c{c[1]}_sp{c[2]}_d{c[6]}")
def test_all_shards_natural_order_is_full_attention(case):
    """With natural-order q / out / lse, one launch writes the whole sequence's
    attention output in natural order: compared with the oracle at every
    position, bf16 output included."""
    S, c, split, B, Hq, Hkv, d, dtype, causal = case
    p = Problem(S, c, split, B, Hq, Hkv, d, dtype, seed=S + 5)
    ref_o, ref_l = oracle.attention(p.q, p.k, p.v, p.scale, causal)
    for out_dtype in (ra.F32, ra.BF16):
        say(f"all shards natural {case} out={out_dtype}")
        out, lse, _ = _all_shards(p, out_dtype=out_dtype, causal=causal, natural=True)
        compare(out, lse, ref_o, ref_l, tol=TOL[dtype], bf16_out=out_dtype == ra.BF16)


def test_all_shards_s8k_workload_every_row():
    """The 8 192-token workload (c = 8 zig-zag, 32 / 8 heads) in the launch the
    benchmark times (bf16 output): every row of heads that cover every key/value
    group and every slot in a group, for every shard; work counts exact."""
    w = workloads.WORKLOAD_BY_NAME["s8k_c8_zigzag_gqa32x8"]
    p = Problem.from_workload(w)
    tq, tk = ra.ring_attn_tile_shape(p.desc())
    out, lse, stats = _all_shards(p, out_dtype=ra.BF16)
    heads = np.array([0, 5, 10, 15, 17, 22, 27, 31])
    want = [0, 0, 0, 0]
    for r in range(p.c):
        say(f"s8k all shards rank {r}")
        ref_o, ref_l = p.reference(r, heads=heads)
        compare(out[r], lse[r], ref_o, ref_l, heads=heads, tol=TOL["bf16"], bf16_out=True)
        want = [a + b for a, b in zip(want, expected_stats(p, r, tq, tk))]
    assert stats.cpu().tolist() == want


@pytest.mark.parametrize("name", ["s32k_c16_contig_16x1", "s32k_c16_zigzag_16x1"])
def test_all_shards_s32k_sampled(name):
    w = workloads.WORKLOAD_BY_NAME[name]
    p = Problem.from_workload(w)
    tq, tk = ra.ring_attn_tile_shape(p.desc())
    out, lse, stats = _all_shards(p, out_dtype=ra.BF16)
    want = [0, 0, 0, 0]
    for r in range(p.c):
        say(f"{name} all shards rank {r}")
        rows = workloads.sample_rows(p.n_loc, p.n_loc // 2 if p.split == ra.SPLIT_ZIGZAG else p.n_loc, 248, 3000 + r)
        heads = np.array([r % p.Hq])
        ref_o, ref_l = p.reference(r, rows=rows, heads=heads)
        compare(out[r], lse[r], ref_o, ref_l, rows=rows, heads=heads, tol=TOL["bf16"], bf16_out=True)
        want = [a + b for a, b in zip(want, expected_stats(p, r, tq, tk))]
    assert stats.cpu().tolist() == want
