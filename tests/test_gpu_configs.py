"""GPU parity on the five benchmark workloads, in the launch configuration the
benchmark times.  Small workloads are checked on every row; large ones on a
seeded row sample (first and last 4 rows of every chunk plus 248 uniform
draws per shard) against the oracle's full visible key set, plus exact work
counts for every shard."""
import numpy as np
import pytest
import torch

import oracle
import ring_parallelism_amd as ra
import workloads
from gpu_util import TOL, Problem, compare, expected_stats, say

pytestmark = pytest.mark.gpu


def _heads_cover_groups(Hq, Hkv, n):
    """n query heads spread over every key/value group and position in the group."""
    g = Hq // Hkv
    heads = sorted({(i * Hq) // n + (i % g) for i in range(n)})
    return np.array([min(h, Hq - 1) for h in heads], dtype=np.int64)


@pytest.fixture(scope="module")
def problems():
    cache = {}

    def get(name):
        if name not in cache:
            cache.clear()
            torch.cuda.empty_cache()
            say(f"building workload {name}")
            cache[name] = Problem.from_workload(workloads.WORKLOAD_BY_NAME[name])
        return cache[name]
    return get


def test_s1k_fp32_all_rows(problems):
    p = problems("s1k_c4_contig_f32_d64")
    tq, tk = ra.ring_attn_tile_shape(p.desc())
    for r in range(p.c):
        say(f"s1k rank {r}")
        out, lse, st = p.run(r)
        ref_o, ref_l = p.reference(r)
        compare(out, lse, ref_o, ref_l, tol=TOL["f32"])
        assert st.cpu().tolist() == expected_stats(p, r, tq, tk)


def test_s8k_gqa_all_rows(problems):
    p = problems("s8k_c8_zigzag_gqa32x8")
    heads = np.array([0, 5, 10, 15, 17, 22, 27, 31])   # every KV group, every slot in a group
    tq, tk = ra.ring_attn_tile_shape(p.desc())
    pairs = []
    for r in range(p.c):
        say(f"s8k rank {r}")
        out, lse, st = p.run(r)
        ref_o, ref_l = p.reference(r, heads=heads)
        compare(out, lse, ref_o, ref_l, heads=heads, tol=TOL["bf16"])
        st = st.cpu().tolist()
        assert st == expected_stats(p, r, tq, tk)
        pairs.append(st[0])
    assert len(set(pairs)) == 1   # zig-zag: equal work on every shard


def _sampled(p, r, heads, causal=True, owners=None, run=None):
    rows = workloads.sample_rows(p.n_loc, p.n_loc // 2 if p.split == ra.SPLIT_ZIGZAG else p.n_loc, 248, 1000 + r)
    out, lse, st = run if run is not None else p.run(r, causal=causal, owners=owners)
    ref_o, ref_l = p.reference(r, rows=rows, heads=heads, causal=causal, owners=owners)
    return compare(out, lse, ref_o, ref_l, rows=rows, heads=heads, tol=TOL["bf16"]), st


@pytest.mark.parametrize("name", ["s32k_c16_contig_16x1", "s32k_c16_zigzag_16x1"])
def test_s32k_all_shards_sampled(problems, name):
    p = problems(name)
    tq, tk = ra.ring_attn_tile_shape(p.desc())
    pairs = []
    for r in range(p.c):
        say(f"{name} rank {r}")
        heads = np.array([r % p.Hq, (r + 7) % p.Hq])
        _, st = _sampled(p, r, heads)
        st = st.cpu().tolist()
        assert st == expected_stats(p, r, tq, tk)
        pairs.append(st[0] // (p.B * p.Hq))
    assert pairs == oracle.pair_counts(p.S, p.c, p.split).tolist()
    if p.split == ra.SPLIT_ZIGZAG:
        assert len(set(pairs)) == 1
    else:
        assert all(a < b for a, b in zip(pairs, pairs[1:]))


def test_s128k_all_shards_sampled(problems):
    p = problems("s128k_c16_zigzag_16x1")
    tq, tk = ra.ring_attn_tile_shape(p.desc())
    for r in range(p.c):
        say(f"s128k rank {r}")
        heads = np.array([r % p.Hq])
        _, st = _sampled(p, r, heads)
        assert st.cpu().tolist() == expected_stats(p, r, tq, tk)


def test_s128k_benched_launch_bf16_out_sampled(problems):
    """The launch the benchmark times -- bf16 output -- against the oracle on
    sampled rows of three shards (every query head of one KV group slot)."""
    p = problems("s128k_c16_zigzag_16x1")
    for r in (0, 7, 15):
        say(f"s128k bf16-out rank {r}")
        rows = workloads.sample_rows(p.n_loc, p.n_loc // 2, 248, 1000 + r)
        heads = np.array([(3 * r) % p.Hq, (3 * r + 8) % p.Hq])
        out, lse, _ = p.run(r, out_dtype=ra.BF16, with_stats=False)
        ref_o, ref_l = p.reference(r, rows=rows, heads=heads)
        compare(out, lse, ref_o, ref_l, rows=rows, heads=heads, tol=TOL["bf16"], bf16_out=True)
        del out, lse


def test_s128k_natural_order_q_out_sampled(problems):
    """The fused gather/scatter at full size: Q read and bf16 out / lse written
    at global positions of the natural-order 131 072-token tensors, compared
    with the oracle at the sampled rows' positions for two ranks."""
    import torch
    from gpu_util import DEV, up
    p = problems("s128k_c16_zigzag_16x1")
    qn = up(p.q, p.dtype)
    out_nat = torch.zeros((p.B, p.Hq, p.S, p.d), dtype=torch.bfloat16, device=DEV)
    lse_nat = torch.zeros((p.B, p.Hq, p.S), dtype=torch.float32, device=DEV)
    desc = p.desc(ra.BF16, True, flags=ra.FLAG_NATURAL_QO)
    for r in (0, 11):
        say(f"s128k natural q/out rank {r}")
        owners = p.ring_owners(r)
        ra.ring_attn_shard_fwd(desc, r, qn, [p.ks[j] for j in owners], [p.vs[j] for j in owners], out_nat, lse_nat,
                               block_owner=owners)
        torch.cuda.synchronize()
        rows = workloads.sample_rows(p.n_loc, p.n_loc // 2, 248, 2000 + r)
        pos = p.perm[r * p.n_loc + rows]
        heads = np.array([r % p.Hq])
        ref_o, ref_l = p.reference(r, rows=rows, heads=heads)
        pos_t = torch.from_numpy(pos).to(DEV)
        compare(out_nat[:, :, pos_t], lse_nat[:, :, pos_t], ref_o, ref_l, heads=heads, tol=TOL["bf16"],
                bf16_out=True)
    del qn, out_nat, lse_nat


def test_s256k_one_shard_fused_partial_and_bidirectional(problems):
    p = problems("s256k_c32_zigzag_64x8")
    r = 0
    heads = _heads_cover_groups(p.Hq, p.Hkv, 4)
    tq, tk = ra.ring_attn_tile_shape(p.desc())
    say("s256k fused causal")
    fused = p.run(r)
    _sampled(p, r, heads, run=fused)
    assert fused[2].cpu().tolist() == expected_stats(p, r, tq, tk)
    # Ring steps as separate partial passes folded with the merge kernel.
    say("s256k partial + merge")
    acc_o = acc_l = None
    for j in p.ring_owners(r):
        po, pl, _ = p.run(r, owners=[j], with_stats=False, fill=0.0)
        if acc_o is None:
            acc_o, acc_l = po, pl
        else:
            ra.ring_attn_merge(p.B, p.Hq, p.n_loc, p.d, [acc_o, po], ra.F32, [acc_l, pl], acc_o, ra.F32, acc_l)
            del po, pl
    torch.cuda.synchronize()
    _sampled(p, r, heads, run=(acc_o, acc_l, None))
    assert (acc_o - fused[0]).abs().max().item() <= 2e-2
    del fused, acc_o, acc_l
    say("s256k bidirectional")
    _sampled(p, r, heads, causal=False)
    say("s256k fused causal, bf16 output (the timed launch)")
    rows = workloads.sample_rows(p.n_loc, p.n_loc // 2, 248, 1000 + r)
    out, lse, _ = p.run(r, out_dtype=ra.BF16, with_stats=False)
    ref_o, ref_l = p.reference(r, rows=rows, heads=heads)
    compare(out, lse, ref_o, ref_l, rows=rows, heads=heads, tol=TOL["bf16"], bf16_out=True)
