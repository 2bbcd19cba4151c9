"""GPU parity on seeded random configurations: shard lengths 1 .. 700, the
three placements, 1 .. 6 shards, batch 1 or 2, GQA groups 1 .. 5 over 1 .. 3
key/value heads, d = 64 or 128, bf16 (fp32 or bf16 output) and fp32, causal
and bidirectional, ring-ordered or a random subset of the blocks in random
order.  Every row of the chosen rank against the oracle restricted to the
visited blocks' keys, and the work counters bit-exact."""
import numpy as np
import pytest
import torch

import oracle
import ring_parallelism_amd as ra
from gpu_util import DEV, TOL, Problem, compare, expected_stats, say, up

pytestmark = pytest.mark.gpu

SPLITS = [ra.SPLIT_CONTIGUOUS, ra.SPLIT_ZIGZAG, ra.SPLIT_STRIPED]


def _cases(n=120, seed=2024):
    g = np.random.default_rng(seed)
    out = []
    for i in range(n):
        split = SPLITS[int(g.integers(0, 3))]
        c = int(g.integers(1, 7))
        n_loc = int(g.integers(1, 701))
        if split == ra.SPLIT_ZIGZAG and n_loc % 2:
            n_loc += 1
        h_kv = int(g.integers(1, 4))
        group = int(g.choice([1, 2, 4, 5]))
        dtype = "f32" if g.random() < 0.25 else "bf16"
        case = dict(S=n_loc * c, c=c, split=split, B=int(g.integers(1, 3)), h_q=h_kv * group, h_kv=h_kv,
                    d=int(g.choice([64, 128])), dtype=dtype, causal=bool(g.random() < 0.75),
                    bf16_out=dtype == "bf16" and bool(g.random() < 0.25), rank=int(g.integers(0, c)),
                    seed=10_000 + i)
        if g.random() < 0.4:  # a random non-empty subset of the blocks, in random order
            k = int(g.integers(1, c + 1))
            case["owners"] = [int(x) for x in g.permutation(c)[:k]]
        else:
            case["owners"] = None
        out.append(case)
    return out


CASES = _cases()


@pytest.mark.parametrize("case", CASES, ids=lambda k: f"S{k['S']}_c{k['c']}_sp{k['split']}_B{k['B']}_h{k['h_q']}x{k['h_kv']}"
                                                     f"_d{k['d']}_{k['dtype']}{'_bf16out' if k['bf16_out'] else ''}"
                                                     f"_{'causal' if k['causal'] else 'full'}_r{k['rank']}"
                                                     f"{'_sub' if k['owners'] else ''}")
def test_random_configuration(case):
    k = case
    say(f"random config {k}")
    p = Problem(k["S"], k["c"], k["split"], k["B"], k["h_q"], k["h_kv"], k["d"], k["dtype"], seed=k["seed"])
    owners = k["owners"] if k["owners"] is not None else p.ring_owners(k["rank"])
    out_dtype = ra.BF16 if k["bf16_out"] else ra.F32
    tq, tk = ra.ring_attn_tile_shape(p.desc(out_dtype=out_dtype, causal=k["causal"]))
    out, lse, stats = p.run(k["rank"], out_dtype=out_dtype, causal=k["causal"], owners=owners)
    ref_o, ref_l = p.reference(k["rank"], causal=k["causal"], owners=owners)
    compare(out, lse, ref_o, ref_l, tol=TOL[k["dtype"]], bf16_out=k["bf16_out"])
    assert stats.cpu().tolist() == expected_stats(p, k["rank"], tq, tk, k["causal"], owners)


def _split_cases(n=40, seed=2025):
    g = np.random.default_rng(seed)
    out = []
    for i in range(n):
        split = SPLITS[int(g.integers(0, 3))]
        c = int(g.integers(1, 9))
        n_loc = int(g.integers(1, 1201))
        if split == ra.SPLIT_ZIGZAG and n_loc % 2:
            n_loc += 1
        h_kv = int(g.integers(1, 3))
        owners = [int(x) for x in g.permutation(c)[:int(g.integers(1, c + 1))]] if g.random() < 0.3 else None
        n_blocks = len(owners) if owners else c
        out.append(dict(S=n_loc * c, c=c, split=split, B=int(g.integers(1, 3)), h_q=h_kv * int(g.choice([1, 2, 4])),
                        h_kv=h_kv, d=int(g.choice([64, 128])), causal=bool(g.random() < 0.75),
                        bf16_out=bool(g.random() < 0.3), rank=int(g.integers(0, c)), owners=owners,
                        n_splits=int(g.integers(1, n_blocks + 1)), seed=20_000 + i))
    return out


@pytest.mark.parametrize("case", _split_cases(), ids=lambda k: f"S{k['S']}_c{k['c']}_sp{k['split']}_h{k['h_q']}x{k['h_kv']}"
                                                             f"_d{k['d']}_splits{k['n_splits']}_r{k['rank']}")
def test_random_split_pass(case):
    """The block list cut into concurrent groups folded by the merge: the
    oracle's result over the visited blocks, and the single pass's counters."""
    k = case
    say(f"random split pass {k}")
    p = Problem(k["S"], k["c"], k["split"], k["B"], k["h_q"], k["h_kv"], k["d"], "bf16", seed=k["seed"])
    r = k["rank"]
    owners = k["owners"] if k["owners"] is not None else p.ring_owners(r)
    out_dtype = ra.BF16 if k["bf16_out"] else ra.F32
    odt = torch.bfloat16 if k["bf16_out"] else torch.float32
    ns, n = k["n_splits"], p.n_loc
    work = torch.full((ns, p.B, p.Hq, n, p.d), float("nan"), dtype=torch.float32, device=DEV)
    work_l = torch.full((ns, p.B, p.Hq, n), float("nan"), dtype=torch.float32, device=DEV)
    out = torch.full((p.B, p.Hq, n, p.d), float("nan"), dtype=odt, device=DEV)
    lse = torch.full((p.B, p.Hq, n), float("nan"), dtype=torch.float32, device=DEV)
    stats = torch.zeros(4, dtype=torch.int64, device=DEV)
    desc = p.desc(out_dtype, k["causal"])
    ra.ring_attn_shard_fwd_split(desc, r, p.qs[r], [p.ks[j] for j in owners], [p.vs[j] for j in owners], ns,
                                 work, work_l, out, lse, block_owner=owners, stats=stats)
    torch.cuda.synchronize()
    ref_o, ref_l = p.reference(r, causal=k["causal"], owners=owners)
    compare(out, lse, ref_o, ref_l, tol=TOL["bf16"], bf16_out=k["bf16_out"])
    _, _, s1 = p.run(r, causal=k["causal"], owners=owners)
    assert torch.equal(stats, s1)


def _natural_cases(n=30, seed=2026):
    g = np.random.default_rng(seed)
    out = []
    for i in range(n):
        split = SPLITS[int(g.integers(0, 3))]
        c = int(g.integers(1, 7))
        n_loc = int(g.integers(1, 501))
        if split == ra.SPLIT_ZIGZAG and n_loc % 2:
            n_loc += 1
        h_kv = int(g.integers(1, 3))
        dtype = "f32" if g.random() < 0.3 else "bf16"
        out.append(dict(S=n_loc * c, c=c, split=split, B=int(g.integers(1, 3)), h_q=h_kv * int(g.choice([1, 3])),
                        h_kv=h_kv, d=int(g.choice([64, 128])), dtype=dtype, causal=bool(g.random() < 0.75),
                        rank=int(g.integers(0, c)), seed=30_000 + i))
    return out


@pytest.mark.parametrize("case", _natural_cases(), ids=lambda k: f"S{k['S']}_c{k['c']}_sp{k['split']}_h{k['h_q']}x{k['h_kv']}"
                                                               f"_d{k['d']}_{k['dtype']}_r{k['rank']}")
def test_random_natural_order_q_out(case):
    """Q read and out / lse written at global positions of natural-order
    tensors: the rank's rows equal its shard-layout result bit for bit, and
    no other row is touched."""
    k = case
    say(f"random natural q/out {k}")
    p = Problem(k["S"], k["c"], k["split"], k["B"], k["h_q"], k["h_kv"], k["d"], k["dtype"], seed=k["seed"])
    r = k["rank"]
    owners = p.ring_owners(r)
    out_nat = torch.full((p.B, p.Hq, p.S, p.d), float("nan"), dtype=torch.float32, device=DEV)
    lse_nat = torch.full((p.B, p.Hq, p.S), float("nan"), dtype=torch.float32, device=DEV)
    ra.ring_attn_shard_fwd(p.desc(ra.F32, k["causal"], flags=ra.FLAG_NATURAL_QO), r, up(p.q, k["dtype"]),
                           [p.ks[j] for j in owners], [p.vs[j] for j in owners], out_nat, lse_nat, block_owner=owners)
    o, l, _ = p.run(r, causal=k["causal"])
    rows = torch.from_numpy(p.perm[r * p.n_loc:(r + 1) * p.n_loc]).to(DEV)
    torch.cuda.synchronize()
    assert torch.equal(out_nat[:, :, rows], o) and torch.equal(lse_nat[:, :, rows], l)
    # ... and both equal the oracle at the rank's global positions.
    ref_o, ref_l = p.reference(r, causal=k["causal"])
    compare(out_nat[:, :, rows], lse_nat[:, :, rows], ref_o, ref_l, tol=TOL[k["dtype"]])
    others = torch.ones(p.S, dtype=torch.bool, device=DEV)
    others[rows] = False
    assert torch.isnan(out_nat[:, :, others]).all() and torch.isnan(lse_nat[:, :, others]).all()


def _decode_cases(n=30, seed=2027):
    g = np.random.default_rng(seed)
    out = []
    for i in range(n):
        split = SPLITS[int(g.integers(0, 3))]
        c = int(g.integers(1, 9))
        n_loc = int(g.integers(1, 1501))
        if split == ra.SPLIT_ZIGZAG and n_loc % 2:
            n_loc += 1
        h_kv = int(g.integers(1, 4))
        blocks = [int(x) for x in g.permutation(c)[:int(g.integers(1, c + 1))]]
        out.append(dict(S=n_loc * c, c=c, split=split, B=int(g.integers(1, 3)),
                        h_q=h_kv * int(g.choice([1, 2, 7, 16, 32])), h_kv=h_kv, d=int(g.choice([64, 128])),
                        blocks=blocks, n_splits=int(g.integers(1, min(9, n_loc) + 1)), seed=40_000 + i))
    return out


@pytest.mark.parametrize("case", _decode_cases(), ids=lambda k: f"S{k['S']}_c{k['c']}_sp{k['split']}_h{k['h_q']}x{k['h_kv']}"
                                                              f"_d{k['d']}_nb{len(k['blocks'])}_splits{k['n_splits']}")
def test_random_decode_and_strided_merge(case):
    """Split-KV decode over a random subset of the blocks in random order:
    every partial against its key range, and the strided merge of all of them
    against attention of a token after the whole cache over those blocks."""
    from test_gpu_decode import Decode, check_parts
    k = case
    say(f"random decode {k}")
    p = Decode(k["S"], k["c"], k["split"], k["B"], k["h_q"], k["h_kv"], k["d"], seed=k["seed"])
    outs, lses = p.run(k["blocks"], k["n_splits"])
    check_parts(p, k["blocks"], k["n_splits"], outs, lses)
    out, lse = p.merged(outs, lses)
    keys = np.concatenate([p.perm[t * p.n:(t + 1) * p.n] for t in k["blocks"]])
    ref_o, ref_l = p.ref(keys=keys)
    compare(out[:, :, None], lse[:, :, None], ref_o, ref_l, tol=TOL["bf16"])


def _partition_cases(n=40, seed=2028):
    g = np.random.default_rng(seed)
    out = []
    for i in range(n):
        split = SPLITS[int(g.integers(0, 3))]
        c = int(g.integers(1, 17))
        n_loc = int(g.integers(1, 400))
        if split == ra.SPLIT_ZIGZAG and n_loc % 2:
            n_loc += 1
        out.append(dict(S=n_loc * c, c=c, split=split, outer=int(g.integers(1, 5)),
                        inner=int(g.choice([1, 2, 3, 4, 6, 8, 12, 16, 24, 32, 100, 256, 512])), seed=50_000 + i))
    return out


@pytest.mark.parametrize("case", _partition_cases(), ids=lambda k: f"S{k['S']}_c{k['c']}_sp{k['split']}_o{k['outer']}_b{k['inner']}")
def test_random_partition_gather_scatter(case):
    """Placement, gather and scatter at random sizes and row widths (any byte
    count): perm and every byte against the oracle's partition."""
    k = case
    say(f"random partition {k}")
    S, c, split, outer, inner = k["S"], k["c"], k["split"], k["outer"], k["inner"]
    g = np.random.default_rng(k["seed"])
    src = g.integers(0, 256, size=(outer, S, inner), dtype=np.uint8)
    d_src = torch.from_numpy(src).to(DEV)
    d_dst = torch.zeros((c, outer, S // c, inner), dtype=torch.uint8, device=DEV)
    perm_d = torch.full((S,), -1, dtype=torch.int64, device=DEV)
    ra.zigzag_partition(S, c, split, perm_d, d_src, d_dst, outer, inner)
    perm = oracle.partition_perm(S, c, split)
    back = torch.zeros_like(d_src)
    ra.zigzag_unpartition(S, c, split, d_dst, back, outer, inner)
    torch.cuda.synchronize()
    assert np.array_equal(perm_d.cpu().numpy(), perm)
    pr = perm.reshape(c, S // c)
    assert np.array_equal(d_dst.cpu().numpy(), np.stack([src[:, pr[r]] for r in range(c)]))
    assert np.array_equal(back.cpu().numpy(), src)


def _merge_cases(n=30, seed=2029):
    g = np.random.default_rng(seed)
    dts = [ra.F32, ra.BF16]
    out = []
    for i in range(n):
        pdt, odt = dts[int(g.integers(0, 2))], dts[int(g.integers(0, 2))]
        out.append(dict(B=int(g.integers(1, 3)), H=int(g.integers(1, 5)), R=int(g.integers(1, 300)),
                        d=int(g.choice([4, 8, 16, 32, 64, 128, 256])), n_parts=int(g.integers(1, 65)),
                        parts_dtype=pdt, out_dtype=odt, in_place=bool(pdt == odt and g.random() < 0.3),
                        seed=60_000 + i))
    return out


@pytest.mark.parametrize("case", _merge_cases(), ids=lambda k: f"B{k['B']}_H{k['H']}_R{k['R']}_d{k['d']}_n{k['n_parts']}"
                                                             f"_p{k['parts_dtype']}_o{k['out_dtype']}{'_inplace' if k['in_place'] else ''}")
def test_random_pointer_merge(case):
    """ring_attn_merge with 1 .. 64 parts of random sizes and dtypes, in place
    or not, with empty parts and empty rows, against the oracle's merge (of
    the values the kernel reads)."""
    k = case
    say(f"random merge {k}")
    g = np.random.default_rng(k["seed"])
    B, H, R, d, n = k["B"], k["H"], k["R"], k["d"], k["n_parts"]
    outs = g.standard_normal((n, B, H, R, d)).astype(np.float32)
    lses = (g.standard_normal((n, B, H, R)) * 4).astype(np.float32)
    empty = g.random((n, B, H, R)) < 0.1             # parts without keys for some rows
    empty[:, 0, 0, 0] = True                         # one row with no keys anywhere
    lses[empty] = -np.inf
    outs[empty] = 0.0
    tdt = torch.float32 if k["parts_dtype"] == ra.F32 else torch.bfloat16
    d_outs = [torch.from_numpy(outs[j]).to(DEV).to(tdt) for j in range(n)]
    d_lses = [torch.from_numpy(lses[j]).to(DEV) for j in range(n)]
    seen = np.stack([x.float().cpu().numpy() for x in d_outs]).astype(np.float64)  # bf16-rounded parts
    ref_o, ref_l = oracle.merge(list(seen), [lses[j].astype(np.float64) for j in range(n)])
    odt = torch.float32 if k["out_dtype"] == ra.F32 else torch.bfloat16
    if k["in_place"]:
        out, lse = d_outs[0], d_lses[0]
    else:
        out = torch.full((B, H, R, d), float("nan"), dtype=odt, device=DEV)
        lse = torch.full((B, H, R), float("nan"), dtype=torch.float32, device=DEV)
    ra.ring_attn_merge(B, H, R, d, d_outs, k["parts_dtype"], d_lses, out, k["out_dtype"], lse)
    torch.cuda.synchronize()
    o = out.float().cpu().numpy()
    bound = 1e-5 + (np.abs(ref_o) * 2.0 ** -8 if k["out_dtype"] == ra.BF16 else 0.0)
    assert np.all(np.abs(o - ref_o) <= bound)
    l = lse.cpu().numpy()
    assert np.array_equal(np.isneginf(l), np.isneginf(ref_l))
    fin = np.isfinite(ref_l)
    assert np.abs(l[fin] - ref_l[fin]).max() <= 1e-5 if fin.any() else True
    assert np.all(o[0, 0, 0] == 0.0)
