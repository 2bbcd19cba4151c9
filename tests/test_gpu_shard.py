"""GPU parity of the shard forward, partition and merge at small sizes (every
row checked), including ragged shards and the method's degenerate cases."""
import numpy as np
import pytest
import torch

import oracle
import ring_parallelism_amd as ra
import workloads
from gpu_util import DEV, TOL, Problem, compare, expected_stats, say, up

pytestmark = pytest.mark.gpu


# ---------------------------------------------------------------- partition

@pytest.mark.parametrize("S,c,split", [
    (1024, 4, ra.SPLIT_CONTIGUOUS), (8192, 8, ra.SPLIT_ZIGZAG), (32768, 16, ra.SPLIT_CONTIGUOUS),
    (32768, 16, ra.SPLIT_ZIGZAG), (131072, 16, ra.SPLIT_ZIGZAG), (262144, 32, ra.SPLIT_ZIGZAG),
    (1000, 8, ra.SPLIT_STRIPED), (6, 3, ra.SPLIT_ZIGZAG), (7, 1, ra.SPLIT_CONTIGUOUS),
])
def test_partition_perm_bit_exact(S, c, split):
    say(f"partition perm S={S} c={c} split={split}")
    perm = torch.full((S,), -1, dtype=torch.int64, device=DEV)
    ra.zigzag_partition(S, c, split, perm)
    torch.cuda.synchronize()
    assert np.array_equal(perm.cpu().numpy(), oracle.partition_perm(S, c, split))


@pytest.mark.parametrize("S,c,split,inner", [
    (1024, 4, ra.SPLIT_ZIGZAG, 256), (8192, 8, ra.SPLIT_ZIGZAG, 256), (1000, 4, ra.SPLIT_CONTIGUOUS, 6),
    (96, 3, ra.SPLIT_STRIPED, 12), (120, 5, ra.SPLIT_ZIGZAG, 3), (32768, 16, ra.SPLIT_CONTIGUOUS, 256),
])
def test_partition_gather_scatter(S, c, split, inner):
    say(f"partition gather S={S} c={c} split={split} inner={inner}")
    outer = 3
    g = np.random.default_rng(S + c)
    src = g.integers(0, 256, size=(outer, S, inner), dtype=np.uint8)
    d_src = torch.from_numpy(src).to(DEV)
    d_dst = torch.zeros((c, outer, S // c, inner), dtype=torch.uint8, device=DEV)
    ra.zigzag_partition(S, c, split, None, d_src, d_dst, outer, inner)
    perm = oracle.partition_perm(S, c, split).reshape(c, S // c)
    want = np.stack([src[:, perm[r]] for r in range(c)])
    assert np.array_equal(d_dst.cpu().numpy(), want)
    back = torch.zeros_like(d_src)
    ra.zigzag_unpartition(S, c, split, d_dst, back, outer, inner)
    torch.cuda.synchronize()
    assert np.array_equal(back.cpu().numpy(), src)


# ---------------------------------------------------------------- shard forward

SMALL_CASES = [
    # (S, c, split, B, Hq, Hkv, d, dtype, causal)
    (1024, 4, ra.SPLIT_CONTIGUOUS, 1, 4, 1, 64, "f32", True),       # the fp32 workload itself
    (1024, 4, ra.SPLIT_ZIGZAG, 1, 4, 2, 128, "bf16", True),
    (1000, 4, ra.SPLIT_CONTIGUOUS, 1, 3, 1, 128, "bf16", True),     # 250-row shards: ragged tiles
    (1040, 4, ra.SPLIT_ZIGZAG, 2, 4, 2, 128, "bf16", True),         # 130-token chunks, batch 2
    (1040, 4, ra.SPLIT_ZIGZAG, 1, 4, 1, 128, "bf16", False),        # bidirectional
    (1024, 8, ra.SPLIT_STRIPED, 1, 2, 1, 128, "bf16", True),        # round-robin placement
    (300, 1, ra.SPLIT_CONTIGUOUS, 1, 2, 2, 128, "bf16", True),      # c = 1: plain attention
    (512, 4, ra.SPLIT_ZIGZAG, 1, 6, 3, 64, "bf16", True),           # d = 64 bf16, GQA 2
    (2, 2, ra.SPLIT_CONTIGUOUS, 1, 1, 1, 128, "bf16", True),        # one token per shard
    (8, 2, ra.SPLIT_ZIGZAG, 1, 2, 1, 128, "bf16", True),            # 2-token chunks
    (1000, 4, ra.SPLIT_CONTIGUOUS, 1, 2, 1, 64, "f32", True),       # fp32 ragged
    (640, 5, ra.SPLIT_ZIGZAG, 1, 2, 1, 128, "f32", False),          # fp32, d = 128, bidirectional
    (4096, 2, ra.SPLIT_ZIGZAG, 1, 2, 1, 128, "bf16", True),         # 2048-row shards: many tiles
]


@pytest.mark.parametrize("case", SMALL_CASES, ids=lambda c: f"S{c[0]}_c{c[1]}_sp{c[2]}_B{c[3]}_h{c[4]}x{c[5]}_d{c[6]}_{c[7]}_{'causal' if c[8] else 'full'}")
def test_shard_fwd_every_row(case):
    S, c, split, B, Hq, Hkv, d, dtype, causal = case
    p = Problem(S, c, split, B, Hq, Hkv, d, dtype, seed=S + c)
    tq, tk = ra.ring_attn_tile_shape(p.desc(causal=causal))
    for r in range(c):
        say(f"shard_fwd {case} rank {r}")
        out, lse, stats = p.run(r, causal=causal)
        ref_o, ref_l = p.reference(r, causal=causal)
        compare(out, lse, ref_o, ref_l, tol=TOL[dtype])
        assert stats.cpu().tolist() == expected_stats(p, r, tq, tk, causal), f"stats rank {r}"


@pytest.mark.parametrize("case", [SMALL_CASES[i] for i in (0, 2, 3, 4, 5, 7, 9, 10, 11)],
                         ids=lambda c: f"S{c[0]}_c{c[1]}_sp{c[2]}_d{c[6]}_{c[7]}_{'causal' if c[8] else 'full'}")
def test_natural_qo_matches_shard_layout(case):
    """Q read and out / lse written at global positions: after every rank has
    run, the natural-order result is the shard-layout result scattered back,
    bit for bit, and every row was written."""
    S, c, split, B, Hq, Hkv, d, dtype, causal = case
    p = Problem(S, c, split, B, Hq, Hkv, d, dtype, seed=S + c + 1)
    qn = up(p.q, dtype)
    out_nat = torch.full((B, Hq, S, d), float("nan"), dtype=torch.float32, device=DEV)
    lse_nat = torch.full((B, Hq, S), float("nan"), dtype=torch.float32, device=DEV)
    desc = p.desc(ra.F32, causal, flags=ra.FLAG_NATURAL_QO)
    n = S // c
    perm = torch.from_numpy(p.perm).to(DEV)
    for r in range(c):
        say(f"natural q/out {case} rank {r}")
        owners = p.ring_owners(r)
        ra.ring_attn_shard_fwd(desc, r, qn, [p.ks[j] for j in owners], [p.vs[j] for j in owners], out_nat, lse_nat,
                               block_owner=owners)
        o, l, _ = p.run(r, causal=causal)
        rows = perm[r * n:(r + 1) * n]
        torch.cuda.synchronize()
        assert torch.equal(out_nat[:, :, rows], o) and torch.equal(lse_nat[:, :, rows], l), f"rank {r}"
    assert not torch.isnan(out_nat).any() and not torch.isnan(lse_nat).any()


@pytest.mark.parametrize("case", [SMALL_CASES[i] for i in (0, 1, 3, 4, 5, 7, 9, 10, 11)],
                         ids=lambda c: f"S{c[0]}_c{c[1]}_sp{c[2]}_d{c[6]}_{c[7]}_{'causal' if c[8] else 'full'}")
def test_natural_qo_matches_oracle(case):
    """Q read and out / lse written at global positions of natural-order
    tensors ("Splitting the Sequence", intro: device k holds chunks k and
    2c-1-k): after every rank has run, the natural-order tensors are compared
    element by element with the oracle's full attention at every position, in
    both output dtypes."""
    S, c, split, B, Hq, Hkv, d, dtype, causal = case
    p = Problem(S, c, split, B, Hq, Hkv, d, dtype, seed=S + c + 2)
    qn = up(p.q, dtype)
    ref_o, ref_l = oracle.attention(p.q, p.k, p.v, p.scale, causal)
    for out_dtype in ([ra.F32] if dtype == "f32" else [ra.F32, ra.BF16]):
        odt = torch.float32 if out_dtype == ra.F32 else torch.bfloat16
        out_nat = torch.full((B, Hq, S, d), float("nan"), dtype=odt, device=DEV)
        lse_nat = torch.full((B, Hq, S), float("nan"), dtype=torch.float32, device=DEV)
        desc = p.desc(out_dtype, causal, flags=ra.FLAG_NATURAL_QO)
        for r in range(c):
            say(f"natural q/out vs oracle {case} out={out_dtype} rank {r}")
            owners = p.ring_owners(r)
            ra.ring_attn_shard_fwd(desc, r, qn, [p.ks[j] for j in owners], [p.vs[j] for j in owners], out_nat,
                                   lse_nat, block_owner=owners)
        torch.cuda.synchronize()
        compare(out_nat, lse_nat, ref_o, ref_l, tol=TOL[dtype], bf16_out=out_dtype == ra.BF16)


@pytest.mark.parametrize("S,c,split,B,Hq,Hkv,d,n_splits,out_dtype", [
    (4096, 4, ra.SPLIT_ZIGZAG, 1, 4, 1, 128, 2, ra.F32),
    (4096, 8, ra.SPLIT_CONTIGUOUS, 1, 4, 2, 128, 8, ra.F32),   # one block per group
    (1040, 4, ra.SPLIT_ZIGZAG, 2, 4, 2, 128, 3, ra.F32),        # ragged tiles, uneven groups
    (2048, 4, ra.SPLIT_STRIPED, 1, 2, 1, 64, 4, ra.F32),
    (4096, 4, ra.SPLIT_ZIGZAG, 1, 4, 1, 128, 4, ra.BF16),
])
def test_split_pass_matches_oracle_and_counts(S, c, split, B, Hq, Hkv, d, n_splits, out_dtype):
    """Concurrent groups of blocks folded by the merge: same result as the
    oracle, same work counters as the single pass."""
    p = Problem(S, c, split, B, Hq, Hkv, d, "bf16", seed=S + n_splits)
    odt = torch.float32 if out_dtype == ra.F32 else torch.bfloat16
    n = S // c
    work = torch.full((n_splits, B, Hq, n, d), float("nan"), dtype=torch.float32, device=DEV)
    work_l = torch.full((n_splits, B, Hq, n), float("nan"), dtype=torch.float32, device=DEV)
    for r in range(c):
        say(f"split pass S={S} c={c} rank {r} splits {n_splits}")
        owners = p.ring_owners(r)
        out = torch.full((B, Hq, n, d), float("nan"), dtype=odt, device=DEV)
        lse = torch.full((B, Hq, n), float("nan"), dtype=torch.float32, device=DEV)
        stats = torch.zeros(4, dtype=torch.int64, device=DEV)
        ra.ring_attn_shard_fwd_split(p.desc(out_dtype), r, p.qs[r], [p.ks[j] for j in owners],
                                     [p.vs[j] for j in owners], n_splits, work, work_l, out, lse,
                                     block_owner=owners, stats=stats)
        torch.cuda.synchronize()
        ref_o, ref_l = p.reference(r)
        compare(out, lse, ref_o, ref_l, tol=TOL["bf16"], bf16_out=out_dtype == ra.BF16)
        _, _, s1 = p.run(r)
        assert torch.equal(stats, s1), f"stats rank {r}"


@pytest.mark.parametrize("split", [ra.SPLIT_ZIGZAG, ra.SPLIT_CONTIGUOUS, ra.SPLIT_STRIPED])
def test_maximum_block_count(split):
    """RA_MAX_BLOCKS (128) ring blocks in one call: every row of three ranks,
    and the work counters (blocks 64-127 take the second lane register of
    the kernel's per-block count table)."""
    S, c = 16384, 128
    p = Problem(S, c, split, 1, 2, 1, 128, "bf16", seed=77)
    tq, tk = ra.ring_attn_tile_shape(p.desc())
    for r in (0, 63, 127):
        say(f"128 blocks split {split} rank {r}")
        out, lse, stats = p.run(r)
        ref_o, ref_l = p.reference(r)
        compare(out, lse, ref_o, ref_l, tol=TOL["bf16"])
        assert stats.cpu().tolist() == expected_stats(p, r, tq, tk), f"stats rank {r}"


def test_bf16_output_mode():
    p = Problem(2048, 4, ra.SPLIT_ZIGZAG, 1, 4, 1, 128, "bf16", seed=11)
    for r in range(4):
        say(f"bf16 out rank {r}")
        out, lse, _ = p.run(r, out_dtype=ra.BF16)
        ref_o, ref_l = p.reference(r)
        compare(out, lse, ref_o, ref_l, tol=TOL["bf16"], bf16_out=True)


def test_deterministic_and_writes_every_row():
    p = Problem(4096, 4, ra.SPLIT_ZIGZAG, 1, 4, 1, 128, "bf16", seed=3)
    say("determinism")
    o1, l1, s1 = p.run(1, fill=float("nan"))
    o2, l2, s2 = p.run(1, fill=0.0)
    assert torch.equal(o1, o2) and torch.equal(l1, l2) and torch.equal(s1, s2)
    assert torch.isfinite(o1).all() and torch.isfinite(l1).all()


def test_sync_loads_flag_is_bitwise_neutral():
    """The no-overlap measurement mode only changes when loads are awaited."""
    p = Problem(8192, 4, ra.SPLIT_ZIGZAG, 1, 4, 1, 128, "bf16", seed=17)
    for r in (0, 3):
        say(f"sync loads rank {r}")
        o1, l1, s1 = p.run(r)
        o2, l2, s2 = p.run(r, flags=ra.FLAG_SYNC_LOADS, fill=0.0)
        assert torch.equal(o1, o2) and torch.equal(l1, l2) and torch.equal(s1, s2)


# ---------------------------------------------------------------- partial results and merge

@pytest.mark.parametrize("dtype,split", [("bf16", ra.SPLIT_ZIGZAG), ("f32", ra.SPLIT_CONTIGUOUS), ("bf16", ra.SPLIT_CONTIGUOUS)])
def test_partials_merge_to_full(dtype, split):
    S, c = 1024, 4
    d = 128 if dtype == "bf16" else 64
    p = Problem(S, c, split, 1, 4, 2, d, dtype, seed=21)
    tol = TOL[dtype]
    for r in (0, 2, 3):
        say(f"partials dtype={dtype} split={split} rank {r}")
        fused_o, fused_l, _ = p.run(r)
        acc_o, acc_l = None, None
        for t, j in enumerate(p.ring_owners(r)):
            po, pl, _ = p.run(r, owners=[j], fill=float("nan"))
            ref_o, ref_l = p.reference(r, owners=[j])
            compare(po, pl, ref_o, ref_l, tol=tol)   # includes rows that see no key: (0, -inf)
            if acc_o is None:
                acc_o, acc_l = po.clone(), pl.clone()
            else:
                ra.ring_attn_merge(p.B, p.Hq, p.n_loc, p.d, [acc_o, po], ra.F32, [acc_l, pl], acc_o, ra.F32, acc_l)
        torch.cuda.synchronize()
        ref_o, ref_l = p.reference(r)
        compare(acc_o, acc_l, ref_o, ref_l, tol=tol)
        assert (acc_o - fused_o).abs().max().item() <= 2 * tol[0]


def test_dropped_block_then_recovered():
    p = Problem(2048, 4, ra.SPLIT_ZIGZAG, 1, 4, 1, 128, "bf16", seed=5)
    r = 3
    owners = p.ring_owners(r)
    kept, dropped = owners[:2] + owners[3:], owners[2]
    say("dropped block")
    out, lse, _ = p.run(r, owners=kept)
    ref_o, ref_l = p.reference(r, owners=kept)
    compare(out, lse, ref_o, ref_l, tol=TOL["bf16"])
    po, pl, _ = p.run(r, owners=[dropped])
    ra.ring_attn_merge(p.B, p.Hq, p.n_loc, p.d, [out, po], ra.F32, [lse, pl], out, ra.F32, lse)
    torch.cuda.synchronize()
    ref_o, ref_l = p.reference(r)
    compare(out, lse, ref_o, ref_l, tol=TOL["bf16"])


def test_reverse_visit_order():
    p = Problem(2048, 4, ra.SPLIT_ZIGZAG, 1, 2, 1, 128, "bf16", seed=8)
    for r in range(4):
        say(f"reverse order rank {r}")
        out, lse, _ = p.run(r, owners=p.ring_owners(r)[::-1])
        ref_o, ref_l = p.reference(r)
        compare(out, lse, ref_o, ref_l, tol=TOL["bf16"])


@pytest.mark.parametrize("parts_dtype,out_dtype,n_parts", [
    (ra.F32, ra.F32, 2), (ra.F32, ra.F32, 5), (ra.BF16, ra.F32, 3), (ra.F32, ra.BF16, 4), (ra.BF16, ra.BF16, 1),
])
def test_merge_kernel_vs_oracle(parts_dtype, out_dtype, n_parts):
    say(f"merge parts={parts_dtype} out={out_dtype} n={n_parts}")
    B, H, rows, d = 2, 3, 77, 128
    g = np.random.default_rng(n_parts)
    outs = g.standard_normal((n_parts, B, H, rows, d)).astype(np.float32)
    lses = (g.standard_normal((n_parts, B, H, rows)) * 3).astype(np.float32)
    lses[:, :, :, 5] = -np.inf                  # a row with no keys in any part
    lses[0, :, :, 6] = -np.inf                  # a row empty in part 0 only
    outs[0, :, :, 6] = 0.0
    tdt = torch.float32 if parts_dtype == ra.F32 else torch.bfloat16
    d_outs = [torch.from_numpy(outs[k]).to(DEV).to(tdt) for k in range(n_parts)]
    host_outs = np.stack([t.float().cpu().numpy() for t in d_outs])
    d_lses = [torch.from_numpy(lses[k]).to(DEV) for k in range(n_parts)]
    odt = torch.float32 if out_dtype == ra.F32 else torch.bfloat16
    out = torch.full((B, H, rows, d), float("nan"), dtype=odt, device=DEV)
    lse = torch.full((B, H, rows), float("nan"), dtype=torch.float32, device=DEV)
    ra.ring_attn_merge(B, H, rows, d, d_outs, parts_dtype, d_lses, out, out_dtype, lse)
    torch.cuda.synchronize()
    ref_o, ref_l = oracle.merge(host_outs.astype(np.float64), lses.astype(np.float64))
    o = out.float().cpu().numpy()
    tol = 1e-5 if out_dtype == ra.F32 else 1e-2
    assert np.abs(o - ref_o).max() <= tol + (0 if out_dtype == ra.F32 else 2.0 ** -8 * np.abs(ref_o).max())
    l = lse.cpu().numpy()
    assert np.array_equal(np.isneginf(l), np.isneginf(ref_l))
    fin = np.isfinite(ref_l)
    assert np.abs(l[fin] - ref_l[fin]).max() <= 1e-5
    assert np.all(o[:, :, 5] == 0.0)


def test_merge_in_place_and_identity():
    say("merge in place")
    B, H, rows, d = 1, 2, 64, 64
    g = np.random.default_rng(1)
    a = torch.from_numpy(g.standard_normal((B, H, rows, d)).astype(np.float32)).to(DEV)
    la = torch.from_numpy(g.standard_normal((B, H, rows)).astype(np.float32)).to(DEV)
    empty_o = torch.zeros_like(a)
    empty_l = torch.full_like(la, float("-inf"))
    a0, la0 = a.clone(), la.clone()
    ra.ring_attn_merge(B, H, rows, d, [a, empty_o], ra.F32, [la, empty_l], a, ra.F32, la)
    torch.cuda.synchronize()
    # merging a part with no keys changes nothing (up to the exp(0) * x / 1 round trip)
    assert (a - a0).abs().max().item() <= 1e-6 and (la - la0).abs().max().item() <= 1e-6


@pytest.mark.parametrize("d", [128, 64])
@pytest.mark.parametrize("c", [1, 2])
@pytest.mark.parametrize("causal", [True, False], ids=["causal", "full"])
def test_pipeline_ends_at_every_step(d, c, causal):
    """Shard lengths 32 .. 672 (1 .. 21 visible 32-key tiles per block and one
    or two query tiles per workgroup): the tile pipeline, unrolled over twenty
    steps (ten LDS stages, two score buffers, a barrier every four steps) with
    K fragments read a step ahead, ends at every position of its unrolled
    loop.  Every row of every rank against the oracle, and the work
    counters."""
    for n_loc in range(32, 673, 32):
        S = n_loc * c
        p = Problem(S, c, ra.SPLIT_CONTIGUOUS, 1, 2, 1, d, "bf16", seed=S + c + d)
        tq, tk = ra.ring_attn_tile_shape(p.desc(causal=causal))
        for r in range(c):
            say(f"pipeline end: d {d} c {c} causal {causal} n_loc {n_loc} rank {r}")
            out, lse, stats = p.run(r, causal=causal)
            ref_o, ref_l = p.reference(r, causal=causal)
            compare(out, lse, ref_o, ref_l, tol=TOL["bf16"])
            assert stats.cpu().tolist() == expected_stats(p, r, tq, tk, causal), f"stats n_loc {n_loc} rank {r}"


def test_half_million_token_shard_sampled():
    """A 524 288-token shard (1 048 576 tokens, c = 2 zig-zag, one head, d =
    128): key-tile offsets inside a block reach 2^27 bytes and a query row
    sees up to a million keys.  Both ranks; chunk edges plus 56 uniform rows
    of each against the oracle over their full visible key sets; the pair
    counter exact (the oracle's per-shard pair count), and the tile classes
    covering every (query tile, key tile, block) once (enumerating the
    classes pair by pair is out of reach at this size)."""
    S, c = 1 << 20, 2
    p = Problem(S, c, ra.SPLIT_ZIGZAG, 1, 1, 1, 128, "bf16", seed=77)
    tq, tk = ra.ring_attn_tile_shape(p.desc())
    pairs = oracle.pair_counts(S, c, oracle.SPLIT_ZIGZAG)
    n_tiles = -(-p.n_loc // tq) * -(-p.n_loc // tk) * c
    for r in range(c):
        say(f"half-million-token shard rank {r}")
        out, lse, stats = p.run(r)
        rows = workloads.sample_rows(p.n_loc, p.n_loc // 2, 56, 500 + r)
        ref_o, ref_l = p.reference(r, rows=rows)
        compare(out, lse, ref_o, ref_l, rows=rows, tol=TOL["bf16"])
        st = stats.cpu().tolist()
        assert st[0] == int(pairs[r]), f"pairs rank {r}: {st[0]} vs {int(pairs[r])}"
        assert st[1] + st[2] + st[3] == n_tiles and st[2] > 0, f"tile classes rank {r}: {st}"
        del out, lse, stats
        torch.cuda.empty_cache()
