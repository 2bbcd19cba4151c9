"""GPU parity where later key blocks score far higher than earlier ones: the
online softmax must rescale what it has already folded when the running max
rises ("Sequence Parallelism and Ring Attention Quiz", Q3 and Q7; the notes,
section 4).  Inputs are built so that, for the rank under test, every block
the ring delivers scores higher than the one before by tens of log2 units;
the event counters prove that the kernel's reference raise (and, for a jump
no exponential can absorb, its exact per-tile path) actually ran."""
import numpy as np
import pytest

import oracle
import ring_parallelism_amd as ra
from gpu_util import TOL, Problem, compare, say

pytestmark = pytest.mark.gpu

LOG2E = 1.4426950408889634


def rising_problem(S, c, split, Hq, Hkv, d, rank, step_log2, last_extra_log2=0.0, seed=7,
                   boosted_queries=None):
    """Q, K, V ~ N(0, 1) plus a shared direction: q[., 0] += a for every
    query (or for the natural positions in `boosted_queries`) and
    k[., 0] += b_t for the keys of the block the ring delivers at step t to
    `rank`, with a * b_t * scale * log2(e) = t * step_log2 (+ an extra jump on
    the last block).  So the score of a key visited at step t exceeds those of
    step 0 by about t * step_log2 log2 units for a boosted query."""
    g = np.random.default_rng(seed)
    q = g.standard_normal((1, Hq, S, d), dtype=np.float32)
    k = g.standard_normal((1, Hkv, S, d), dtype=np.float32)
    v = g.standard_normal((1, Hkv, S, d), dtype=np.float32)
    scale = d ** -0.5
    a = 16.0
    n_loc = S // c
    pm = oracle.partition_perm(S, c, split)
    owner = np.empty(S, dtype=np.int64)
    owner[pm] = np.arange(S) // n_loc
    t = (rank - owner) % c
    b = t * step_log2 / (a * scale * LOG2E)
    b = b + (t == c - 1) * last_extra_log2 / (a * scale * LOG2E)
    if boosted_queries is None:
        q[..., 0] += a
    else:
        q[..., boosted_queries, 0] += a
    k[..., 0] += b[None, None, :].astype(np.float32)
    return Problem(S, c, split, 1, Hq, Hkv, d, "bf16", arrays=(q, k, v))


@pytest.mark.parametrize("d", [64, 128])
@pytest.mark.parametrize("causal", [True, False], ids=["causal", "bidirectional"])
@pytest.mark.parametrize("out_dtype", [ra.F32, ra.BF16], ids=["f32out", "bf16out"])
def test_rising_scores_raise_the_reference(d, causal, out_dtype):
    """Blocks rising 40 log2 units per ring step: every row that sees a later
    block must raise its reference mid-pass; every row matches the oracle."""
    S, c, split, Hq, Hkv = 1024, 4, ra.SPLIT_ZIGZAG, 4, 2
    raises = 0
    for r in range(c):
        p = rising_problem(S, c, split, Hq, Hkv, d, r, step_log2=40.0)
        say(f"rising d={d} causal={causal} out={out_dtype} rank {r}")
        out, lse, st = p.run(r, out_dtype=out_dtype, causal=causal, flags=ra.FLAG_EVENT_COUNTS)
        ref_o, ref_l = p.reference(r, causal=causal)
        compare(out, lse, ref_o, ref_l, tol=TOL["bf16"], bf16_out=out_dtype == ra.BF16)
        st = st.cpu().tolist()
        assert st[5] == 0, "no exponential may leave the fp32 range at 40 log2 units per block"
        raises += st[4]
    # Rows see at least one later block in every rank but the causal case's
    # first rows; with bidirectional attention every row sees all blocks.
    assert raises > 0, "the reference raise never ran"
    if not causal:
        assert raises >= S * Hq, f"{raises} raises for {S * Hq} rows"


@pytest.mark.parametrize("causal", [True, False], ids=["causal", "bidirectional"])
def test_jump_beyond_fp32_range_takes_exact_path(causal):
    """The last block scores 200 log2 units above the one before: its
    exponentials overflow against the running reference, the query tiles that
    see it are recomputed by the plain per-tile online softmax, and the result
    still matches the oracle."""
    S, c, split, Hq, Hkv, d = 1024, 4, ra.SPLIT_ZIGZAG, 2, 1, 128
    exact = 0
    for r in range(c):
        p = rising_problem(S, c, split, Hq, Hkv, d, r, step_log2=5.0, last_extra_log2=200.0, seed=11)
        say(f"overflow jump causal={causal} rank {r}")
        out, lse, st = p.run(r, causal=causal, flags=ra.FLAG_EVENT_COUNTS)
        ref_o, ref_l = p.reference(r, causal=causal)
        compare(out, lse, ref_o, ref_l, tol=TOL["bf16"])
        exact += st.cpu().tolist()[5]
    assert exact > 0, "the exact per-tile path never ran"


@pytest.mark.parametrize("d", [64, 128])
@pytest.mark.parametrize("order", ["fast_then_exact", "exact_then_fast"])
def test_exact_path_beside_a_fast_tile_in_one_workgroup(d, order):
    """4 096 tokens over 4 shards: four 256-row query tiles per (head, shard),
    two per workgroup (tiles p and 3 - p, the first from the first half of the
    sequence).  Only the query tiles that meet the 200-log2-unit jump of the
    last block overflow, so a workgroup recomputes one of its tiles by the
    exact path and runs the other on the fast path.  Causal with every query
    boosted: the second tile (later positions) is the one that sees the jump.
    Bidirectional with only first-half queries boosted: the first tile is
    recomputed and the next tile's first loads follow its exact pass.  Every
    row must match the oracle, and the exact path must run for exactly the
    tiles that overflow."""
    S, c, split, Hq, Hkv = 4096, 4, ra.SPLIT_ZIGZAG, 2, 1
    causal = order == "fast_then_exact"
    boosted = None if causal else np.arange(S // 2)
    exact, tiles = 0, 0
    for r in range(c):
        p = rising_problem(S, c, split, Hq, Hkv, d, r, step_log2=5.0, last_extra_log2=200.0, seed=13,
                           boosted_queries=boosted)
        say(f"exact beside fast d={d} {order} rank {r}")
        out, lse, st = p.run(r, causal=causal, flags=ra.FLAG_EVENT_COUNTS)
        ref_o, ref_l = p.reference(r, causal=causal)
        compare(out, lse, ref_o, ref_l, tol=TOL["bf16"])
        exact += st.cpu().tolist()[5]
        tiles += Hq * (p.n_loc // ra.ring_attn_tile_shape(p.desc())[0])
    assert 0 < exact < tiles, f"{exact} of {tiles} query tiles took the exact path"
    if not causal:
        # Every first-half tile (boosted) overflows; no second-half tile does.
        assert exact == tiles // 2, f"{exact} of {tiles} query tiles took the exact path"


def test_event_counts_are_zero_on_the_benchmark_distribution():
    """N(0, 1) inputs: scores stay within a few log2 units of the first tile's
    max, so neither the raise nor the exact path runs (the fast path is what
    the benchmark times)."""
    p = Problem(4096, 4, ra.SPLIT_ZIGZAG, 1, 4, 1, 128, "bf16", seed=5)
    for r in range(p.c):
        out, lse, st = p.run(r, flags=ra.FLAG_EVENT_COUNTS)
        assert st.cpu().tolist()[4:] == [0, 0]


@pytest.mark.parametrize("d", [64, 128])
def test_ragged_block_ends_before_nan_guard(d):
    """Shards of 250 tokens (the last key tile of a block is 26 rows long):
    each key/value block is the start of a buffer whose following rows are NaN.
    Rows past the block must read as zeros (the buffer range check), so the
    output stays finite and matches the oracle."""
    import torch
    from gpu_util import DEV
    S, c, split, Hq, Hkv = 1000, 4, ra.SPLIT_CONTIGUOUS, 2, 1
    p = Problem(S, c, split, 1, Hq, Hkv, d, "bf16", seed=3)
    n = p.n_loc
    guarded_k, guarded_v = [], []
    for j in range(c):
        for src, dst in ((p.ks[j], guarded_k), (p.vs[j], guarded_v)):
            buf = torch.full((1, Hkv, n + 64, d), float("nan"), dtype=torch.bfloat16, device=DEV)
            buf[:, :, :n] = src
            flat = buf.reshape(-1)
            blk = flat[: Hkv * n * d].view(1, Hkv, n, d)   # Hkv = 1: the block, then NaN rows
            dst.append((blk, buf))
    torch.cuda.synchronize()
    for r in range(c):
        owners = p.ring_owners(r)
        out = torch.full((1, Hq, n, d), float("nan"), dtype=torch.float32, device=DEV)
        lse = torch.full((1, Hq, n), float("nan"), dtype=torch.float32, device=DEV)
        ra.ring_attn_shard_fwd(p.desc(), r, p.qs[r], [guarded_k[j][0] for j in owners],
                               [guarded_v[j][0] for j in owners], out, lse, block_owner=owners)
        torch.cuda.synchronize()
        ref_o, ref_l = p.reference(r)
        compare(out, lse, ref_o, ref_l, tol=TOL["bf16"])
