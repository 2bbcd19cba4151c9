"""Property-based pins of the fp64 oracle (CPU, no GPU): random shapes drawn
by hypothesis, each checked against something other than the oracle itself
-- the pure-Python brute force, the placement rules restated from the pages,
and the exactness of blockwise folding ("Sequence / context parallelism"
notes, section 4: the final answer is exact)."""
import math

import numpy as np
from hypothesis import given, settings, strategies as st

import oracle
from oracle import tiny

SPLITS = [oracle.SPLIT_CONTIGUOUS, oracle.SPLIT_ZIGZAG, oracle.SPLIT_STRIPED]
PROP = settings(max_examples=40, deadline=None)


@st.composite
def placements(draw, max_chunk=24, max_c=8):
    split = draw(st.sampled_from(SPLITS))
    c = draw(st.integers(1, max_c))
    n = draw(st.integers(1, max_chunk))  # chunk length (zig-zag) or shard length
    S = 2 * c * n if split == oracle.SPLIT_ZIGZAG else c * n
    return S, c, split


@st.composite
def attention_inputs(draw, max_S=12, max_d=6):
    B = draw(st.integers(1, 2))
    h_kv = draw(st.integers(1, 2))
    g = draw(st.integers(1, 3))
    S = draw(st.integers(1, max_S))
    d = draw(st.integers(1, max_d))
    sigma = draw(st.sampled_from([0.3, 1.0, 2.0]))
    seed = draw(st.integers(0, 2**31 - 1))
    rng = np.random.default_rng(seed)
    q = rng.standard_normal((B, h_kv * g, S, d)) * sigma
    k = rng.standard_normal((B, h_kv, S, d)) * sigma
    v = rng.standard_normal((B, h_kv, S, d))
    return q, k, v, 1.0 / math.sqrt(d), draw(st.booleans())


@PROP
@given(attention_inputs())
def test_oracle_matches_pure_python_brute_force(case):
    q, k, v, scale, causal = case
    out, lse = oracle.attention(q, k, v, scale, causal)
    t_out, t_lse = tiny.attention(q.tolist(), k.tolist(), v.tolist(), scale, causal)
    assert np.max(np.abs(out - np.array(t_out))) <= 1e-12
    assert np.max(np.abs(lse - np.array(t_lse))) <= 1e-12


def _positions_by_rule(S, c, split, r):
    """Shard r's global positions restated from the placement rules: a
    contiguous run; chunks r and 2c-1-r of 2c; or every c-th token."""
    n_loc = S // c
    if split == oracle.SPLIT_CONTIGUOUS:
        return list(range(r * n_loc, (r + 1) * n_loc))
    if split == oracle.SPLIT_ZIGZAG:
        n = S // (2 * c)
        return list(range(r * n, (r + 1) * n)) + list(range((2 * c - 1 - r) * n, (2 * c - r) * n))
    return list(range(r, S, c))


@PROP
@given(placements())
def test_partition_follows_the_placement_rules(pl):
    S, c, split = pl
    perm = oracle.partition_perm(S, c, split)
    assert sorted(perm.tolist()) == list(range(S))
    n_loc = S // c
    for r in range(c):
        assert perm[r * n_loc:(r + 1) * n_loc].tolist() == _positions_by_rule(S, c, split, r)


@PROP
@given(placements(), st.booleans())
def test_pair_counts_by_enumeration_and_zigzag_balance(pl, causal):
    S, c, split = pl
    got = oracle.pair_counts(S, c, split, causal)
    n_loc = S // c
    for r in range(c):
        pos = _positions_by_rule(S, c, split, r)
        assert got[r] == sum((p + 1) if causal else S for p in pos)
    if split == oracle.SPLIT_ZIGZAG and causal:
        n = S // (2 * c)
        assert set(got.tolist()) == {n * n * (2 * c - 1) + n * (n + 1)}


@PROP
@given(attention_inputs(max_S=20, max_d=5), st.integers(1, 6), st.integers(0, 2**31 - 1))
def test_blockwise_fold_and_merge_equal_full_attention(case, n_blocks, seed):
    """Keys cut into random blocks visited in random order: the online fold
    and the merge of per-block partials both equal attention over all keys."""
    q, k, v, scale, causal = case
    S = k.shape[2]
    rng = np.random.default_rng(seed)
    order = rng.permutation(S)
    cuts = np.sort(rng.choice(np.arange(1, S), size=min(n_blocks, S) - 1, replace=False)) if S > 1 else []
    blocks = [np.sort(b) for b in np.split(order, cuts)]
    full_o, full_l = oracle.attention(q, k, v, scale, causal)
    outs, lses = zip(*[oracle.attention(q, k, v, scale, causal, keys=b) for b in blocks])
    mo, ml = oracle.merge(list(outs), list(lses))
    assert np.max(np.abs(mo - full_o)) <= 1e-12
    fin = np.isfinite(full_l)
    assert np.array_equal(np.isneginf(ml), ~fin) and np.max(np.abs(ml[fin] - full_l[fin]), initial=0.0) <= 1e-12
    perm = rng.permutation(len(blocks))
    po, pl_ = oracle.merge([outs[i] for i in perm], [lses[i] for i in perm])
    assert np.max(np.abs(po - mo)) <= 1e-12
    h = int(rng.integers(0, q.shape[1]))
    hk = h // (q.shape[1] // k.shape[1])
    bo, bl = oracle.blockwise_online(q[0, h], k[0, hk], v[0, hk], scale, causal, np.arange(S), blocks)
    assert np.max(np.abs(bo - full_o[0, h])) <= 1e-12
    assert np.max(np.abs(bl[fin[0, h]] - full_l[0, h][fin[0, h]]), initial=0.0) <= 1e-12
