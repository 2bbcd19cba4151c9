"""ring_attn_shard_fwd_split_noalloc (the split shard pass with its partials in
the library's static device scratch) against ring_attn_shard_fwd_split with a
caller workspace: the same kernels on the same inputs, so the results must be
identical bit for bit -- on two calls in a row, the second smaller than the
first (the scratch keeps the first call's contents) -- and both within the
bf16 bound of the oracle."""
import numpy as np
import pytest
import torch

import ring_parallelism_amd as ra
from gpu_util import DEV, TOL, Problem, compare, say

pytestmark = pytest.mark.gpu


def _split_pair(p, rank, n_splits, out_dtype):
    owners = p.ring_owners(rank)
    kb, vb = [p.ks[j] for j in owners], [p.vs[j] for j in owners]
    odt = torch.float32 if out_dtype == ra.F32 else torch.bfloat16
    desc = p.desc(out_dtype)
    o_ws = torch.full((p.B, p.Hq, p.n_loc, p.d), float("nan"), dtype=odt, device=DEV)
    l_ws = torch.full((p.B, p.Hq, p.n_loc), float("nan"), dtype=torch.float32, device=DEV)
    work = torch.empty((n_splits, p.B, p.Hq, p.n_loc, p.d), dtype=torch.float32, device=DEV)
    work_l = torch.empty((n_splits, p.B, p.Hq, p.n_loc), dtype=torch.float32, device=DEV)
    s_ws = torch.zeros(4, dtype=torch.int64, device=DEV)
    ra.ring_attn_shard_fwd_split(desc, rank, p.qs[rank], kb, vb, n_splits, work, work_l, o_ws, l_ws,
                                 block_owner=owners, stats=s_ws)
    o_na = torch.full_like(o_ws, float("nan"))
    l_na = torch.full_like(l_ws, float("nan"))
    s_na = torch.zeros(4, dtype=torch.int64, device=DEV)
    ra.ring_attn_shard_fwd_split_noalloc(desc, rank, p.qs[rank], kb, vb, n_splits, o_na, l_na, block_owner=owners,
                                         stats=s_na)
    torch.cuda.synchronize()
    return (o_ws, l_ws, s_ws), (o_na, l_na, s_na)


def test_noalloc_split_matches_workspace_split_twice():
    # First call: the 8 192-token shape (c = 8, 32 / 8 heads), 4 groups -- the
    # whole scratch.  Second call: a smaller shard (256 rows, 4 / 1 heads),
    # 2 groups, so stale partials of the first call sit beyond its rows.
    big = Problem(8192, 8, ra.SPLIT_ZIGZAG, 1, 32, 8, 128, "bf16", seed=21)
    small = Problem(1024, 4, ra.SPLIT_ZIGZAG, 1, 4, 1, 128, "bf16", seed=22)
    for p, rank, n_splits, out_dtype in ((big, 3, 4, ra.BF16), (small, 1, 2, ra.F32)):
        say(f"noalloc split S={p.S} c={p.c} h={p.Hq}x{p.Hkv} rank {rank} splits {n_splits}")
        (o_ws, l_ws, s_ws), (o_na, l_na, s_na) = _split_pair(p, rank, n_splits, out_dtype)
        assert torch.equal(o_ws, o_na) and torch.equal(l_ws, l_na) and torch.equal(s_ws, s_na)
        heads = np.arange(0, p.Hq, max(1, p.Hq // 8))
        ref_o, ref_l = p.reference(rank, heads=heads)
        compare(o_na, l_na, ref_o, ref_l, heads=heads, tol=TOL["bf16"], bf16_out=out_dtype == ra.BF16)


def test_noalloc_rejects_sizes_beyond_the_scratch():
    p = Problem(8192, 8, ra.SPLIT_ZIGZAG, 1, 32, 8, 128, "bf16", seed=23)
    owners = p.ring_owners(0)
    out = torch.empty((p.B, p.Hq, p.n_loc, p.d), dtype=torch.float32, device=DEV)
    lse = torch.empty((p.B, p.Hq, p.n_loc), dtype=torch.float32, device=DEV)
    with pytest.raises(ra.RingAttnError, match="static scratch"):
        ra.ring_attn_shard_fwd_split_noalloc(p.desc(), 0, p.qs[0], [p.ks[j] for j in owners],
                                             [p.vs[j] for j in owners], 8, out, lse, block_owner=owners)
