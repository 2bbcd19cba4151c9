"""GPU parity on seeded random configurations: shard lengths 1 .. 700, the
three placements, 1 .. 6 shards, batch 1 or 2, GQA groups 1 .. 5 over 1 .. 3
key/value heads, d = 64 or 128, bf16 (fp32 or bf16 output) and fp32, causal
and bidirectional, ring-ordered or a random subset of the blocks in random
order.  Every row of the chosen rank against the oracle restricted to the
visited blocks' keys, and the work counters bit-exact."""
import numpy as np
import pytest

import ring_parallelism_amd as ra
from gpu_util import TOL, Problem, compare, expected_stats, say

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
