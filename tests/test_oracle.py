"""CPU tests that pin the fp64 oracle (no GPU)."""
import json
import os
from fractions import Fraction

import numpy as np
import pytest

import oracle
import pins

GOLDEN = os.path.join(os.path.dirname(__file__), "golden", "pages_printed_values.json")


@pytest.fixture(scope="module")
def golden():
    with open(GOLDEN) as f:
        return json.load(f)


@pytest.mark.parametrize("pin", pins.ALL_PINS, ids=lambda p: p.__name__)
def test_attention_pins(oracle_lib, pin):
    pin(oracle_lib)


# ---------------------------------------------------------------- partition

@pytest.mark.parametrize("split", [oracle.SPLIT_CONTIGUOUS, oracle.SPLIT_ZIGZAG, oracle.SPLIT_STRIPED])
@pytest.mark.parametrize("S,c", [(16, 1), (64, 4), (96, 3), (1024, 8), (4096, 16)])
def test_partition_is_bijection(split, S, c):
    if split == oracle.SPLIT_ZIGZAG and S % (2 * c):
        pytest.skip("not divisible")
    perm = oracle.partition_perm(S, c, split)
    assert perm.dtype == np.int64 and perm.shape == (S,)
    assert np.array_equal(np.sort(perm), np.arange(S))
    # within a shard, token positions ascend
    n_loc = S // c
    assert np.all(np.diff(perm.reshape(c, n_loc), axis=1) > 0)


def test_partition_identity_cases():
    assert np.array_equal(oracle.partition_perm(1000, 4, oracle.SPLIT_CONTIGUOUS), np.arange(1000))
    for split in (oracle.SPLIT_CONTIGUOUS, oracle.SPLIT_STRIPED):
        assert np.array_equal(oracle.partition_perm(77, 1, split), np.arange(77))
    # c = 1 zig-zag: chunks 0 and 1 of 2, i.e. the whole sequence in order
    assert np.array_equal(oracle.partition_perm(64, 1, oracle.SPLIT_ZIGZAG), np.arange(64))


def test_partition_pages_examples(golden):
    S, c = 32768, 4
    perm = oracle.partition_perm(S, c, oracle.SPLIT_CONTIGUOUS)
    for r, (lo, hi) in enumerate(golden["contiguous_tokens_c4_s32k"]["value"]):
        assert np.array_equal(perm[r * (S // c):(r + 1) * (S // c)], np.arange(lo, hi))
    n = 8
    perm = oracle.partition_perm(2 * 4 * n, 4, oracle.SPLIT_ZIGZAG)
    for r, chunks in enumerate(golden["zigzag_chunks_c4"]["value"]):
        got = perm[r * 2 * n:(r + 1) * 2 * n]
        want = np.concatenate([np.arange(ch * n, (ch + 1) * n) for ch in chunks])
        assert np.array_equal(got, want)


def test_partition_striped_round_robin():
    perm = oracle.partition_perm(12, 3, oracle.SPLIT_STRIPED)
    assert perm.tolist() == [0, 3, 6, 9, 1, 4, 7, 10, 2, 5, 8, 11]


def test_partition_rejects_bad_sizes():
    with pytest.raises(ValueError):
        oracle.partition_perm(100, 3, oracle.SPLIT_CONTIGUOUS)
    with pytest.raises(ValueError):
        oracle.partition_perm(100, 8, oracle.SPLIT_ZIGZAG)


# ---------------------------------------------------------------- work counts

@pytest.mark.parametrize("split", [oracle.SPLIT_CONTIGUOUS, oracle.SPLIT_ZIGZAG, oracle.SPLIT_STRIPED])
@pytest.mark.parametrize("S,c", [(8, 1), (24, 3), (32, 4), (48, 2), (64, 8)])
@pytest.mark.parametrize("causal", [True, False])
def test_pair_counts_brute_force(split, S, c, causal):
    if split == oracle.SPLIT_ZIGZAG and S % (2 * c):
        pytest.skip("not divisible")
    assert oracle.pair_counts(S, c, split, causal).tolist() == oracle.pair_counts_brute(S, c, split, causal)


@pytest.mark.parametrize("S,c", [(1024, 4), (8192, 8), (32768, 16), (131072, 16), (262144, 32), (4096, 64)])
def test_pair_counts_closed_forms(S, c):
    cont = oracle.pair_counts(S, c, oracle.SPLIT_CONTIGUOUS)
    n = S // c
    want = [r * n * n + n * (n + 1) // 2 for r in range(c)]
    assert cont.tolist() == want
    zz = oracle.pair_counts(S, c, oracle.SPLIT_ZIGZAG)
    n = S // (2 * c)
    assert zz.tolist() == [n * n * (2 * c - 1) + n * (n + 1)] * c
    assert int(cont.sum()) == int(zz.sum()) == S * (S + 1) // 2


def test_busiest_over_average_matches_pages(golden):
    g = golden["contiguous_busiest_over_average_c16"]
    S, c = g["seq_len"], g["n_shards"]
    cont = oracle.pair_counts(S, c, oracle.SPLIT_CONTIGUOUS)
    ratio = Fraction(int(cont.max()) * c, int(cont.sum()))
    n = S // c
    assert ratio == Fraction(2 * n * c - n + 1, c * n + 1)       # exact closed form
    assert round(float(ratio), g["printed_digits"]) == g["value"]  # the printed 1.94
    assert abs(float(ratio) - (2 * c - 1) / c) < 1e-4              # its large-S limit
    zz = oracle.pair_counts(S, c, oracle.SPLIT_ZIGZAG)
    assert golden["zigzag_work_equal"]["value"] and len(set(zz.tolist())) == 1


def test_contiguous_later_shards_do_more(golden):
    assert golden["later_tokens_more_work"]["value"]
    for S, c in [(1024, 4), (32768, 16)]:
        cont = oracle.pair_counts(S, c, oracle.SPLIT_CONTIGUOUS)
        assert np.all(np.diff(cont) > 0)


def test_block_granular_last_over_first_is_c(golden):
    assert golden["contiguous_last_over_first_blocks"]["value"] == "N"
    for S, c in [(64, 4), (1024, 8), (4096, 16)]:
        blk = oracle.block_pair_counts(S, c, oracle.SPLIT_CONTIGUOUS)
        assert blk[0] == 1 and blk[-1] == c
        assert np.all(oracle.block_pair_counts(S, c, oracle.SPLIT_CONTIGUOUS, causal=False) == c)


@pytest.mark.parametrize("split", [oracle.SPLIT_CONTIGUOUS, oracle.SPLIT_ZIGZAG])
def test_tile_counts_consistent(split):
    S, c = 1000 if split == oracle.SPLIT_CONTIGUOUS else 1040, 4
    for causal in (True, False):
        for r in range(c):
            t = oracle.tile_counts(S, c, split, causal, r, 64, 32)
            assert t["pairs"] == oracle.pair_counts(S, c, split, causal)[r]
            n_loc = S // c
            assert t["full"] + t["partial"] + t["skipped"] == c * (-(-n_loc // 64)) * (-(-n_loc // 32))


def test_tile_counts_large_shard():
    # 131 072 tokens, c = 16 zig-zag, 128 x 64 tiles: per head the diagonal
    # chunk pairs give 2 x 64 partial tiles, the rest split evenly.
    t = oracle.tile_counts(131072, 16, oracle.SPLIT_ZIGZAG, True, 5, 128, 64)
    assert t == dict(pairs=536875008, full=65472, partial=128, skipped=65472)
