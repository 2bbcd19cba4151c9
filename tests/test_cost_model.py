"""The pages' modelled figures reproduced from the cost model in ``oracle``.

Each printed number is compared at the precision it is printed with; every
term of the model moves at least one of them off its printed value (the
(c - 1)/c factor, the causal half, the KV heads per device, the layers per
stage, the 10**6 tokens of "1M").
"""
import json
import os

import pytest

import oracle
from oracle import cost_model as cm

GOLDEN = os.path.join(os.path.dirname(__file__), "golden", "pages_printed_values.json")


@pytest.fixture(scope="module")
def golden():
    with open(GOLDEN) as f:
        return json.load(f)


def printed(g, x):
    """True when x rounds to the printed value at the printed precision."""
    return round(x, g["decimals"]) == g["value"]


M = cm.LLAMA3_405B
T, P = 8, 16


def test_ring_transfer_over_attention_time(golden):
    g = golden["kv_transfer_over_attention_pct"]
    r = cm.transfer_over_compute(M, g["seq_len"], T, g["n_shards"], cm.gbit_per_s(400),
                                 0.45 * cm.H100_BF16_DENSE_FLOPS)
    assert printed(g, 100 * r["ratio"])
    # Both terms by hand: 16 query heads and 1 KV head per device under t = 8.
    S, c, d = 131072, 16, 128
    assert r["bytes"] == 2 * S * 1 * d * 2 * (c - 1) / c == 62914560
    assert r["flop"] == 4 * d * 16 * (S * (S + 1) // 2) // c
    assert r["flop"] == 4398080065536


def test_ratio_terms_each_matter(golden):
    """Plausible slips in the model miss the printed 12.7 %."""
    g = golden["kv_transfer_over_attention_pct"]
    r = cm.transfer_over_compute(M, 131072, T, 16, cm.gbit_per_s(400), 0.45 * cm.H100_BF16_DENSE_FLOPS)
    slips = {
        "whole share sent": r["ratio"] * 16 / 15,
        "no causal half": r["ratio"] / 2,
        "GB/s taken for Gb/s": r["ratio"] / 8,
        "all 8 KV heads": r["ratio"] * 8,
        "2 FLOP per pair": r["ratio"] * 2,
    }
    for name, x in slips.items():
        assert not printed(g, 100 * x), name


def test_attention_flop_is_the_shard_pass_workload():
    """The busiest device's causal work at 131 072 tokens, c = 16 equals the
    FLOP the shard pass counts for its 16-head, d = 128 shard (zig-zag: every
    device equal; contiguous: the last device does more)."""
    zz = oracle.pair_counts(131072, 16, oracle.SPLIT_ZIGZAG)
    assert len(set(zz.tolist())) == 1
    assert cm.attention_flop_per_layer(M, 131072, T, 16) == 4 * 128 * 16 * int(zz[0])
    contiguous = cm.attention_flop_per_layer(M, 131072, T, 16, oracle.SPLIT_CONTIGUOUS)
    assert contiguous > cm.attention_flop_per_layer(M, 131072, T, 16)


def test_activation_memory(golden):
    assert printed(golden["activations_s131072_t8_p16_GB"], cm.activation_bytes_per_device(M, 131072, T, P) / 1e9)
    assert printed(golden["activations_s131072_t8_p16_c16_GB"],
                   cm.activation_bytes_per_device(M, 131072, T, P, cp=16) / 1e9)
    assert printed(golden["activations_s8192_t8_p16_GB"], cm.activation_bytes_per_device(M, 8192, T, P) / 1e9)
    assert round(M.layers / P) == golden["layers_per_stage_p16"]["value"]
    # A whole layer count per stage (8 rather than 126/16) would miss 71.9.
    assert round(34 * 131072 * M.hidden / T * 8 / 1e9, 1) != golden["activations_s131072_t8_p16_GB"]["value"]


def test_kv_cache_sizes(golden):
    m = cm.LLAMA3_8B
    assert printed(golden["kv_cache_1M_tokens_8b_class_GB"], cm.kv_cache_bytes(m, 1e6) / 1e9)
    assert printed(golden["kv_per_gpu_tp8_GB"], cm.kv_cache_bytes(m, 1e6, tp=8) / 1e9)
    assert printed(golden["kv_per_gpu_tp8_sp4_GB"], cm.kv_cache_bytes(m, 1e6, tp=8, sp=4) / 1e9)
    assert cm.kv_cache_bytes(m, 1, elem_bytes=2) == 131072  # bytes per token
    # 2**20 tokens would print 137 GB.
    assert not printed(golden["kv_cache_1M_tokens_8b_class_GB"], cm.kv_cache_bytes(m, 2 ** 20) / 1e9)


def test_degenerate_cases():
    assert cm.ring_bytes_per_layer(M, 131072, T, 1) == 0.0  # one device sends nothing
    assert cm.heads_per_device(8, 16) == 1
    assert cm.activation_bytes_per_device(M, 0, T, P) == 0.0
