"""Plant plausible mistakes in a copy of the oracle and check the pins catch each.

Every mutant is built from ``oracle/oracle.cpp`` by one text substitution,
compiled into a temporary directory on the CPU, and run through the pins in
``pins.py``; at least one pin must fail for every mutant.
"""
import os
import tempfile

import pytest

import oracle
import pins

SRC = os.path.join(os.path.dirname(oracle.__file__), "oracle.cpp")

MUTANTS = {
    "causal_excludes_self": ("if (!causal || j <= pos)", "if (!causal || j < pos)"),
    "gqa_head_modulo": ("const int64_t hk = h / group;", "const int64_t hk = h % Hkv;"),
    "dropped_scale": ("score[t] = scale * dot;", "score[t] = dot;"),
    "lse_missing_max": ("lse[item] = mx + std::log(z);", "lse[item] = std::log(z);"),
    "scores_use_values": ("dot += qrow[e] * load(k, dtype, kbase + e);", "dot += qrow[e] * load(v, dtype, kbase + e);"),
    "missing_normaliser": ("o[e] = acc[e] / z;", "o[e] = acc[e];"),
    "wrong_exp_sign": ("std::exp(score[t] - mx)", "std::exp(mx - score[t])"),
    "q_indexed_by_position": ("((b * Hq + h) * Sq + row) * d + e", "((b * Hq + h) * Sq + pos) * d + e"),
    "key_set_ignored": ("const int64_t j = keys ? keys[t] : t;", "const int64_t j = t;"),
    "bf16_widen_shift": ("static_cast<const uint16_t*>(base)[idx]) << 16;", "static_cast<const uint16_t*>(base)[idx]) << 15;"),
    "value_head_transposed": ("const int64_t vbase = ((b * Hkv + hk) * S + vis[t]) * d;",
                              "const int64_t vbase = ((b * Hkv + (Hkv - 1 - hk)) * S + vis[t]) * d;"),
}


@pytest.fixture(scope="module")
def src_text():
    with open(SRC) as f:
        return f.read()


@pytest.mark.parametrize("name", sorted(MUTANTS))
def test_pins_catch_mutant(src_text, name, tmp_path):
    before, after = MUTANTS[name]
    assert src_text.count(before) == 1, f"mutation anchor not unique for {name}"
    mutant_src = tmp_path / "oracle_mutant.cpp"
    mutant_src.write_text(src_text.replace(before, after))
    so = str(tmp_path / "liboracle_mutant.so")
    oracle.build(out=so, src=str(mutant_src))
    lib = oracle.load_lib(so)
    failed = []
    for pin in pins.ALL_PINS:
        try:
            pin(lib)
        except AssertionError:
            failed.append(pin.__name__)
    assert failed, f"no pin catches mutant {name}"
