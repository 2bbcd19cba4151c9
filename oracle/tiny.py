"""Pure-Python brute-force softmax attention for tiny inputs (S <= 16, d <= 8).

TEST INFRASTRUCTURE ONLY.  A second, independent spelling of the definition
the fp64 oracle computes, with no max subtraction and nothing but ``math``:

    out_i = sum_j exp(s_ij) v_j / sum_j exp(s_ij),   lse_i = log sum_j exp(s_ij),
    s_ij  = scale * <q_i, k_j>,  j over the keys visible to query i

(causal: key position <= query position, "Splitting the Sequence", intro;
grouped-query attention: query head h reads key/value head h // (Hq/Hkv)).
"""
from __future__ import annotations

import math


def attention(q, k, v, scale, causal):
    """q: nested lists [B][Hq][S][d]; k, v: [B][Hkv][S][d].  Returns (out, lse)."""
    B = len(q)
    Hq = len(q[0])
    Hkv = len(k[0])
    S = len(k[0][0])
    d = len(k[0][0][0])
    group = Hq // Hkv
    out = [[[[0.0] * d for _ in range(len(q[0][0]))] for _ in range(Hq)] for _ in range(B)]
    lse = [[[0.0] * len(q[0][0]) for _ in range(Hq)] for _ in range(B)]
    for b in range(B):
        for h in range(Hq):
            hk = h // group
            for i in range(len(q[b][h])):
                weights = []
                for j in range(S):
                    if causal and j > i:
                        continue
                    s = scale * sum(q[b][h][i][e] * k[b][hk][j][e] for e in range(d))
                    weights.append((math.exp(s), j))
                z = sum(w for w, _ in weights)
                for e in range(d):
                    out[b][h][i][e] = sum(w * v[b][hk][j][e] for w, j in weights) / z
                lse[b][h][i] = math.log(z)
    return out, lse
