"""Textbook attention as plain Python loops, for tiny inputs only.

TEST INFRASTRUCTURE ONLY (see ``oracle/__init__.py``).  Used to pin the numpy
oracle: no numpy arithmetic, no layout, just lists of floats.

out[i][d] = sum_t p_t * V[t][d],  p_t = exp(s_t - m) / sum_u exp(s_u - m),
s_t = scale * sum_d q[i][d] * K[t][d],  m = max_t s_t.
"""
from __future__ import annotations

import math


def attention_one_query(q, K, V, scale):
    """q: list[D]; K, V: list[L][D] -> list[D]."""
    s = []
    for krow in K:
        acc = 0.0
        for qd, kd in zip(q, krow):
            acc += qd * kd
        s.append(scale * acc)
    m = max(s)
    e = [math.exp(x - m) for x in s]
    z = sum(e)
    D = len(V[0])
    out = [0.0] * D
    for w, vrow in zip(e, V):
        p = w / z
        for d in range(D):
            out[d] += p * vrow[d]
    return out


def gqa_decode(q, K, V, scale):
    """q: [Hq][D]; K, V: [Hkv][L][D] -> [Hq][D]; head i reads KV head i // (Hq/Hkv)."""
    Hq, Hkv = len(q), len(K)
    G = Hq // Hkv
    return [attention_one_query(q[i], K[i // G], V[i // G], scale) for i in range(Hq)]
