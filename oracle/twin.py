"""Independent brute-force attention in pure Python -- TEST INFRASTRUCTURE ONLY.

A second, deliberately different spelling of the textbook definition used to
pin ``oracle.c`` on tiny shapes: nested Python loops, ``math.fsum`` sums, and
the softmax written as exp(s_j) / sum exp(s_j) without the max shift (safe at
the tiny magnitudes it is used on).  It shares no code with ``oracle.c``.

Definition ("S12 FlashAttention", llminference.xinbetween.com, section
"Motivation / The problem"): S = q k^T (scaled by 1/sqrt(d) as in the
section "Core idea / The solution"), softmax over each row, times V.
"""
from __future__ import annotations

import math


def _f(x) -> float:
    return float(x)


def attention(q, k, v, scale, visible):
    """q: list of query rows, k/v: lists of key/value rows (nested lists of
    floats).  visible(i, j) -> bool.  Returns (o rows, lse list)."""
    outs, lses = [], []
    d = len(v[0]) if v else 0
    for i, qi in enumerate(q):
        keys = [j for j in range(len(k)) if visible(i, j)]
        if not keys:
            outs.append([0.0] * d)
            lses.append(-math.inf)
            continue
        scores = {j: scale * math.fsum(_f(a) * _f(b) for a, b in zip(qi, k[j])) for j in keys}
        weights = {j: math.exp(scores[j]) for j in keys}
        z = math.fsum(weights.values())
        row = []
        for c in range(d):
            row.append(math.fsum(weights[j] * _f(v[j][c]) for j in keys) / z)
        outs.append(row)
        lses.append(math.log(z))
    return outs, lses


def dense(q, k, v, causal, scale):
    """q [B, Nq, Hq, d], k/v [B, Nk, Hkv, d] as float arrays.  Returns
    o [B][Hq][Nq][d] and lse [B][Hq][Nq] as nested lists."""
    B, Nq, Hq, _ = q.shape
    Nk, Hkv = k.shape[1], k.shape[2]
    group = Hq // Hkv
    o_all, l_all = [], []
    for b in range(B):
        ob, lb = [], []
        for h in range(Hq):
            g = h // group
            qs = [list(q[b, i, h]) for i in range(Nq)]
            ks = [list(k[b, j, g]) for j in range(Nk)]
            vs = [list(v[b, j, g]) for j in range(Nk)]
            if causal:
                vis = lambda i, j: j - (Nk - Nq) <= i  # noqa: E731
            else:
                vis = lambda i, j: True  # noqa: E731
            o, l = attention(qs, ks, vs, scale, vis)
            ob.append(o)
            lb.append(l)
        o_all.append(ob)
        l_all.append(lb)
    return o_all, l_all
