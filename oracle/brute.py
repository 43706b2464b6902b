"""Scalar pure-Python attention for tiny inputs (TEST INFRASTRUCTURE ONLY).

A second, independent spelling of the definition in [BLOG]
"AI infra. 一层全看懂(五)Flash Attention" §一 / §四 and [KB]
"FlashAttention：为什么少搬数据，反而算得更快" §02: for every query row, the
scaled dot product with every key it may see, the safe softmax (subtract the
row maximum, exponentiate, divide by the sum) and the weighted sum of the
value rows. Python floats and explicit loops only, no numpy, no shared
helper: the causal rule (key j visible to query i iff j <= i + N_kv - N_q)
and the head grouping (q-head h reads kv-head h // (Hq / Hkv)) are spelled out
again here.
"""

from __future__ import annotations

import math


def brute_forward(q, k, v, causal: bool, scale: float):
    """q [B][Hq][N_q][d], k and v [B][Hkv][N_kv][d] as nested sequences.

    Returns (O, LSE) as nested lists.
    """
    B = len(q)
    Hq = len(q[0])
    Hkv = len(k[0])
    G = Hq // Hkv
    O, LSE = [], []
    for b in range(B):
        ob, lb = [], []
        for h in range(Hq):
            kh = k[b][h // G]
            vh = v[b][h // G]
            nq = len(q[b][h])
            nkv = len(kh)
            oh, lh = [], []
            for i in range(nq):
                qi = q[b][h][i]
                scores = []
                for j in range(nkv):
                    if causal and j > i + (nkv - nq):
                        continue
                    dot = 0.0
                    for c in range(len(qi)):
                        dot += float(qi[c]) * float(kh[j][c])
                    scores.append((j, scale * dot))
                dv = len(vh[0])
                if not scores:
                    oh.append([0.0] * dv)
                    lh.append(-math.inf)
                    continue
                mx = max(s for _, s in scores)
                weights = [(j, math.exp(s - mx)) for j, s in scores]
                total = sum(w for _, w in weights)
                row = [0.0] * dv
                for j, w in weights:
                    for c in range(dv):
                        row[c] += (w / total) * float(vh[j][c])
                oh.append(row)
                lh.append(mx + math.log(total))
            ob.append(oh)
            lb.append(lh)
        O.append(ob)
        LSE.append(lb)
    return O, LSE
