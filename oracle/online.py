"""Blockwise online softmax, float64 (TEST INFRASTRUCTURE ONLY).

Follows the update rule of [KB] "FlashAttention：为什么少搬数据，反而算得更快"
§04, in its notation. Each query row keeps three quantities:

* m -- the largest score seen so far,
* l -- the sum of exp(score - m) over the keys seen so far,
* U -- the output accumulated so far, not yet divided by l,

starting from m = -inf, l = 0, U = 0. A block of scores s with values V_blk
is folded in by

    m_new = max(m_old, max(s))
    a     = exp(m_old - m_new)          (rescales what is already held)
    p     = exp(s - m_new)
    l     = a * l + sum(p)
    U     = a * U + p @ V_blk

and once every block has been seen O = U / l. The log-sum-exp of the row is
m + ln l.

Reading of the edge case the page only says must be handled (exp of
-inf - -inf): when m_old = -inf nothing is held yet and a = 0; when
m_new = -inf the block is entirely masked, so p = 0 and the state is kept.

This module is used only to pin the oracle: to reproduce the page's worked
example state by state, and to show that every block size reaches the same
result as ``reference``.
"""

from __future__ import annotations

import math

import numpy as np

from .reference import visible_mask


def online_row(scores, values, block: int):
    """Fold one score row into (m, l, U) ``block`` keys at a time.

    scores: [n] (already scaled; -inf where masked). values: [n] or [n, d].
    Returns (O, LSE, trace) where trace holds, per block, the state after the
    old part was rescaled ("a", "l_rescaled", "U_rescaled") and after the
    block was added ("m", "l", "U").
    """
    s = np.asarray(scores, dtype=np.float64)
    vals = np.asarray(values, dtype=np.float64)
    scalar = vals.ndim == 1
    if scalar:
        vals = vals[:, None]
    m = -math.inf
    l = 0.0
    u = np.zeros(vals.shape[1], dtype=np.float64)
    trace = []
    for lo in range(0, s.size, block):
        blk = s[lo:lo + block]
        m_new = max(m, float(np.max(blk)))
        if m_new == -math.inf:
            trace.append(dict(m=m, a=1.0, l_rescaled=l, U_rescaled=u.copy(), l=l, U=u.copy()))
            continue
        a = 0.0 if m == -math.inf else math.exp(m - m_new)
        l_r, u_r = a * l, a * u
        p = np.exp(blk - m_new)
        l = l_r + float(np.sum(p))
        u = u_r + p @ vals[lo:lo + block]
        m = m_new
        trace.append(dict(m=m, a=a, l_rescaled=l_r, U_rescaled=u_r.copy(), l=l, U=u.copy()))
    if l > 0:
        o = u / l
        lse = m + math.log(l)
    else:
        o = np.zeros_like(u)
        lse = -math.inf
    if scalar:
        o = float(o[0])
        for t in trace:
            t["U"] = float(t["U"][0])
            t["U_rescaled"] = float(t["U_rescaled"][0])
    return o, lse, trace


def online_forward(q, k, v, causal: bool, scale: float, block: int):
    """Whole tensors ([B, H, N, d] layout) through :func:`online_row`.

    All rows of a head are advanced together, one key block at a time, with
    the same rule as :func:`online_row`.
    """
    q = np.asarray(q, dtype=np.float64)
    k = np.asarray(k, dtype=np.float64)
    v = np.asarray(v, dtype=np.float64)
    B, Hq, nq, _ = q.shape
    Hkv, nkv = k.shape[1], k.shape[2]
    G = Hq // Hkv
    o = np.zeros((B, Hq, nq, v.shape[3]))
    lse = np.zeros((B, Hq, nq))
    vis = visible_mask(np.arange(nq), nq, nkv, causal)
    for b in range(B):
        for h in range(Hq):
            kh, vh = k[b, h // G], v[b, h // G]
            s = np.where(vis, scale * (q[b, h] @ kh.T), -np.inf)
            m = np.full(nq, -np.inf)
            l = np.zeros(nq)
            u = np.zeros((nq, v.shape[3]))
            for lo in range(0, nkv, block):
                blk = s[:, lo:lo + block]
                m_new = np.maximum(m, np.max(blk, axis=1))
                live = np.isfinite(m_new)
                m_use = np.where(live, m_new, 0.0)
                a = np.where(np.isfinite(m), np.exp(m - m_use), 0.0)
                a = np.where(live, a, 1.0)
                p = np.where(live[:, None], np.exp(blk - m_use[:, None]), 0.0)
                l = a * l + np.sum(p, axis=1)
                u = a[:, None] * u + p @ vh[lo:lo + block]
                m = m_new
            with np.errstate(invalid="ignore", divide="ignore"):
                o[b, h] = np.where(l[:, None] > 0, u / np.where(l > 0, l, 1.0)[:, None], 0.0)
                lse[b, h] = np.where(l > 0, m + np.log(np.where(l > 0, l, 1.0)), -np.inf)
    return o, lse
