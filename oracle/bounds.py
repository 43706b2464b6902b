"""Magnitude sums that bound the rounding error of computed gradients
(TEST INFRASTRUCTURE ONLY; nothing in the product path uses this module).

The gradients of [KB] "FlashAttention：为什么少搬数据，反而算得更快" §05 are
sums of products: with P, dP and D as in ``reference.head_backward``

    dV_jc = sum_i P_ij dO_ic
    dK_jc = scale sum_i dS_ij Q_ic,   dQ_ic = scale sum_j dS_ij K_jc,
    dS_ij = P_ij (dP_ij - D_i).

An implementation that rounds each probability (or each dS) to a 16-bit
format with unit roundoff u before the products changes every term by at
most u of its size, so its error in one gradient element is at most u times
the sum of the terms' magnitudes. Computing D_i from the rounded output O
(the forward's own output, each element within u of the exact one) changes
D_i by at most u * Dabs_i with Dabs_i = sum_c |dO_ic| |O_ic|. Writing

    A_ij = P_ij (|dP_ij| + Dabs_i)   (>= |dS_ij|, and >= P_ij |error of D_i| / u)

the magnitudes returned here are

    Mv = P^T |dO|,   Mk = scale A^T |Q|,   Mq = scale A |K|,

so a 16-bit implementation's error is at most u Mv (dV) and 2 u Mk, 2 u Mq
(dK, dQ), plus u |g| for rounding the result. With dropout (keep mask Z,
factor r) P enters dV as r P o Z and dP as r Z o dP.

Tiny values also carry an absolute error, whatever their size: an fp16
value below its normal range is off by up to half its smallest subnormal,
and float32 arithmetic may flush values below its smallest normal (2^-126)
to zero, bf16 sharing float32's range. With an absolute error t in every P
and every dS, the gradients move by at most t times

    Cv = vis^T |dO|,  Ck = scale W^T |Q|,  Cq = scale W |K|,
    W_ij = vis_ij (|dP_ij| + Dabs_i + 1)

(vis: the visible entries; a flushed P_ij moves dS_ij by up to
t (|dP_ij| + Dabs_i), a rounded dS_ij by up to t).
"""

from __future__ import annotations

import numpy as np

from .reference import _softmax_rows, visible_mask


def head_backward_magnitudes(q, k, v, do, causal: bool, scale: float, keep=None, r: float = 1.0):
    """One head, all rows: (Mq, Mk, Mv, Cq, Ck, Cv, Rq, Rk, Rv, Lq) as in the
    module text, each shaped like the gradient it belongs to.

    R* are the root-sum-squares of the same terms (sqrt(sum_i x_i^2) where
    M sums |x_i|): independent rounding errors of the terms add up like a
    random walk, to about u R rather than the worst case u M. Lq is the part
    of dQ's error that is common to all terms of a row (the error of D_i,
    which multiplies every dS_ij of the row alike), scale Dabs_i sum_j
    P_ij |K_jc|; for dK and dV that error differs from term to term and is
    inside R.

    ``keep`` is an optional boolean keep mask [N_q, N_kv] with factor r
    (dropout); without it every entry is kept and r = 1."""
    q = np.asarray(q, dtype=np.float64)
    k = np.asarray(k, dtype=np.float64)
    v = np.asarray(v, dtype=np.float64)
    do = np.asarray(do, dtype=np.float64)
    nq, nkv = q.shape[0], k.shape[0]
    vis = visible_mask(np.arange(nq), nq, nkv, causal)
    s = np.where(vis, scale * (q @ k.T), -np.inf)
    p, _ = _softmax_rows(s)
    z = np.ones((nq, nkv)) if keep is None else np.asarray(keep, dtype=np.float64)
    pz = r * p * z
    o = pz @ v                                   # the exact output
    dabs = np.sum(np.abs(do) * np.abs(o), axis=1, keepdims=True)
    a = p * (r * z * np.abs(do @ v.T) + dabs)
    visf = vis.astype(np.float64)
    mq = scale * (a @ np.abs(k))
    mk = scale * (a.T @ np.abs(q))
    mv = pz.T @ np.abs(do)
    w = visf * (r * z * np.abs(do @ v.T) + dabs + 1.0)
    cq = scale * (w @ np.abs(k))
    ck = scale * (w.T @ np.abs(q))
    cv = visf.T @ np.abs(do)
    rq = scale * np.sqrt((a * a) @ (k * k))
    rk = scale * np.sqrt((a * a).T @ (q * q))
    rv = np.sqrt((pz * pz).T @ (do * do))
    lq = scale * dabs * (p @ np.abs(k))
    return mq, mk, mv, cq, ck, cv, rq, rk, rv, lq
def group_backward_magnitudes(q, k, v, do, causal: bool, scale: float, b: int, hk: int,
                              keep_of=None, r: float = 1.0):
    """The magnitudes of one kv head's group in the [B, H, N, d] layout, as
    :func:`head_backward_magnitudes` returns them: the dQ-shaped ones
    stacked over the G query heads [G, N_q, d], the dK / dV-shaped ones for
    kv head hk of batch b (sums over the G query heads that read it; the
    root-sum-squares combine as such). ``keep_of(h)`` gives query head h's
    keep mask when dropout is on."""
    G = q.shape[1] // k.shape[1]
    per_q = ([], [], [], [])            # Mq, Cq, Rq, Lq
    mk = np.zeros(k.shape[2:])
    mv, ck, cv = np.zeros_like(mk), np.zeros_like(mk), np.zeros_like(mk)
    rk2, rv2 = np.zeros_like(mk), np.zeros_like(mk)
    for h in range(hk * G, (hk + 1) * G):
        z = None if keep_of is None else keep_of(h)
        mq, mkh, mvh, cq, ckh, cvh, rq, rkh, rvh, lq = head_backward_magnitudes(
            q[b, h], k[b, hk], v[b, hk], do[b, h], causal, scale, z, r)
        mk += mkh
        mv += mvh
        ck += ckh
        cv += cvh
        rk2 += rkh * rkh
        rv2 += rvh * rvh
        for lst, x in zip(per_q, (mq, cq, rq, lq)):
            lst.append(x)
    mq, cq, rq, lq = (np.stack(x) for x in per_q)
    return mq, mk, mv, cq, ck, cv, rq, np.sqrt(rk2), np.sqrt(rv2), lq


def attention_backward_magnitudes(q, k, v, do, causal: bool, scale: float, keep_of=None,
                                  r: float = 1.0):
    """The magnitudes for whole tensors in the [B, H, N, d] layout, in the
    order of :func:`head_backward_magnitudes`, each shaped like its gradient.
    ``keep_of(b, h)`` gives the keep mask of query head h of batch b when
    dropout is on."""
    B, Hkv = q.shape[0], k.shape[1]
    G = q.shape[1] // Hkv
    shapes = (q, k, v, q, k, v, q, k, v, q)
    out = [np.zeros(np.shape(x)) for x in shapes]
    for b in range(B):
        for hk in range(Hkv):
            kf = None if keep_of is None else (lambda h, b=b: keep_of(b, h))
            parts = group_backward_magnitudes(q, k, v, do, causal, scale, b, hk, kf, r)
            for i, x in enumerate(parts):
                if shapes[i] is q:
                    out[i][b, hk * G:(hk + 1) * G] = x
                else:
                    out[i][b, hk] = x
    return tuple(out)
