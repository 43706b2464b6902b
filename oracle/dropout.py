"""Dropout on the attention probabilities, float64 (TEST INFRASTRUCTURE ONLY).

Only ``tests/``, ``__graft_entry__.smoke()`` and ``bench.py``'s cpu_baseline
leg may use this module. It shares no code with the HIP library.

Page [KB] "FlashAttention：为什么少搬数据，反而算得更快" §04 names dropout among the
things the tiled computation must still get right, and its §08 example call
carries a dropout probability; [KB] §05 rebuilds P in the backward instead of
storing it. Neither page fixes the random numbers or where the mask acts.
Readings taken here (and in the design notes of the repository):

* inverted dropout on the normalised probabilities: with keep mask Z,
  O = r (P o Z) V where r = 1 / (1 - p_eff); the row log-sum-exp is that of
  the scores without dropout (the statistic the backward needs to rebuild
  P), so it does not depend on the mask;
* the mask is drawn from the counter-based generator Philox4x64 with 10
  rounds (Salmon, Moraes, Dror and Shaw, "Parallel Random Numbers: As Easy
  as 1, 2, 3", SC 2011) and regenerated, never stored: element (b, h, i, j)
  of query head h, query row i, key j takes byte t = j mod 32 of the 256-bit
  block philox(counter, key) with counter = (floor(j / 32), i, b * Hq + h,
  offset) and key = (seed, 0); byte t is bits 8 (t mod 8) .. +7 of output
  word floor(t / 8);
* the element is kept iff its byte u >= theta, theta = min(255,
  floor(256 p + 1/2)); so p_eff = theta / 256 and r = 256 / (256 - theta);
* backward (the chain rule through O = r (P o Z) V): dV = r (P o Z)^T dO,
  dP = r Z o (dO V^T), dS = P o (dP - rowsum(P o dP)), dQ = scale dS K,
  dK = scale dS^T Q; rowsum(P o dP) equals rowsum(dO o O) exactly as without
  dropout.

The generator is pinned by a CPU test to an independent implementation of
the same published definition (numpy.random.Philox); the attention side is
pinned by finite differences with a fixed mask and by p = 0 reducing to the
plain definition.
"""

from __future__ import annotations

import numpy as np

from .reference import _check_heads, _softmax_rows, visible_mask

# Philox4x64 round multipliers and key increments (the published constants).
_M0 = np.uint64(0xD2E7470EE14C6C93)
_M1 = np.uint64(0xCA5A826395121157)
_W0 = np.uint64(0x9E3779B97F4A7C15)
_W1 = np.uint64(0xBB67AE8584CAA73B)
_LO32 = np.uint64(0xFFFFFFFF)
_S32 = np.uint64(32)


def _mulhilo(a: np.ndarray, m: np.uint64):
    """(high, low) 64-bit halves of the 128-bit products a * m (a: uint64 array)."""
    a = np.asarray(a, dtype=np.uint64)
    a0, a1 = a & _LO32, a >> _S32
    m0, m1 = m & _LO32, m >> _S32
    p00, p01, p10, p11 = a0 * m0, a0 * m1, a1 * m0, a1 * m1
    mid = (p00 >> _S32) + (p01 & _LO32) + (p10 & _LO32)
    hi = p11 + (p01 >> _S32) + (p10 >> _S32) + (mid >> _S32)
    lo = a * m  # wraps modulo 2^64
    return hi, lo


def philox4x64(counter, key, rounds: int = 10):
    """Philox4x64-R of counters [..., 4] under keys [..., 2] (uint64, broadcast).

    Each round maps (c0, c1, c2, c3) to (hi(M1 c2) ^ c1 ^ k0, lo(M1 c2),
    hi(M0 c0) ^ c3 ^ k1, lo(M0 c0)); the key is advanced by the two Weyl
    constants between rounds. Returns the four output words [..., 4].
    """
    c = np.array(counter, dtype=np.uint64)
    k = np.array(key, dtype=np.uint64)
    c0, c1, c2, c3 = (c[..., i] for i in range(4))
    k0, k1 = k[..., 0], k[..., 1]
    with np.errstate(over="ignore"):
        for r in range(rounds):
            if r:
                k0 = k0 + _W0
                k1 = k1 + _W1
            hi0, lo0 = _mulhilo(c0, _M0)
            hi1, lo1 = _mulhilo(c2, _M1)
            c0, c1, c2, c3 = hi1 ^ c1 ^ k0, lo1, hi0 ^ c3 ^ k1, lo0
    return np.stack(np.broadcast_arrays(c0, c1, c2, c3), axis=-1)


def threshold(p: float) -> int:
    """theta: a key is kept iff its byte >= theta (p in [0, 1))."""
    if not (0.0 <= p < 1.0):
        raise ValueError("dropout probability must be in [0, 1)")
    return min(255, int(np.floor(256.0 * p + 0.5)))


def keep_scale(p: float) -> float:
    """r = 1 / (1 - p_eff) with p_eff = theta / 256."""
    return 256.0 / (256.0 - threshold(p))


def dropout_bytes(bh: int, rows, nkv: int, seed: int, offset: int) -> np.ndarray:
    """The uniform bytes of query rows ``rows`` (all keys 0..nkv-1) of the head
    with flat index bh = b * Hq + h: uint8 [len(rows), nkv]."""
    rows = np.asarray(rows, dtype=np.uint64)
    n_groups = -(-nkv // 32)
    ctr = np.zeros((rows.size, n_groups, 4), dtype=np.uint64)
    ctr[..., 0] = np.arange(n_groups, dtype=np.uint64)[None, :]
    ctr[..., 1] = rows[:, None]
    ctr[..., 2] = np.uint64(bh)
    ctr[..., 3] = np.uint64(offset)
    words = philox4x64(ctr, np.array([seed, 0], dtype=np.uint64))  # [rows, groups, 4]
    # Little-endian bytes of the four words: byte t of a group is bits
    # 8 (t % 8) .. of word t // 8.
    b = words.astype("<u8").view(np.uint8).reshape(rows.size, n_groups * 32)
    return b[:, :nkv]


def keep_mask(bh: int, rows, nkv: int, p: float, seed: int, offset: int) -> np.ndarray:
    """Boolean keep mask Z of the given rows of head bh: [len(rows), nkv]."""
    return dropout_bytes(bh, rows, nkv, seed, offset) >= threshold(p)


def head_forward_dropout(q, k, v, causal: bool, scale: float, keep, r: float):
    """One head, all rows, with keep mask ``keep`` [N_q, N_kv] and factor r."""
    q = np.asarray(q, dtype=np.float64)
    k = np.asarray(k, dtype=np.float64)
    v = np.asarray(v, dtype=np.float64)
    nq, nkv = q.shape[0], k.shape[0]
    s = scale * (q @ k.T)
    s = np.where(visible_mask(np.arange(nq), nq, nkv, causal), s, -np.inf)
    p, lse = _softmax_rows(s)
    o = r * ((p * keep) @ v)
    return o, lse


def head_backward_dropout(q, k, v, do, causal: bool, scale: float, keep, r: float):
    """Gradients of sum(dO * O) for :func:`head_forward_dropout`."""
    q = np.asarray(q, dtype=np.float64)
    k = np.asarray(k, dtype=np.float64)
    v = np.asarray(v, dtype=np.float64)
    do = np.asarray(do, dtype=np.float64)
    nq, nkv = q.shape[0], k.shape[0]
    s = scale * (q @ k.T)
    s = np.where(visible_mask(np.arange(nq), nq, nkv, causal), s, -np.inf)
    p, _ = _softmax_rows(s)
    pz = r * (p * keep)
    dv = pz.T @ do
    dp = r * keep * (do @ v.T)
    ds = p * (dp - np.sum(p * dp, axis=1, keepdims=True))
    return scale * (ds @ k), scale * (ds.T @ q), dv


def attention_forward_dropout(q, k, v, causal: bool, scale: float, p: float, seed: int,
                              offset: int, heads=None):
    """Layout of ``reference.attention_forward``; returns (O, LSE). ``heads``
    optionally restricts the work to (b, h) pairs (others left NaN)."""
    B, Hq, Hkv, G = _check_heads(q, k)
    nq, nkv = q.shape[2], k.shape[2]
    r = keep_scale(p)
    o = np.full((B, Hq, nq, v.shape[3]), np.nan)
    lse = np.full((B, Hq, nq), np.nan)
    todo = heads if heads is not None else [(b, h) for b in range(B) for h in range(Hq)]
    for b, h in todo:
        z = keep_mask(b * Hq + h, np.arange(nq), nkv, p, seed, offset)
        o[b, h], lse[b, h] = head_forward_dropout(q[b, h], k[b, h // G], v[b, h // G], causal,
                                                  scale, z, r)
    return o, lse


def attention_backward_dropout(q, k, v, do, causal: bool, scale: float, p: float, seed: int,
                               offset: int):
    """Gradients for :func:`attention_forward_dropout` (dK, dV summed over each
    kv head's query heads)."""
    B, Hq, Hkv, G = _check_heads(q, k)
    nq, nkv = q.shape[2], k.shape[2]
    r = keep_scale(p)
    dq = np.zeros(np.shape(q), dtype=np.float64)
    dk = np.zeros(np.shape(k), dtype=np.float64)
    dv = np.zeros(np.shape(v), dtype=np.float64)
    for b in range(B):
        for h in range(Hq):
            z = keep_mask(b * Hq + h, np.arange(nq), nkv, p, seed, offset)
            g, kg, vg = head_backward_dropout(q[b, h], k[b, h // G], v[b, h // G], do[b, h],
                                              causal, scale, z, r)
            dq[b, h] = g
            dk[b, h // G] += kg
            dv[b, h // G] += vg
    return dq, dk, dv
