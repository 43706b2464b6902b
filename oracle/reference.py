"""The attention definition written out in float64 (TEST INFRASTRUCTURE ONLY).

Only ``tests/``, ``__graft_entry__.smoke()`` and ``bench.py``'s cpu_baseline
leg may use this module. It shares no code with the HIP library.

What is computed (per batch b and query head h, with kv head h // G):

* forward ([BLOG] §一 and §三; [KB] §02): S = scale * Q K^T; entries a causal
  query may not see are set to -inf; P = softmax(S) row-wise, in the safe form
  that subtracts the row maximum first ([BLOG] §四); O = P V. The row
  statistic kept for the backward ([KB] §05) is LSE_i = m_i + ln sum_j
  exp(S_ij - m_i).
* backward ([KB] §05 names the quantities, prints no formula): the textbook
  chain rule applied to the forward above -- dV = P^T dO, dP = dO V^T,
  dS_ij = P_ij (dP_ij - sum_k P_ik dP_ik), dQ = scale dS K, dK = scale dS^T Q.
  For grouped heads ([NEWS]: MHA / MQA / GQA) dK and dV of a kv head are the
  sums over the query heads that read it.

Readings taken where the pages are silent (each also listed in the design
notes of the repository):

* scale is a caller-supplied float, applied to QK^T before mask and softmax;
* causal visibility is aligned to the bottom-right corner: query i may see key
  j iff j <= i + (N_kv - N_q); it is j <= i when N_q == N_kv and every key
  when N_q == 1;
* q-head h reads kv-head floor(h / G) with G = Hq / Hkv (contiguous groups);
* layout [batch, heads, sequence, head_dim] for every tensor ([KB] §08);
* LSE uses the natural logarithm;
* a query row that sees no key has O = 0 and LSE = -inf and passes no
  gradient. LSE = -inf is the log-sum-exp of an empty set; O = 0 is a
  convention (parity unpinned for that value); given it, the zero gradient
  follows and is pinned by finite differences;
* "equivalent" means the same mathematical result, not the same bits
  ([KB] §04), so the comparison with the GPU is tolerance based.

Rows are processed in chunks to bound memory; rows are independent, so each
chunk holds complete rows of S and P and the chunking changes nothing.
"""

from __future__ import annotations

import numpy as np

_CHUNK_ELEMS = 1 << 23  # rows per chunk chosen so a chunk of S is <= 64 MiB


def visible_mask(row_index, nq: int, nkv: int, causal: bool) -> np.ndarray:
    """Boolean [len(row_index), nkv]: which keys each query row may see."""
    rows = np.asarray(row_index, dtype=np.int64)
    if not causal:
        return np.ones((rows.size, nkv), dtype=bool)
    cols = np.arange(nkv, dtype=np.int64)
    return cols[None, :] <= (rows[:, None] + (nkv - nq))


def _softmax_rows(s: np.ndarray):
    """Safe softmax of each row of s (entries may be -inf).

    Returns (P, LSE). A row whose entries are all -inf, or that has no
    entries at all (no keys), gets P = 0, LSE = -inf: the log-sum-exp of an
    empty set.
    """
    m = np.max(s, axis=1, keepdims=True, initial=-np.inf)
    empty = ~np.isfinite(m[:, 0])
    m_safe = np.where(np.isfinite(m), m, 0.0)
    e = np.exp(s - m_safe)
    denom = np.sum(e, axis=1, keepdims=True)
    with np.errstate(invalid="ignore", divide="ignore"):
        p = np.where(denom > 0, e / np.where(denom > 0, denom, 1.0), 0.0)
        lse = (m_safe + np.log(denom))[:, 0]
    lse[empty] = -np.inf
    return p, lse


def _chunks(n: int, nkv: int):
    step = max(1, _CHUNK_ELEMS // max(1, nkv))
    for lo in range(0, n, step):
        yield lo, min(n, lo + step)


def head_forward(q, k, v, causal: bool, scale: float, row_index=None, nq=None):
    """One head. q [n, d], k and v [N_kv, d] -> (O [n, d], LSE [n]).

    ``row_index`` gives the absolute query positions of the rows in q (for the
    causal mask) and ``nq`` the head's full query length; by default q holds
    all rows 0..n-1. Sampling rows this way computes exactly the same values
    as the full head, because attention rows are independent.
    """
    q = np.asarray(q, dtype=np.float64)
    k = np.asarray(k, dtype=np.float64)
    v = np.asarray(v, dtype=np.float64)
    n = q.shape[0]
    if row_index is None:
        row_index = np.arange(n)
        nq = n if nq is None else nq
    row_index = np.asarray(row_index, dtype=np.int64)
    nkv = k.shape[0]
    o = np.zeros((n, v.shape[1]), dtype=np.float64)
    lse = np.empty(n, dtype=np.float64)
    for lo, hi in _chunks(n, nkv):
        s = scale * (q[lo:hi] @ k.T)
        vis = visible_mask(row_index[lo:hi], nq, nkv, causal)
        s = np.where(vis, s, -np.inf)
        p, l = _softmax_rows(s)
        o[lo:hi] = p @ v
        lse[lo:hi] = l
    return o, lse


def head_backward(q, k, v, do, causal: bool, scale: float):
    """One head, all rows. Returns (dQ [N_q, d], dK [N_kv, d], dV [N_kv, d])."""
    q = np.asarray(q, dtype=np.float64)
    k = np.asarray(k, dtype=np.float64)
    v = np.asarray(v, dtype=np.float64)
    do = np.asarray(do, dtype=np.float64)
    nq, nkv = q.shape[0], k.shape[0]
    dq = np.zeros_like(q)
    dk = np.zeros_like(k)
    dv = np.zeros_like(v)
    for lo, hi in _chunks(nq, nkv):
        s = scale * (q[lo:hi] @ k.T)
        vis = visible_mask(np.arange(lo, hi), nq, nkv, causal)
        s = np.where(vis, s, -np.inf)
        p, _ = _softmax_rows(s)
        dp = do[lo:hi] @ v.T
        # Jacobian of the row softmax: dS = P * (dP - sum_k P_k dP_k).
        ds = p * (dp - np.sum(p * dp, axis=1, keepdims=True))
        dv += p.T @ do[lo:hi]
        dq[lo:hi] = scale * (ds @ k)
        dk += scale * (ds.T @ q[lo:hi])
    return dq, dk, dv


def _check_heads(q, k):
    B, Hq = q.shape[0], q.shape[1]
    Hkv = k.shape[1]
    if Hq % Hkv != 0:
        raise ValueError("Hq must be a multiple of Hkv")
    return B, Hq, Hkv, Hq // Hkv


def attention_forward(q, k, v, causal: bool, scale: float, heads=None):
    """q [B, Hq, N_q, d]; k, v [B, Hkv, N_kv, d] -> (O, LSE [B, Hq, N_q]).

    ``heads`` optionally restricts the work to a list of (b, h) pairs; the
    other heads of the result are left as NaN.
    """
    B, Hq, Hkv, G = _check_heads(q, k)
    nq, d = q.shape[2], q.shape[3]
    o = np.full((B, Hq, nq, v.shape[3]), np.nan)
    lse = np.full((B, Hq, nq), np.nan)
    todo = heads if heads is not None else [(b, h) for b in range(B) for h in range(Hq)]
    for b, h in todo:
        o[b, h], lse[b, h] = head_forward(q[b, h], k[b, h // G], v[b, h // G], causal, scale)
    return o, lse


def attention_backward(q, k, v, do, causal: bool, scale: float):
    """Gradients of sum(dO * O) for the layout of :func:`attention_forward`."""
    B, Hq, Hkv, G = _check_heads(q, k)
    dq = np.zeros(np.shape(q), dtype=np.float64)
    dk = np.zeros(np.shape(k), dtype=np.float64)
    dv = np.zeros(np.shape(v), dtype=np.float64)
    for b in range(B):
        for h in range(Hq):
            g, kg, vg = head_backward(q[b, h], k[b, h // G], v[b, h // G], do[b, h], causal, scale)
            dq[b, h] = g
            dk[b, h // G] += kg
            dv[b, h // G] += vg
    return dq, dk, dv


def paged_gather(pool, page_table_row, n_keys: int):
    """The first n_keys keys of one sequence from a page pool
    [num_pages, Hkv, page_size, d] and its row of the page table: logical page
    p (keys p*page_size ..) lives in pool page page_table_row[p]. Returns
    ([Hkv, n, d], valid [n]): keys whose table entry lies outside
    [0, num_pages) name no page; they are returned as zeros and marked
    invalid (reading: such keys are dropped from the attention)."""
    num_pages, Hkv, page_size, d = pool.shape
    n_pages = -(-n_keys // page_size)
    if n_pages == 0:
        return np.zeros((Hkv, 0, d)), np.zeros(0, dtype=bool)
    pages, valid = [], []
    for p in range(n_pages):
        e = int(page_table_row[p])
        ok = 0 <= e < num_pages
        pages.append(pool[e] if ok else np.zeros((Hkv, page_size, d)))
        valid.append(np.full(page_size, ok))
    return np.concatenate(pages, axis=1)[:, :n_keys], np.concatenate(valid)[:n_keys]


def paged_decode_forward(q, k_pages, v_pages, page_table, seq_lens, scale: float):
    """Decode over a paged K/V cache ([KB] §09 pairs paged KV with decode):
    q [B, Hq, 1, d]; k_pages, v_pages [num_pages, Hkv, page_size, d];
    page_table [B, max_pages]; seq_lens [B]. Each sequence's K and V are
    gathered through its table row and the single query row attends to all of
    them (no mask), except keys whose table entry is out of range, which are
    dropped. Returns (O [B, Hq, 1, d], LSE [B, Hq, 1])."""
    B, Hq = q.shape[0], q.shape[1]
    Hkv = k_pages.shape[1]
    G = Hq // Hkv
    o = np.zeros((B, Hq, 1, v_pages.shape[3]))
    lse = np.full((B, Hq, 1), -np.inf)
    for b in range(B):
        n = int(seq_lens[b])
        if n == 0:
            continue
        kb, valid = paged_gather(k_pages, page_table[b], n)
        vb, _ = paged_gather(v_pages, page_table[b], n)
        kb, vb = kb[:, valid], vb[:, valid]
        if kb.shape[1] == 0:
            continue
        for h in range(Hq):
            o[b, h], lse[b, h] = head_forward(q[b, h], kb[h // G], vb[h // G], False, scale)
    return o, lse
