"""FP8 (E4M3) forward, float64 (TEST INFRASTRUCTURE ONLY).

Only ``tests/``, ``__graft_entry__.smoke()`` and ``bench.py``'s cpu_baseline
leg may use this module. It shares no code with the HIP library.

Page [KB] "FlashAttention：为什么少搬数据，反而算得更快" §07 notes that the Hopper
generation adds an FP8 path; the pages fix neither the format nor the
scaling. Readings taken here (and in the design notes of the repository):

* q, k and v arrive as 8-bit floats in the OCP E4M3 format (1 sign bit,
  4 exponent bits with bias 7, 3 mantissa bits, subnormals, no infinities,
  the two all-ones codes are NaN; largest finite value 448) with one
  float32 "descale" factor per tensor: the real input is code value times
  descale;
* the result is the attention of those real inputs, exactly as
  ``reference.head_forward`` defines it (scale, causal mask, softmax),
  returned as O (16-bit in the kernel) and the row LSE;
* the kernel rounds the probabilities to E4M3 for the P V product; the
  oracle does not, and the comparison allows that rounding (see
  ``p_rounding_bound``).
"""

from __future__ import annotations

import numpy as np

from .reference import _softmax_rows, head_forward, visible_mask

# Error of one 8-bit matrix-core product (32x32x64 with E4M3 operands),
# relative to the sum of the magnitudes of the 64 terms it adds: the
# products are exact, but their sum is not formed exactly in float32. This
# constant is a measurement, not a definition: the GPU test
# test_fp8_score_accumulation_error (tests/test_parity_fp8.py) reads the
# scores the kernel computes back through the LSE of a one-key softmax and
# checks that no score is off by more than EPS8 * scale * sum_c |q_c k_c|.
# Largest seen on MI355X: 2^-12.27 with elements scaled by powers of two
# from 2^-6 to 2^6, 2^-12.64 over uniformly random codes, 2^-15.6 on N(0, 1)
# draws; EPS8 leaves a factor of 2.4 over the largest.
EPS8 = 2.0 ** -11


def e4m3_value(code: int) -> float:
    """Real value of one E4M3 code, from the format's definition."""
    code = int(code) & 0xFF
    sign = -1.0 if code & 0x80 else 1.0
    e = (code >> 3) & 0xF
    m = code & 0x7
    if e == 0xF and m == 0x7:
        return float("nan")
    if e == 0:
        return sign * (m / 8.0) * 2.0 ** (1 - 7)  # subnormal
    return sign * (1.0 + m / 8.0) * 2.0 ** (e - 7)


E4M3_TABLE = np.array([e4m3_value(c) for c in range(256)], dtype=np.float64)


def decode(codes, descale: float = 1.0) -> np.ndarray:
    """Real values of an array of E4M3 codes (uint8) times descale."""
    return E4M3_TABLE[np.asarray(codes, dtype=np.uint8)] * float(descale)


def head_forward_fp8(q8, k8, v8, causal: bool, scale: float, dq: float, dk: float, dv: float):
    """One head: E4M3 codes q8 [N_q, d], k8, v8 [N_kv, d] with their descale
    factors -> (O, LSE) of the real inputs, float64."""
    return head_forward(decode(q8, dq), decode(k8, dk), decode(v8, dv), causal, scale)


def p_rounding_bound(q8, k8, v8, causal: bool, scale: float, dq: float, dk: float, dv: float):
    """Per-element bound on what rounding P to E4M3 can change in O.

    With the running maximum m used for P (every kernel P value is
    exp(S - m) with m at most the row's true maximum in log units, so each
    row's sum l of those values is >= 1), rounding to nearest E4M3 changes a
    value x by at most 2^-4 x when x is normal (>= 2^-6) and by at most
    2^-10 otherwise; dividing by l >= 1, each normalised weight P_ij moves by
    at most max(2^-4 P_ij, 2^-10). The bound on O_ic is therefore
    sum_j max(2^-4 P_ij, 2^-10) |V_jc|. Returns that bound [N_q, d]."""
    q = decode(q8, dq)
    k = decode(k8, dk)
    v = decode(v8, dv)
    nq, nkv = q.shape[0], k.shape[0]
    s = scale * (q @ k.T)
    vis = visible_mask(np.arange(nq), nq, nkv, causal)
    s = np.where(vis, s, -np.inf)
    p, _ = _softmax_rows(s)
    w = np.where(vis, np.maximum(p * 2.0 ** -4, 2.0 ** -10), 0.0)
    return w @ np.abs(v)


def accumulation_bound(q8, k8, v8, causal: bool, scale: float, dq: float, dk: float, dv: float,
                       eps8: float = EPS8):
    """Bound on what the inexact sums of the 8-bit products can change in O
    and in the LSE: returns (O bound [N_q, d], LSE bound [N_q]).

    Each score moves by at most E_ij = eps8 * scale * sum_c |q_ic k_jc|.
    Scores moved by at most E_i = max_j E_ij (over the visible keys) move
    LSE_i by at most E_i, and every softmax weight by at most a factor
    exp(+-2 E_i), so O_ic by at most (exp(2 E_i) - 1) sum_j P_ij |V_jc|.
    The P V products add their terms with the same relative error, at most
    eps8 times the sum of the magnitudes of the (rounded) terms, which the
    rounding of P keeps within (1 + 2^-4) sum_j P_ij |V_jc|; the O bound
    adds that."""
    q = decode(q8, dq)
    k = decode(k8, dk)
    v = decode(v8, dv)
    nq, nkv = q.shape[0], k.shape[0]
    vis = visible_mask(np.arange(nq), nq, nkv, causal)
    s = np.where(vis, scale * (q @ k.T), -np.inf)
    p, _ = _softmax_rows(s)
    e = np.where(vis, eps8 * scale * (np.abs(q) @ np.abs(k).T), 0.0)
    e_row = e.max(axis=1) if nkv else np.zeros(nq)
    pv = p @ np.abs(v)
    o_bound = np.expm1(2.0 * e_row)[:, None] * pv + eps8 * (1.0 + 2.0 ** -4) * pv
    return o_bound, e_row
