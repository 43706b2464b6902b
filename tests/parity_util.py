"""Helpers for the GPU parity tests: run the HIP path, run the oracle on the
same (already rounded) inputs, and compare with the stated tolerances."""

from __future__ import annotations

import sys

import numpy as np
import torch

import exact_attention_115_amd as fa
import oracle
from synth import to_f64

# Tolerances. Forward O: float32 max-abs 1e-5; 16-bit max-abs 2e-2 and
# mean-abs 2e-3. Gradients: per-tensor Frobenius relative error 5e-2.
# LSE (not in the stated bar, our own): 1e-4 float32, 1e-3 16-bit.
TOL = {
    "f32": dict(o_max=1e-5, lse=1e-4),
    "bf16": dict(o_max=2e-2, o_mean=2e-3, lse=1e-3, grad_rel=5e-2),
    "f16": dict(o_max=2e-2, o_mean=2e-3, lse=1e-3, grad_rel=5e-2),
}

DT_NAME = {torch.float32: "f32", torch.bfloat16: "bf16", torch.float16: "f16"}


def say(*a):
    print(*a, flush=True)
    sys.stdout.flush()


def gpu(t):
    return None if t is None else t.to("cuda").contiguous()


def run_forward(q, k, v, causal, scale):
    """q, k, v CPU tensors -> (O, LSE) of the HIP path as float64 numpy."""
    o, lse = fa.forward(gpu(q), gpu(k), gpu(v), causal=causal, scale=scale)
    torch.cuda.synchronize()
    return o, lse


def forward_nan_filled(qg, kg, vg, causal, scale):
    """fa_fwd on device tensors into NaN-filled o / lse (so an element the
    kernels never write stays NaN and fails the finiteness checks)."""
    B, Hq, Nq, d = qg.shape
    Hkv, Nkv = kg.shape[1], kg.shape[2]
    o = torch.full_like(qg, float("nan"))
    lse = torch.full((B, Hq, Nq), float("nan"), dtype=torch.float32, device=qg.device)
    nbytes = fa.fa_fwd_workspace_size(B, Hq, Hkv, Nq, Nkv, d, qg.dtype)
    ws = torch.full((nbytes,), 0xFF, dtype=torch.uint8, device=qg.device) if nbytes else None
    st = fa.fa_fwd(qg, kg, vg, o, lse, ws, scale, causal)
    assert st == 0, fa.fa_strerror(st)
    return o, lse


def backward_nan_filled(qg, kg, vg, o, lse, dog, causal, scale):
    """fa_bwd into NaN-filled dq / dk / dv and a NaN-filled workspace."""
    B, Hq, Nq, d = qg.shape
    Hkv, Nkv = kg.shape[1], kg.shape[2]
    dq, dk, dv = (torch.full_like(t, float("nan")) for t in (qg, kg, vg))
    nbytes = fa.fa_bwd_workspace_size(B, Hq, Hkv, Nq, Nkv, d, qg.dtype)
    ws = torch.full((nbytes,), 0xFF, dtype=torch.uint8, device=qg.device) if nbytes else None
    st = fa.fa_bwd(qg, kg, vg, o, lse, dog, dq, dk, dv, ws, scale, causal)
    assert st == 0, fa.fa_strerror(st)
    return dq, dk, dv


def all_finite(name, t):
    """Every element finite (an element left unwritten in a NaN-filled
    output is caught here)."""
    bad = int((~torch.isfinite(t)).sum().item())
    say(f"  {name}: {t.numel()} elements, {bad} not finite")
    assert bad == 0, f"{name}: {bad} elements not finite (unwritten or overflowed)"


def lse_compare(got, ref, tol):
    got = np.asarray(got, dtype=np.float64)
    ref = np.asarray(ref, dtype=np.float64)
    fin = np.isfinite(ref)
    assert np.array_equal(np.isfinite(got), fin), "LSE finiteness differs"
    assert np.all(np.isneginf(got[~fin])), "rows with no visible key must have LSE = -inf"
    err = float(np.max(np.abs(got[fin] - ref[fin]))) if fin.any() else 0.0
    assert err <= tol, f"LSE max-abs {err:.3e} > {tol}"
    return err


def check_forward(o_gpu, lse_gpu, o_ref, lse_ref, dtype: str, label: str = ""):
    """Compare HIP outputs (torch, any device) with oracle outputs (numpy)."""
    tol = TOL[dtype]
    o = to_f64(o_gpu)
    lse = to_f64(lse_gpu)
    assert np.all(np.isfinite(o)), "non-finite output"
    diff = np.abs(o - o_ref)
    mx = float(diff.max()) if diff.size else 0.0
    mean = float(diff.mean()) if diff.size else 0.0
    lerr = lse_compare(lse, lse_ref, tol["lse"])
    say(f"  [{label}] O max-abs {mx:.3e} mean-abs {mean:.3e}  LSE max-abs {lerr:.3e}")
    assert mx <= tol["o_max"], f"O max-abs {mx:.3e} > {tol['o_max']}"
    if "o_mean" in tol:
        assert mean <= tol["o_mean"], f"O mean-abs {mean:.3e} > {tol['o_mean']}"
    return mx, mean, lerr


def rel_fro(got, ref):
    n = np.linalg.norm(ref)
    return float(np.linalg.norm(got - ref) / (n if n > 0 else 1.0))


# Element-wise gradient checks (besides the stated per-tensor Frobenius bar).
# With u the unit roundoff of the 16-bit format (2^-8 bf16, 2^-11 fp16), sub
# the absolute error of a tiny value (half of fp16's smallest subnormal,
# 2^-25; for bf16 float32's smallest normal 2^-126, below which the float32
# arithmetic may flush to zero) and the oracle's
# magnitude sums (oracle.bounds: M the sum of the terms' magnitudes, R their
# root-sum-square, L dQ's common-mode part, C the subnormal counts):
#  * per tensor: max |g - ref| <= GRAD_MAX_REL * max |ref|;
#  * per element, the worst-case rounding bound
#      |g - ref| <= SAFETY (f u M + u |ref| + sub (C + 1)),
#    f = 1 for dV (P rounded once) and 2 for dQ, dK (dS rounded, and D
#    formed from the rounded O), u |ref| for rounding the result; SAFETY = 2
#    for the float32 sums and exponentials the derivation leaves out;
#  * per row (a key's dK / dV row, a query's dQ row, of d elements): the
#    stated 5e-2 relative bar, plus what independent roundings of the terms
#    add up to (a random walk, about u R / sqrt(3) per element; ROW_LAMBDA u
#    R allows 10x that), plus the common-mode and result terms:
#      ||g_r - ref_r|| <= GRAD_ROW_REL ||ref_r|| + ROW_LAMBDA u ||R_r||
#                         + SAFETY (u ||L_r|| + u ||ref_r|| + sub ||C_r + 1||).
#    A row that is wrong as a whole (e.g. left unwritten, or computed from
#    another row's data) has an error of the size of ||ref_r|| and fails it
#    unless cancellation made ||ref_r|| tiny against the terms.
GRAD_MAX_REL = 2e-2
GRAD_ROW_REL = 5e-2
ROW_LAMBDA = 6.0
UNIT_ROUNDOFF = {"bf16": 2.0 ** -8, "f16": 2.0 ** -11}
SUBNORMAL_HALF = {"bf16": 2.0 ** -126, "f16": 2.0 ** -25}
SAFETY = 2.0


def _rows(x, d):
    return np.linalg.norm(np.asarray(x, dtype=np.float64).reshape(-1, d), axis=1)


def check_grads(grads_gpu, grads_ref, dtype: str, label: str = "", mags=None):
    """grads_gpu: (dq, dk, dv) of the HIP path; grads_ref: the oracle's; mags:
    the oracle.bounds magnitudes (Mq, Mk, Mv, Cq, Ck, Cv, Rq, Rk, Rv, Lq),
    shaped like the gradients."""
    tol = TOL[dtype]["grad_rel"]
    u, sub = UNIT_ROUNDOFF[dtype], SUBNORMAL_HALF[dtype]
    out = {}
    for i, (name, g, r) in enumerate(zip(("dq", "dk", "dv"), grads_gpu, grads_ref)):
        gg = to_f64(g)
        r = np.asarray(r, dtype=np.float64)
        assert gg.shape == r.shape, f"{name} shape {gg.shape} vs {r.shape}"
        assert np.all(np.isfinite(gg)), f"non-finite {name}"
        rel = rel_fro(gg, r)
        err = np.abs(gg - r)
        scale = float(np.max(np.abs(r))) if r.size else 0.0
        mx = float(err.max()) / scale if scale > 0 else float(err.max()) if err.size else 0.0
        msg = f"  [{label}] {name}: Frobenius rel {rel:.3e}  max-abs/max|ref| {mx:.3e}"
        res = dict(fro=rel, max_rel=mx)
        elem_used = row_used = None
        if mags is not None and r.size:
            m, c, rr = (np.asarray(mags[j]) for j in (i, i + 3, i + 6))
            lin = np.asarray(mags[9]) if name == "dq" else np.zeros_like(r)
            f = 1.0 if name == "dv" else 2.0
            bound = SAFETY * (f * u * m + u * np.abs(r) + sub * (c + 1.0))
            ratio = err / np.maximum(bound, 1e-300)
            elem_used = float(ratio.max())
            d = r.shape[-1]
            row_allow = (GRAD_ROW_REL * _rows(r, d) + ROW_LAMBDA * u * _rows(rr, d)
                         + SAFETY * (u * _rows(lin, d) + u * _rows(r, d) + sub * _rows(c + 1.0, d)))
            row_ratio = _rows(gg - r, d) / np.maximum(row_allow, 1e-300)
            row_used = float(row_ratio.max())
            msg += f"  element bound used {elem_used:.3f}  row bound used {row_used:.3f}"
            if elem_used > 1.0 or row_used > 1.0:
                j = np.unravel_index(int(np.argmax(ratio)), r.shape)
                rw = int(np.argmax(row_ratio))
                msg += (f"\n    worst element {j}: got {gg[j]:.6e} ref {r[j]:.6e} M {m[j]:.3e} "
                        f"C {c[j]:.3e} bound {bound[j]:.3e}"
                        f"\n    worst row {rw} (flattened): |err| {_rows(gg - r, d)[rw]:.3e} "
                        f"|ref| {_rows(r, d)[rw]:.3e} |R| {_rows(rr, d)[rw]:.3e} "
                        f"allowed {row_allow[rw]:.3e}")
        res.update(element_bound_used=elem_used, row_bound_used=row_used)
        out[name] = res
        say(msg)
        assert rel <= tol, f"{name} relative error {rel:.3e} > {tol}"
        assert mx <= GRAD_MAX_REL, f"{name} max-abs/max|ref| {mx:.3e} > {GRAD_MAX_REL}"
        if elem_used is not None:
            assert elem_used <= 1.0, f"{name} exceeds the element rounding bound by {elem_used:.3f}x"
            assert row_used <= 1.0, f"{name} exceeds the row bound by {row_used:.3f}x"
    return out


def sample_heads(B, Hq, n=3):
    """Deterministic sample of (b, h) pairs: first, last and middle heads."""
    cand = [(0, 0), (B - 1, Hq - 1), (B // 2, Hq // 2), (0, Hq - 1), (B - 1, 0)]
    seen = []
    for x in cand:
        if x not in seen:
            seen.append(x)
    return seen[:n]


def oracle_heads_forward(q, k, v, causal, scale, heads):
    """Oracle O, LSE for the sampled heads only ([len(heads), N_q, d])."""
    G = q.shape[1] // k.shape[1]
    os_, ls = [], []
    for b, h in heads:
        o, l = oracle.head_forward(to_f64(q[b, h]), to_f64(k[b, h // G]), to_f64(v[b, h // G]),
                                   causal, scale)
        os_.append(o)
        ls.append(l)
    return np.stack(os_), np.stack(ls)


def oracle_heads_backward(q, k, v, do, causal, scale, heads_kv, with_mags=False):
    """Oracle dq (per q head), dk, dv (per kv head) for the sampled kv heads:
    every q head of each sampled group contributes, as in the full result.
    With ``with_mags`` each entry also carries the group's magnitude sums
    (oracle.bounds) as a fourth element."""
    G = q.shape[1] // k.shape[1]
    res = []
    for b, hk in heads_kv:
        dk = np.zeros(k.shape[2:])
        dv = np.zeros(v.shape[2:])
        dqs = []
        for h in range(hk * G, (hk + 1) * G):
            dq, dkh, dvh = oracle.head_backward(to_f64(q[b, h]), to_f64(k[b, hk]), to_f64(v[b, hk]),
                                                to_f64(do[b, h]), causal, scale)
            dk += dkh
            dv += dvh
            dqs.append(dq)
        entry = (np.stack(dqs), dk, dv)
        if with_mags:
            sl_q = slice(hk * G, (hk + 1) * G)
            entry = entry + (oracle.group_backward_magnitudes(
                to_f64(q[b:b + 1, sl_q]), to_f64(k[b:b + 1, hk:hk + 1]), to_f64(v[b:b + 1, hk:hk + 1]),
                to_f64(do[b:b + 1, sl_q]), causal, scale, 0, 0),)
        res.append(entry)
    return res


def full_magnitudes(q, k, v, do, causal, scale):
    return oracle.attention_backward_magnitudes(to_f64(q), to_f64(k), to_f64(v), to_f64(do),
                                                causal, scale)
