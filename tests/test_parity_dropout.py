"""GPU parity of dropout (fa_fwd_dropout, fa_bwd_dropout, fa_dropout_mask)
against the float64 oracle in oracle/dropout.py.

The keep mask is integer work and must match bit for bit. Outputs use the
forward's 16-bit bar scaled by r = 1 / (1 - p_eff): every kept probability,
and so O itself, is multiplied by r before the output is rounded, so the
rounding error (a fixed number of units in the last place of O) grows by the
same factor. LSE does not depend on the mask and keeps its own bar. Gradients
keep the relative bar of the plain backward (it is scale-free).
"""

import numpy as np
import pytest
import torch

import exact_attention_115_amd as fa
import oracle
from oracle import dropout as drop
from parity_util import TOL, check_grads, gpu, say
from synth import WORKLOADS, make_inputs, random_tensors, to_f64

pytestmark = pytest.mark.gpu


def f32(p):
    """The probability as the library receives it (a C float)."""
    return float(np.float32(p))


def check_dropout_forward(o, lse, o_ref, lse_ref, dtype, p, label):
    r = drop.keep_scale(f32(p))
    tol = TOL[dtype]
    og, lg = to_f64(o), to_f64(lse)
    assert np.all(np.isfinite(og)), "non-finite output"
    diff = np.abs(og - o_ref)
    mx, mean = float(diff.max()), float(diff.mean())
    fin = np.isfinite(lse_ref)
    assert np.array_equal(np.isfinite(lg), fin)
    lerr = float(np.max(np.abs(lg[fin] - lse_ref[fin]))) if fin.any() else 0.0
    say(f"  [{label}] r={r:.4f} O max-abs {mx:.3e} mean-abs {mean:.3e} LSE max-abs {lerr:.3e}")
    assert mx <= tol["o_max"] * r, mx
    assert mean <= tol["o_mean"] * r, mean
    assert lerr <= tol["lse"], lerr


@pytest.mark.parametrize("shape", [(1, 2, 5, 70), (2, 3, 33, 129), (1, 1, 1, 1000), (1, 2, 64, 64)])
@pytest.mark.parametrize("p,seed,offset", [(0.1, 7, 0), (0.5, 2**40 + 3, 11), (0.9, 0, 2**63 + 5)])
def test_mask_bit_exact(shape, p, seed, offset):
    B, Hq, Nq, Nkv = shape
    say(f"mask {shape} p={p} seed={seed} offset={offset}")
    keep = fa.dropout_mask(B, Hq, Nq, Nkv, p, seed, offset).cpu().numpy()
    for b in range(B):
        for h in range(Hq):
            ref = drop.keep_mask(b * Hq + h, np.arange(Nq), Nkv, f32(p), seed, offset)
            assert np.array_equal(keep[b, h].astype(bool), ref), (b, h)


def test_mask_zero_probability_keeps_everything():
    keep = fa.dropout_mask(1, 2, 17, 45, 0.0, 3, 0)
    assert bool((keep == 1).all())


CASES = [
    # B, Hq, Hkv, Nq, Nkv, d, causal, dtype, p
    (1, 4, 2, 200, 300, 64, True, "bf16", 0.2),
    (2, 4, 4, 130, 130, 128, False, "f16", 0.5),
    (1, 2, 1, 1, 500, 128, True, "bf16", 0.3),
    (1, 8, 2, 1000, 1000, 128, True, "bf16", 0.1),
    (3, 6, 3, 65, 129, 64, True, "f16", 0.75),
]


@pytest.mark.parametrize("case", CASES, ids=[str(c) for c in CASES])
def test_forward_dropout_parity(case):
    B, Hq, Hkv, Nq, Nkv, d, causal, dtype, p = case
    scale = 1.0 / np.sqrt(d)
    seed, offset = 1234 + Nq, 5
    say(f"forward dropout {case}")
    q, k, v, _ = random_tensors((B, Hq, Nq, d), (B, Hkv, Nkv, d), dtype, seed=77)
    o, lse = fa.forward_dropout(gpu(q), gpu(k), gpu(v), p, seed, offset, causal=causal, scale=scale)
    torch.cuda.synchronize()
    o_ref, lse_ref = drop.attention_forward_dropout(to_f64(q), to_f64(k), to_f64(v), causal, scale,
                                                    f32(p), seed, offset)
    check_dropout_forward(o, lse, o_ref, lse_ref, dtype, p, str(case))


@pytest.mark.parametrize("causal", [True, False])
def test_forward_dropout_long_sampled_heads(causal):
    """256-row workgroups (N_q >= 4096, enough tiles to fill the GPU), ragged
    tail, sampled heads."""
    w = WORKLOADS["c3"].replace(name="drop_long", Hq=16, Hkv=16, Nq=4100, Nkv=4100,
                                causal=causal, seed=39)
    p, seed, offset = 0.25, 99, 3
    say(f"{w} p={p}")
    q, k, v, _ = make_inputs(w, with_grad=False)
    o, lse = fa.forward_dropout(gpu(q), gpu(k), gpu(v), p, seed, offset, causal=w.causal,
                                scale=w.scale)
    torch.cuda.synchronize()
    heads = [(0, 0), (0, w.Hq - 1)]
    o_ref, lse_ref = drop.attention_forward_dropout(to_f64(q), to_f64(k), to_f64(v), w.causal,
                                                    w.scale, f32(p), seed, offset, heads=heads)
    o_s = torch.stack([o[b, h] for b, h in heads])
    l_s = torch.stack([lse[b, h] for b, h in heads])
    check_dropout_forward(o_s, l_s, np.stack([o_ref[b, h] for b, h in heads]),
                          np.stack([lse_ref[b, h] for b, h in heads]), w.dtype, p,
                          f"long causal={causal}")


def test_forward_dropout_zero_probability_equals_forward():
    q, k, v, _ = random_tensors((2, 4, 300, 128), (2, 2, 300, 128), "bf16", seed=78)
    qg, kg, vg = gpu(q), gpu(k), gpu(v)
    o0, l0 = fa.forward(qg, kg, vg, causal=True)
    o1, l1 = fa.forward_dropout(qg, kg, vg, 0.0, 5, 0, causal=True)
    torch.cuda.synchronize()
    assert torch.equal(o0, o1) and torch.equal(l0, l1)


def test_forward_dropout_repeatable_and_mask_dependent():
    q, k, v, _ = random_tensors((1, 4, 256, 64), (1, 4, 256, 64), "bf16", seed=79)
    qg, kg, vg = gpu(q), gpu(k), gpu(v)
    a = fa.forward_dropout(qg, kg, vg, 0.3, 42, 0)
    b = fa.forward_dropout(qg, kg, vg, 0.3, 42, 0)
    c = fa.forward_dropout(qg, kg, vg, 0.3, 42, 1)
    torch.cuda.synchronize()
    assert torch.equal(a[0], b[0]) and torch.equal(a[1], b[1])
    assert not torch.equal(a[0], c[0])
    assert torch.equal(a[1], c[1])  # LSE does not depend on the mask


# ------------------------------------------------------------------ backward

def check_dropout_grads(grads, q, k, v, do, causal, scale, p, seed, offset, dtype, label):
    """Gradients against the dropout oracle, with the element-wise checks of
    parity_util.check_grads and its rounding bound on the magnitudes of the
    dropout backward's terms (the same keep masks)."""
    q64, k64, v64, do64 = to_f64(q), to_f64(k), to_f64(v), to_f64(do)
    g_ref = drop.attention_backward_dropout(q64, k64, v64, do64, causal, scale, f32(p), seed,
                                            offset)
    Hq, nq, nkv = q.shape[1], q.shape[2], k.shape[2]
    keep_of = lambda b, h: drop.keep_mask(b * Hq + h, np.arange(nq), nkv, f32(p), seed,  # noqa: E731
                                          offset)
    mags = oracle.attention_backward_magnitudes(q64, k64, v64, do64, causal, scale, keep_of,
                                                drop.keep_scale(f32(p)))
    check_grads(grads, g_ref, dtype, label, mags=mags)


BWD_CASES = [
    # B, Hq, Hkv, Nq, Nkv, d, causal, dtype, p
    (1, 4, 2, 200, 300, 64, True, "bf16", 0.2),
    (2, 4, 4, 130, 130, 128, False, "f16", 0.5),
    (1, 8, 1, 160, 96, 128, True, "bf16", 0.3),     # MQA: split head group, float32 partials
    (1, 8, 2, 1000, 1000, 128, True, "bf16", 0.1),
    (3, 6, 3, 65, 129, 64, True, "f16", 0.75),
]


@pytest.mark.parametrize("case", BWD_CASES, ids=[str(c) for c in BWD_CASES])
def test_backward_dropout_parity(case):
    B, Hq, Hkv, Nq, Nkv, d, causal, dtype, p = case
    scale = 1.0 / np.sqrt(d)
    seed, offset = 4321 + Nkv, 9
    say(f"backward dropout {case}")
    q, k, v, do = random_tensors((B, Hq, Nq, d), (B, Hkv, Nkv, d), dtype, seed=81, with_grad=True)
    qg, kg, vg, dog = gpu(q), gpu(k), gpu(v), gpu(do)
    o, lse = fa.forward_dropout(qg, kg, vg, p, seed, offset, causal=causal, scale=scale)
    grads = fa.backward_dropout(qg, kg, vg, o, lse, dog, p, seed, offset, causal=causal, scale=scale)
    torch.cuda.synchronize()
    check_dropout_grads(grads, q, k, v, do, causal, scale, p, seed, offset, dtype, str(case))


def test_backward_dropout_zero_probability_equals_backward():
    q, k, v, do = random_tensors((2, 4, 300, 128), (2, 2, 300, 128), "bf16", seed=82, with_grad=True)
    qg, kg, vg, dog = gpu(q), gpu(k), gpu(v), gpu(do)
    o, lse = fa.forward(qg, kg, vg, causal=True)
    a = fa.backward(qg, kg, vg, o, lse, dog, causal=True)
    b = fa.backward_dropout(qg, kg, vg, o, lse, dog, 0.0, 5, 0, causal=True)
    torch.cuda.synchronize()
    for x, y in zip(a, b):
        assert torch.equal(x, y)


def test_backward_dropout_long_sampled():
    """Long causal case (the 256-row dQ workgroups, 8 waves) on a reduced head
    count; the oracle's gradients are computed per head for two heads."""
    w = WORKLOADS["c3"].replace(name="drop_bwd_long", Hq=16, Hkv=16, Nq=4096, Nkv=4096, seed=40)
    p, seed, offset = 0.2, 17, 2
    q, k, v, do = make_inputs(w, with_grad=True)
    qg, kg, vg, dog = gpu(q), gpu(k), gpu(v), gpu(do)
    o, lse = fa.forward_dropout(qg, kg, vg, p, seed, offset, causal=True, scale=w.scale)
    dq, dk, dv = fa.backward_dropout(qg, kg, vg, o, lse, dog, p, seed, offset, causal=True,
                                     scale=w.scale)
    torch.cuda.synchronize()
    r = drop.keep_scale(f32(p))
    dq, dk, dv = dq.cpu(), dk.cpu(), dv.cpu()
    for h in (0, w.Hq - 1):
        z = drop.keep_mask(h, np.arange(w.Nq), w.Nkv, f32(p), seed, offset)
        args = (to_f64(q[0, h]), to_f64(k[0, h]), to_f64(v[0, h]), to_f64(do[0, h]), True, w.scale,
                z, r)
        g_ref = drop.head_backward_dropout(*args)
        mags = oracle.head_backward_magnitudes(*args)
        check_grads((dq[0, h], dk[0, h], dv[0, h]), g_ref, w.dtype, f"long head {h}", mags=mags)


@pytest.mark.parametrize("ramp", ["up", "wave"])
def test_dropout_under_score_ramps(ramp):
    """The rescale of the online softmax with dropout on: key rows scaled by a
    factor rising or oscillating along the sequence (scores to about 250
    natural-log units, a new maximum on every tile for "up"; see
    tests/test_parity_rescale.py); forward and backward against the oracle."""
    from synth import ramp_tensors

    B, Hq, Hkv, Nq, Nkv, d, causal, dtype, p = 1, 4, 2, 300, 500, 128, True, "bf16", 0.3
    scale = 1.0 / np.sqrt(d)
    seed, offset = 77 + len(ramp), 4
    say(f"dropout ramp {ramp}")
    q, k, v, do = ramp_tensors((B, Hq, Nq, d), (B, Hkv, Nkv, d), dtype, seed=83, ramp=ramp,
                               peak=32.0, with_grad=True)
    qg, kg, vg, dog = gpu(q), gpu(k), gpu(v), gpu(do)
    o, lse = fa.forward_dropout(qg, kg, vg, p, seed, offset, causal=causal, scale=scale)
    grads = fa.backward_dropout(qg, kg, vg, o, lse, dog, p, seed, offset, causal=causal,
                                scale=scale)
    torch.cuda.synchronize()
    o_ref, lse_ref = drop.attention_forward_dropout(to_f64(q), to_f64(k), to_f64(v), causal, scale,
                                                    f32(p), seed, offset)
    check_dropout_forward(o, lse, o_ref, lse_ref, dtype, p, f"ramp {ramp}")
    check_dropout_grads(grads, q, k, v, do, causal, scale, p, seed, offset, dtype, f"ramp {ramp}")
