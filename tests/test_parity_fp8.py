"""GPU parity of the FP8 (E4M3) forward (fa_fwd_fp8) against the float64
oracle in oracle/fp8.py.

The oracle is the definition on the decoded inputs; the kernel also rounds
the probabilities to E4M3 for the P V product, and its 8-bit matrix-core
products do not add their terms exactly. The bar per output element is the
sum of the oracle's bounds for those two effects (oracle.fp8.p_rounding_bound:
each normalised weight moves by at most max(2^-4 P, 2^-10);
oracle.fp8.accumulation_bound: every score moves by at most EPS8 * scale *
sum_c |q_c k_c|, every P V term by EPS8 of itself, EPS8 measured below),
plus the bf16 rounding of O (2^-8 |O|, twice its half-unit) and 1e-4 for
float32 sums. LSE: the accumulation bound plus 1e-4.
"""

import numpy as np
import pytest
import torch

import exact_attention_115_amd as fa
from oracle import fp8 as f8
from parity_util import say, to_f64

pytestmark = pytest.mark.gpu


def e4m3_inputs(B, Hq, Hkv, Nq, Nkv, seed, descales=(0.5, 0.25, 2.0)):
    """E4M3 codes of N(0, 1) draws divided by each tensor's descale factor."""
    g = torch.Generator(device="cpu").manual_seed(seed)
    dq, dk, dv = descales
    q = (torch.randn((B, Hq, Nq, 128), generator=g) / dq).to(torch.float8_e4m3fn)
    k = (torch.randn((B, Hkv, Nkv, 128), generator=g) / dk).to(torch.float8_e4m3fn)
    v = (torch.randn((B, Hkv, Nkv, 128), generator=g) / dv).to(torch.float8_e4m3fn)
    return q.view(torch.uint8), k.view(torch.uint8), v.view(torch.uint8)


def check_fp8(o, lse, q8, k8, v8, heads, causal, scale, descales, label):
    G = q8.shape[1] // k8.shape[1]
    dq, dk, dv = descales
    worst = 0.0
    for b, h in heads:
        qq, kk, vv = (x.numpy() for x in (q8[b, h], k8[b, h // G], v8[b, h // G]))
        o_ref, lse_ref = f8.head_forward_fp8(qq, kk, vv, causal, scale, dq, dk, dv)
        bound = f8.p_rounding_bound(qq, kk, vv, causal, scale, dq, dk, dv)
        o_acc, lse_acc = f8.accumulation_bound(qq, kk, vv, causal, scale, dq, dk, dv)
        og = to_f64(o[b, h])
        lg = to_f64(lse[b, h])
        assert np.all(np.isfinite(og))
        err = np.abs(og - o_ref)
        allowed = bound + o_acc + 2.0 ** -8 * np.abs(o_ref) + 1e-4
        worst = max(worst, float(np.max(err / allowed)))
        fin = np.isfinite(lse_ref)
        assert np.array_equal(np.isfinite(lg), fin)
        lerr_all = np.abs(lg[fin] - lse_ref[fin])
        lallow = lse_acc[fin] + 1e-4
        lerr = float(lerr_all.max()) if fin.any() else 0.0
        lused = float(np.max(lerr_all / lallow)) if fin.any() else 0.0
        say(f"  [{label} head {b},{h}] O max-abs {err.max():.3e} (max |O| {np.abs(o_ref).max():.2f}), "
            f"worst err/bound {float(np.max(err / allowed)):.3f}, LSE max-abs {lerr:.3e} "
            f"(largest score {float(np.max(np.where(fin, lse_ref, -np.inf))):.1f}, "
            f"LSE bound used {lused:.3f})")
        assert np.all(err <= allowed), float(np.max(err / allowed))
        assert np.all(lerr_all <= lallow), lused
    return worst


CASES = [
    # B, Hq, Hkv, Nq, Nkv, causal
    (1, 4, 2, 200, 300, True),
    (2, 8, 8, 1000, 1000, False),
    (1, 2, 1, 1, 700, False),
    (1, 2, 2, 130, 70, True),       # N_q > N_kv: the first rows see no key
    (3, 6, 3, 65, 129, True),
]


@pytest.mark.parametrize("case", CASES, ids=[str(c) for c in CASES])
def test_fp8_forward_parity(case):
    B, Hq, Hkv, Nq, Nkv, causal = case
    scale = 1.0 / np.sqrt(128)
    descales = (0.5, 0.25, 2.0)
    say(f"fp8 forward {case}")
    q8, k8, v8 = e4m3_inputs(B, Hq, Hkv, Nq, Nkv, seed=101 + Nq, descales=descales)
    o, lse = fa.forward_fp8(q8.cuda(), k8.cuda(), v8.cuda(), *descales, causal=causal, scale=scale)
    torch.cuda.synchronize()
    heads = sorted({(0, 0), (B - 1, Hq - 1), (B // 2, Hq // 2)})
    check_fp8(o.cpu(), lse.cpu(), q8, k8, v8, heads, causal, scale, descales, str(case))


@pytest.mark.parametrize("causal", [True, False])
def test_fp8_forward_long_sampled(causal):
    """256-row workgroups (N_q >= 4096 and enough tiles to fill the GPU) with a
    ragged tail; two sampled heads."""
    B, Hq, Hkv, N = 1, 16, 16, 4100
    scale = 1.0 / np.sqrt(128)
    descales = (1.0, 1.0, 1.0)
    q8, k8, v8 = e4m3_inputs(B, Hq, Hkv, N, N, seed=111, descales=descales)
    o, lse = fa.forward_fp8(q8.cuda(), k8.cuda(), v8.cuda(), *descales, causal=causal, scale=scale)
    torch.cuda.synchronize()
    check_fp8(o.cpu(), lse.cpu(), q8, k8, v8, [(0, 0), (0, Hq - 1)], causal, scale, descales,
              f"long causal={causal}")


def test_fp8_forward_no_keys_and_repeatable():
    q8, k8, v8 = e4m3_inputs(1, 2, 2, 40, 64, seed=113)
    qg, kg, vg = q8.cuda(), k8.cuda(), v8.cuda()
    o1, l1 = fa.forward_fp8(qg, kg, vg, 0.5, 0.25, 2.0, causal=True)
    o2, l2 = fa.forward_fp8(qg, kg, vg, 0.5, 0.25, 2.0, causal=True)
    torch.cuda.synchronize()
    assert torch.equal(o1, o2) and torch.equal(l1, l2)
    empty = torch.empty((1, 2, 0, 128), dtype=torch.uint8, device="cuda")
    o3, l3 = fa.forward_fp8(qg, empty, empty, causal=False)
    torch.cuda.synchronize()
    assert bool((o3 == 0).all()) and bool(torch.isneginf(l3).all())


RAMP_CASES = [
    # B, Hq, Hkv, Nq, Nkv, causal
    (1, 4, 2, 300, 700, True),
    (2, 2, 1, 1, 2000, False),
]


@pytest.mark.parametrize("ramp", ["up", "down", "wave"])
@pytest.mark.parametrize("case", RAMP_CASES, ids=[str(c) for c in RAMP_CASES])
def test_fp8_forward_under_score_ramps(case, ramp):
    """The online-softmax rescale of the FP8 kernel: key rows scaled by a
    factor rising, falling or oscillating along the sequence (see
    tests/test_parity_rescale.py), quantised to E4M3 with descale factors 1.

    Peak factor 32, as in the 16-bit tests: scores reach about 250
    natural-log units and, for "up", every 64-key tile raises each row's
    maximum past the kernel's rescale threshold. At that size the inexact
    sums of the 8-bit products move the scores by up to EPS8 * scale *
    sum_c |q_c k_c| (measured by test_fp8_score_accumulation_error), which
    the O and LSE bars include (oracle.fp8.accumulation_bound)."""
    from synth import ramp_tensors

    B, Hq, Hkv, Nq, Nkv, causal = case
    scale = 1.0 / np.sqrt(128)
    descales = (1.0, 1.0, 1.0)
    say(f"fp8 ramp {ramp} {case}")
    q, k, v, _ = ramp_tensors((B, Hq, Nq, 128), (B, Hkv, Nkv, 128), "f32", seed=121 + Nq,
                              ramp=ramp, peak=32.0)
    assert float(k.abs().max()) < 448.0
    q8, k8, v8 = (x.to(torch.float8_e4m3fn).view(torch.uint8) for x in (q, k, v))
    o, lse = fa.forward_fp8(q8.cuda(), k8.cuda(), v8.cuda(), *descales, causal=causal, scale=scale)
    torch.cuda.synchronize()
    heads = sorted({(0, 0), (B - 1, Hq - 1)})
    check_fp8(o.cpu(), lse.cpu(), q8, k8, v8, heads, causal, scale, descales, f"{ramp} {case}")


# ------------------------------------------- 8-bit accumulation, measured

# Bound on the error of the 8-bit matrix-core products, relative to the sum
# of the magnitudes of the terms each sums: EPS8 * sum_c |x_c y_c|. Measured
# by test_fp8_score_accumulation_error below (largest seen: 2^-12.27).
EPS8 = f8.EPS8


@pytest.mark.parametrize("dist", ["normal", "all_codes", "wide"])
def test_fp8_score_accumulation_error(dist):
    """With one key, the softmax is a single weight 1, so LSE_i = scale * s_i:
    the LSE returns each score as the 8-bit matrix-core products computed it.
    Compare with the exact dot product of the decoded inputs: the error must
    stay within EPS8 * scale * sum_c |q_ic k_c|, the term the O / LSE bound
    (oracle.fp8.accumulation_bound) is built on. Three operand mixes:
    N(0, 1) draws, uniformly random codes (every finite E4M3 value, so the
    64 products of one instruction span the whole exponent range), and
    N(0, 1) rows scaled by powers of two from 2^-6 to 2^6 per element."""
    B, H, Nq = 16, 8, 256
    g = torch.Generator(device="cpu").manual_seed({"normal": 131, "all_codes": 132, "wide": 133}[dist])
    if dist == "normal":
        q = torch.randn((B, H, Nq, 128), generator=g)
        k = torch.randn((B, H, 1, 128), generator=g)
    elif dist == "wide":
        e = lambda s: torch.randint(-6, 7, s, generator=g).float()  # noqa: E731
        q = torch.randn((B, H, Nq, 128), generator=g) * torch.exp2(e((B, H, Nq, 128)))
        k = torch.randn((B, H, 1, 128), generator=g) * torch.exp2(e((B, H, 1, 128)))
    if dist == "all_codes":
        codes = lambda s: torch.randint(0, 256, s, generator=g, dtype=torch.uint8)  # noqa: E731
        q8, k8 = codes((B, H, Nq, 128)), codes((B, H, 1, 128))
        for t in (q8, k8):
            t[(t & 0x7F) == 0x7F] = 0x38  # no NaN codes
    else:
        q8 = q.to(torch.float8_e4m3fn).view(torch.uint8)
        k8 = k.to(torch.float8_e4m3fn).view(torch.uint8)
    scale = 1.0 / np.sqrt(128)
    o, lse = fa.forward_fp8(q8.cuda(), k8.cuda(), k8.cuda(), causal=False, scale=scale)
    torch.cuda.synchronize()
    qd, kd = f8.decode(q8.numpy()), f8.decode(k8.numpy())
    exact = scale * np.einsum("bhic,bhc->bhi", qd, kd[:, :, 0])
    mag = scale * np.einsum("bhic,bhc->bhi", np.abs(qd), np.abs(kd[:, :, 0]))
    got = to_f64(lse.cpu())
    rel = np.abs(got - exact) / np.maximum(mag, 1e-30)
    worst = float(rel.max())
    say(f"  [{dist}] largest score error / (scale sum |q k|): {worst:.3e} = 2^{np.log2(max(worst, 1e-30)):.2f}"
        f" over {rel.size} scores (EPS8 = 2^{np.log2(EPS8):.1f})")
    assert worst <= EPS8
