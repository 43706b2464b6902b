"""GPU parity of the backward (fa_bwd) against the float64 oracle.

The backward consumes the library's own forward outputs (O, LSE); the oracle
computes the gradients of sum(dO * O) from q, k, v, dO alone.
"""

import math

import numpy as np
import pytest
import torch

import exact_attention_115_amd as fa
import oracle
from synth import WORKLOADS, make_inputs, random_tensors, to_f64
from tests.parity_util import (all_finite, backward_nan_filled, check_grads, forward_nan_filled,
                               full_magnitudes, gpu, oracle_heads_backward, say)

pytestmark = [
    pytest.mark.gpu,
    pytest.mark.skipif(not torch.cuda.is_available(), reason="needs a GPU"),
]


def run_fwd_bwd(q, k, v, do, causal, scale):
    qg, kg, vg, dog = gpu(q), gpu(k), gpu(v), gpu(do)
    o, lse = fa.forward(qg, kg, vg, causal=causal, scale=scale)
    dq, dk, dv = fa.backward(qg, kg, vg, o, lse, dog, causal=causal, scale=scale)
    torch.cuda.synchronize()
    return (o, lse), (dq, dk, dv)


def full_oracle_bwd(q, k, v, do, causal, scale):
    return oracle.attention_backward(to_f64(q), to_f64(k), to_f64(v), to_f64(do), causal, scale)


@pytest.mark.parametrize("name", ["c2", "c2c"])
def test_c2_backward(name):
    w = WORKLOADS[name]
    say(f"{name}: {w}")
    q, k, v, do = make_inputs(w)
    _, grads = run_fwd_bwd(q, k, v, do, w.causal, w.scale)
    check_grads(grads, full_oracle_bwd(q, k, v, do, w.causal, w.scale), w.dtype, name,
                mags=full_magnitudes(q, k, v, do, w.causal, w.scale))


# kv heads compared with the oracle at full size. The grids keep all
# workgroups of kv head h on XCD h mod 8; at c3 the four heads lie on four
# different XCDs and include both ends of the head range.
FULL_KV_HEADS = {
    "c3": [(0, 0), (0, 9), (0, 22), (0, 31)],
    "c4": [(0, 0), (0, 31)],
    "c5g": [(0, 0), (3, 7)],
    "c5m": [(2, 0)],
}


@pytest.mark.parametrize("name", ["c3", "c4", "c5g", "c5m"])
def test_full_size_backward_sampled_heads(name):
    """Full-size launch (the bench's launch configuration) into NaN-filled
    gradient buffers and workspace: every element must be written and finite.
    The oracle computes complete kv-head groups (every q head that reads a
    sampled kv head), which is all dK / dV of that head depend on; each is
    compared element by element."""
    w = WORKLOADS[name]
    say(f"{name}: {w}")
    q, k, v, do = make_inputs(w)
    qg, kg, vg, dog = gpu(q), gpu(k), gpu(v), gpu(do)
    o, lse = forward_nan_filled(qg, kg, vg, w.causal, w.scale)
    dq, dk, dv = backward_nan_filled(qg, kg, vg, o, lse, dog, w.causal, w.scale)
    torch.cuda.synchronize()
    for nm, t in (("o", o), ("lse", lse), ("dq", dq), ("dk", dk), ("dv", dv)):
        all_finite(f"{name} {nm}", t)
    G = w.Hq // w.Hkv
    heads_kv = FULL_KV_HEADS[name]
    refs = oracle_heads_backward(q, k, v, do, w.causal, w.scale, heads_kv, with_mags=True)
    dq, dk, dv = dq.cpu(), dk.cpu(), dv.cpu()
    for (b, hk), (dq_r, dk_r, dv_r, mags) in zip(heads_kv, refs):
        dq_g = dq[b, hk * G:(hk + 1) * G]
        check_grads((dq_g, dk[b, hk], dv[b, hk]), (dq_r, dk_r, dv_r), w.dtype,
                    f"{name} kv head {(b, hk)}", mags=mags)


@pytest.mark.parametrize("causal", [False, True])
def test_long_ragged_backward_sampled_heads(causal):
    """256-row dQ workgroups and many key blocks (N >= 4096), ragged last
    tiles, causal and not."""
    w = WORKLOADS["c3"].replace(name="long_ragged", Hq=16, Hkv=16, Nq=4100, Nkv=4100,
                                causal=causal, seed=38)
    say(f"{w}")
    q, k, v, do = make_inputs(w)
    qg, kg, vg, dog = gpu(q), gpu(k), gpu(v), gpu(do)
    o, lse = forward_nan_filled(qg, kg, vg, w.causal, w.scale)
    dq, dk, dv = backward_nan_filled(qg, kg, vg, o, lse, dog, w.causal, w.scale)
    torch.cuda.synchronize()
    for nm, t in (("dq", dq), ("dk", dk), ("dv", dv)):
        all_finite(f"long ragged {nm}", t)
    heads_kv = [(0, 0), (0, w.Hkv - 1)]
    refs = oracle_heads_backward(q, k, v, do, w.causal, w.scale, heads_kv, with_mags=True)
    dq, dk, dv = dq.cpu(), dk.cpu(), dv.cpu()
    for (b, hk), (dq_r, dk_r, dv_r, mags) in zip(heads_kv, refs):
        check_grads((dq[b, hk:hk + 1], dk[b, hk], dv[b, hk]), (dq_r, dk_r, dv_r), w.dtype,
                    f"long ragged causal={causal} kv head {hk}", mags=mags)


EDGE = [
    # (B, Hq, Hkv, Nq, Nkv, d, causal)
    (1, 2, 2, 300, 300, 64, True),
    (1, 2, 2, 300, 300, 128, False),
    (2, 4, 2, 200, 333, 128, True),    # N_q < N_kv, GQA
    (1, 4, 1, 333, 200, 64, True),     # N_q > N_kv: rows with no visible key, MQA
    (1, 2, 2, 1, 1, 64, False),
    (1, 2, 2, 5, 1, 128, False),
    (1, 2, 2, 130, 7, 64, True),
    (1, 2, 1, 1, 1000, 128, True),     # single query row
    (3, 6, 3, 65, 129, 64, True),
    (1, 2, 2, 7, 300, 64, False),      # few queries, many keys
]


@pytest.mark.parametrize("dtype", ["bf16", "f16"])
@pytest.mark.parametrize("case", EDGE, ids=[str(c) for c in EDGE])
def test_backward_edge_cases(dtype, case):
    B, Hq, Hkv, nq, nkv, d, causal = case
    say(f"bwd edge {dtype} {case}")
    q, k, v, do = random_tensors((B, Hq, nq, d), (B, Hkv, nkv, d), dtype, seed=nq * 5 + nkv, with_grad=True)
    scale = 1.0 / math.sqrt(d)
    _, grads = run_fwd_bwd(q, k, v, do, causal, scale)
    ref = full_oracle_bwd(q, k, v, do, causal, scale)
    check_grads(grads, ref, dtype, str(case), mags=full_magnitudes(q, k, v, do, causal, scale))


def test_rows_without_keys_pass_no_gradient():
    say("bwd masked rows")
    q, k, v, do = random_tensors((1, 2, 100, 64), (1, 2, 40, 64), "bf16", seed=9, with_grad=True)
    _, (dq, dk, dv) = run_fwd_bwd(q, k, v, do, True, 0.125)
    # Rows 0..59 see no key (bottom-right causal, 100 queries, 40 keys).
    assert torch.all(dq[:, :, :60] == 0)


def test_gqa_backward_equals_summed_mha():
    say("bwd gqa vs mha")
    q, k, v, do = random_tensors((1, 8, 200, 128), (1, 2, 200, 128), "bf16", seed=11, with_grad=True)
    _, (dq1, dk1, dv1) = run_fwd_bwd(q, k, v, do, True, 0.09)
    kr, vr = k.repeat_interleave(4, dim=1), v.repeat_interleave(4, dim=1)
    _, (dq2, dk2, dv2) = run_fwd_bwd(q, kr, vr, do, True, 0.09)
    dk2s = dk2.float().reshape(1, 2, 4, 200, 128).sum(dim=2)
    dv2s = dv2.float().reshape(1, 2, 4, 200, 128).sum(dim=2)
    rel = lambda a, b: ((a.float() - b.float()).norm() / b.float().norm()).item()
    assert rel(dq1, dq2) <= 1e-2
    assert rel(dk1, dk2s) <= 1e-2
    assert rel(dv1, dv2s) <= 1e-2


def test_key_gradients_sum_to_zero():
    """Each softmax row's dS sums to zero, so sum_j dK_j = 0 per kv head."""
    say("bwd dk sum")
    q, k, v, do = random_tensors((1, 4, 256, 64), (1, 4, 256, 64), "f16", seed=12, with_grad=True)
    _, (dq, dk, dv) = run_fwd_bwd(q, k, v, do, True, 0.125)
    s = dk.float().sum(dim=2).abs().max().item()
    assert s <= 2e-2 * dk.float().abs().max().item() * 16


def test_stages_equal_fused_and_deterministic():
    say("bwd stages")
    w = WORKLOADS["c2c"]
    q, k, v, do = make_inputs(w)
    qg, kg, vg, dog = gpu(q), gpu(k), gpu(v), gpu(do)
    o, lse = fa.forward(qg, kg, vg, causal=True)
    dq1, dk1, dv1 = fa.backward(qg, kg, vg, o, lse, dog, causal=True)
    ws = torch.empty(fa.fa_bwd_workspace_size(*q.shape[:2], k.shape[1], q.shape[2], k.shape[2],
                                              q.shape[3], q.dtype), dtype=torch.uint8, device="cuda")
    dq2, dk2, dv2 = (torch.full_like(t, float("nan")) for t in (dq1, dk1, dv1))
    for stage in range(3):
        assert fa.fa_bwd_stage(stage, qg, kg, vg, o, lse, dog, dq2, dk2, dv2, ws, w.scale, True) == 0
    torch.cuda.synchronize()
    # No atomics anywhere: all three gradients are bitwise reproducible.
    assert torch.equal(dk1, dk2) and torch.equal(dv1, dv2) and torch.equal(dq1, dq2)


@pytest.mark.parametrize("dtype", ["bf16", "f16"])
def test_stage0_row_terms(dtype):
    """Stage 0 (the dQ kernel) leaves the row terms -D_i = -sum_c dO_ic O_ic
    and -LSE_i / scale of every row in the workspace, at the offsets the
    header states; ragged N_q, one kv head for three q heads."""
    say(f"bwd stage-0 row terms {dtype}")
    B, Hq, Hkv, N, d = 2, 3, 1, 300, 128
    scale = 1.0 / math.sqrt(d)
    q, k, v, do = random_tensors((B, Hq, N, d), (B, Hkv, N, d), dtype, seed=14, with_grad=True)
    qg, kg, vg, dog = gpu(q), gpu(k), gpu(v), gpu(do)
    o, lse = fa.forward(qg, kg, vg, causal=True, scale=scale)
    nbytes = fa.fa_bwd_workspace_size(B, Hq, Hkv, N, N, d, q.dtype)
    ws = torch.full((nbytes,), 0xFF, dtype=torch.uint8, device="cuda")  # NaN floats
    dq, dk, dv = (torch.empty_like(t) for t in (qg, kg, vg))
    assert fa.fa_bwd_stage(0, qg, kg, vg, o, lse, dog, dq, dk, dv, ws, scale, True) == 0
    torch.cuda.synchronize()
    rows = B * Hq * N
    off = (rows * 4 + 255) // 256 * 256
    nd = ws[:rows * 4].view(torch.float32).cpu().double().numpy()
    lneg = ws[off:off + rows * 4].view(torch.float32).cpu().double().numpy()
    prod = to_f64(o.cpu()).reshape(rows, d) * to_f64(do).reshape(rows, d)
    D = prod.sum(axis=1)
    # float32 sum of d products: |error| <= d * 2^-24 * sum |terms|.
    assert np.all(np.abs(nd + D) <= d * 2.0**-24 * np.abs(prod).sum(axis=1) + 1e-30)
    want = -to_f64(lse.cpu()).reshape(rows) / scale
    assert np.all(np.abs(lneg - want) <= 2.0**-22 * np.abs(want))


def test_empty_query_side_clears_key_gradients():
    say("bwd empty queries")
    q, k, v, do = random_tensors((1, 2, 0, 64), (1, 2, 50, 64), "bf16", seed=13, with_grad=True)
    qg, kg, vg, dog = gpu(q), gpu(k), gpu(v), gpu(do)
    o = torch.empty_like(qg)
    lse = torch.empty((1, 2, 0), dtype=torch.float32, device="cuda")
    dq, dk, dv = fa.backward(qg, kg, vg, o, lse, dog, causal=False)
    torch.cuda.synchronize()
    assert torch.all(dk == 0) and torch.all(dv == 0)
