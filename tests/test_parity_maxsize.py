"""GPU parity at the largest sizes the library accepts.

One head's K (or V) is addressed with 32-bit byte offsets, and the calls
accept N_kv * d * 4 < 2^31: at d = 128 the largest key count is 4 194 303
(a 1 GiB K and a 1 GiB V for one kv head). These cases run the decode and
the tiled forward at exactly that size, and the backward at a million keys,
so that every per-head offset in the kernels comes close to its range, and
compare with the float64 oracle on the same seeded inputs.

The query side is addressed with 64-bit offsets (one tile's rows at a
time), so a head's Q, O and dO may pass 4 GiB: the backward runs with
N_q = 2^24 + 100 at d = 128 (Q of one head 4 GiB + 25 KiB), and the decode
with B * Hq = 2^24 query rows, each checked on sampled rows.

With i.i.d. N(0, 1) inputs and scale 1/sqrt(d), millions of keys share the
softmax almost evenly and O is close to zero, which would let a wrong kernel
pass the absolute O bar; those cases lean on the LSE (wrong by ln 2 if half
the keys were lost). The cases with scale 1 make each row's softmax peak on
a few keys out of millions, so O is of order one and must pick them out.
"""

import numpy as np
import pytest
import torch

import exact_attention_115_amd as fa
import oracle
from parity_util import all_finite, check_forward, check_grads, gpu, oracle_heads_backward, say
from synth import random_device_tensor, random_tensors, to_f64

pytestmark = pytest.mark.gpu

D = 128
MAX_NKV = (1 << 31) // (D * 4) - 1  # 4194303


@pytest.fixture(scope="module")
def max_inputs():
    say(f"drawing q [1, 4, 3, {D}], k and v [1, 1, {MAX_NKV}, {D}] (bf16)")
    q, k, v, _ = random_tensors((1, 4, 3, D), (1, 1, MAX_NKV, D), "bf16", seed=95)
    kg, vg = gpu(k), gpu(v)
    k64, v64 = to_f64(k[0, 0]), to_f64(v[0, 0])
    del k, v
    return q, kg, vg, k64, v64


@pytest.mark.parametrize("scale", [1.0 / np.sqrt(D), 1.0])
def test_decode_at_max_keys(max_inputs, scale):
    q, kg, vg, k64, v64 = max_inputs
    qd = q[:, :, :1].contiguous()
    say(f"decode B=1 Hq=4 Hkv=1 N_kv={MAX_NKV} scale={scale:.4f}")
    o, lse = fa.forward(gpu(qd), kg, vg, causal=True, scale=scale)
    torch.cuda.synchronize()
    o_ref = np.empty((1, 4, 1, D))
    lse_ref = np.empty((1, 4, 1))
    for h in range(4):
        o_ref[0, h], lse_ref[0, h] = oracle.head_forward(to_f64(qd[0, h]), k64, v64, True, scale)
    check_forward(o.cpu(), lse.cpu(), o_ref, lse_ref, "bf16", f"decode max N_kv scale={scale:.3f}")


@pytest.mark.parametrize("causal", [False, True])
def test_tiled_forward_at_max_keys(max_inputs, causal):
    q, kg, vg, k64, v64 = max_inputs
    say(f"tiled forward B=1 Hq=4 Hkv=1 N_q=3 N_kv={MAX_NKV} causal={causal} scale=1")
    o, lse = fa.forward(gpu(q), kg, vg, causal=causal, scale=1.0)
    torch.cuda.synchronize()
    o_ref = np.empty((1, 4, 3, D))
    lse_ref = np.empty((1, 4, 3))
    for h in range(4):
        o_ref[0, h], lse_ref[0, h] = oracle.head_forward(to_f64(q[0, h]), k64, v64, causal, 1.0)
    assert float(np.abs(o_ref).max()) > 0.5  # the peaked case: O is of order one
    check_forward(o.cpu(), lse.cpu(), o_ref, lse_ref, "bf16", f"tiled max N_kv causal={causal}")


def test_backward_at_a_million_keys():
    nkv = (1 << 20) + 37
    say(f"backward B=1 Hq=2 Hkv=1 N_q=24 N_kv={nkv} causal scale=1")
    q, k, v, do = random_tensors((1, 2, 24, D), (1, 1, nkv, D), "bf16", seed=96, with_grad=True)
    qg, kg, vg, dog = gpu(q), gpu(k), gpu(v), gpu(do)
    o, lse = fa.forward(qg, kg, vg, causal=True, scale=1.0)
    dq, dk, dv = fa.backward(qg, kg, vg, o, lse, dog, causal=True, scale=1.0)
    torch.cuda.synchronize()
    (dq_ref, dk_ref, dv_ref, mags), = oracle_heads_backward(q, k, v, do, True, 1.0, [(0, 0)],
                                                           with_mags=True)
    check_grads((dq[0].cpu(), dk[0, 0].cpu(), dv[0, 0].cpu()), (dq_ref, dk_ref, dv_ref), "bf16",
                f"backward N_kv={nkv}", mags=mags)


def test_backward_query_side_past_4gib():
    """B = Hq = Hkv = 1, N_q = 2^24 + 100, N_kv = 130, d = 128, not causal:
    Q, O, dO and dQ of the one head each hold 4 GiB + 25 KiB, so every byte
    offset of a query row past row 2^24 exceeds 32 bits. dO is zero except on
    a few rows R (spread over the range, some past 2^24): rows with dO = 0
    have D = 0 and dS = 0, so dK and dV are sums over R alone, and dQ is
    exactly zero off R. Outputs are NaN-filled first."""
    nq, nkv = (1 << 24) + 100, 130
    rows = [0, 5, (1 << 23) + 3, (1 << 24) - 1, (1 << 24) + 50, nq - 1]
    say(f"backward B=1 Hq=Hkv=1 N_q={nq} N_kv={nkv} d={D}, dO nonzero on rows {rows}")
    qg = random_device_tensor((1, 1, nq, D), "bf16", seed=97)
    _, k, v, _ = random_tensors((1, 1, 1, D), (1, 1, nkv, D), "bf16", seed=98)
    kg, vg = gpu(k), gpu(v)
    dog = torch.zeros_like(qg)
    dsel = random_tensors((1, 1, len(rows), D), (1, 1, 1, D), "bf16", seed=99)[0]
    ridx = torch.tensor(rows, device="cuda")
    dog[0, 0, ridx] = gpu(dsel)[0, 0]
    scale = 1.0 / np.sqrt(D)
    o = torch.full_like(qg, float("nan"))
    lse = torch.full((1, 1, nq), float("nan"), device="cuda")
    assert fa.fa_fwd(qg, kg, vg, o, lse, None, scale, False) == 0
    dq, dk, dv = (torch.full_like(t, float("nan")) for t in (qg, kg, vg))
    nb = fa.fa_bwd_workspace_size(1, 1, 1, nq, nkv, D, torch.bfloat16)
    ws = torch.full((nb,), 0xFF, dtype=torch.uint8, device="cuda")
    assert fa.fa_bwd(qg, kg, vg, o, lse, dog, dq, dk, dv, ws, scale, False) == 0
    torch.cuda.synchronize()
    for name, t in (("o", o), ("lse", lse), ("dq", dq), ("dk", dk), ("dv", dv)):
        all_finite(name, t)
    q_r = qg[0, 0, ridx].cpu()
    o_ref, lse_ref = oracle.head_forward(to_f64(q_r), to_f64(k[0, 0]), to_f64(v[0, 0]), False, scale)
    check_forward(o[0, 0, ridx].cpu(), lse[0, 0, ridx].cpu(), o_ref, lse_ref, "bf16",
                  "rows R of the 4 GiB head")
    args = (to_f64(q_r), to_f64(k[0, 0]), to_f64(v[0, 0]), to_f64(dsel[0, 0]), False, scale)
    g_ref = oracle.head_backward(*args)
    mags = oracle.head_backward_magnitudes(*args)
    check_grads((dq[0, 0, ridx].cpu(), dk[0, 0].cpu(), dv[0, 0].cpu()), g_ref, "bf16",
                "rows R of the 4 GiB head", mags=mags)
    dq[0, 0, ridx] = 0
    assert int(torch.count_nonzero(dq).item()) == 0, "dQ is nonzero on a row with dO = 0"
    del qg, dog, o, dq, ws
    torch.cuda.empty_cache()


def test_decode_query_rows_past_4gib():
    """Decode with B = 2^19, Hq = 32, Hkv = 1, N_kv = 64, d = 128: Q and O
    hold 2^24 rows (4 GiB each), so the byte offset of every query row past
    row 2^24 - 1 needs more than 32 bits (the last group's rows end exactly
    at 4 GiB). Sampled (b, h) rows against the oracle; outputs NaN-filled."""
    B, Hq, nkv = 1 << 19, 32, 64
    say(f"decode B={B} Hq={Hq} Hkv=1 N_kv={nkv} d={D}")
    qg = random_device_tensor((B, Hq, 1, D), "bf16", seed=101)
    kg = random_device_tensor((B, 1, nkv, D), "bf16", seed=102)
    vg = random_device_tensor((B, 1, nkv, D), "bf16", seed=103)
    scale = 1.0 / np.sqrt(D)
    o = torch.full_like(qg, float("nan"))
    lse = torch.full((B, Hq, 1), float("nan"), device="cuda")
    nb = fa.fa_fwd_workspace_size(B, Hq, 1, 1, nkv, D, torch.bfloat16)
    ws = torch.full((nb,), 0xFF, dtype=torch.uint8, device="cuda")
    assert fa.fa_fwd(qg, kg, vg, o, lse, ws, scale, True) == 0
    torch.cuda.synchronize()
    all_finite("o", o)
    all_finite("lse", lse)
    picks = [(0, 0), (B // 2 + 7, 13), (B - 1, 0), (B - 1, Hq - 1)]
    o_ref = np.empty((len(picks), 1, D))
    l_ref = np.empty((len(picks), 1))
    for i, (b, h) in enumerate(picks):
        o_ref[i], l_ref[i] = oracle.head_forward(to_f64(qg[b, h].cpu()), to_f64(kg[b, 0].cpu()),
                                                 to_f64(vg[b, 0].cpu()), True, scale)
    check_forward(torch.stack([o[b, h].cpu() for b, h in picks]),
                  torch.stack([lse[b, h].cpu() for b, h in picks]), o_ref, l_ref, "bf16",
                  f"decode rows {picks}")
    del qg, kg, vg, o, ws
    torch.cuda.empty_cache()
