"""GPU parity of the forward (fa_fwd) against the float64 oracle.

Inputs come from ``synth`` (seeded N(0,1), rounded to the storage dtype); the
oracle receives the same rounded values widened to float64.
"""

import math

import numpy as np
import pytest
import torch

import exact_attention_115_amd as fa
import oracle
from synth import WORKLOADS, make_inputs, random_tensors, to_f64
from tests.parity_util import (all_finite, check_forward, forward_nan_filled, gpu,
                               oracle_heads_forward, run_forward, sample_heads, say)

pytestmark = [
    pytest.mark.gpu,
    pytest.mark.skipif(not torch.cuda.is_available(), reason="needs a GPU"),
]


def full_oracle(q, k, v, causal, scale):
    return oracle.attention_forward(to_f64(q), to_f64(k), to_f64(v), causal, scale)


# ------------------------------------------------------------- the worked example

def hand_example(nq, dtype):
    """The worked example of page "FlashAttention：为什么少搬数据，反而算得更快" §04,
    embedded at d = 64: q = e0, k_j = ln(e_j) e0, v_j = V_j e0 with exp-scores
    e = [1, 2, 4, 3] and V = [10, 20, 30, 40]; scale 1, so O[:, 0] = 29,
    O[:, 1:] = 0 and LSE = ln 10."""
    e = torch.tensor([1.0, 2.0, 4.0, 3.0], dtype=torch.float64)
    vals = torch.tensor([10.0, 20.0, 30.0, 40.0], dtype=torch.float64)
    q = torch.zeros(1, 1, nq, 64, dtype=torch.float64)
    q[..., 0] = 1.0
    k = torch.zeros(1, 1, 4, 64, dtype=torch.float64)
    k[0, 0, :, 0] = torch.log(e)
    v = torch.zeros(1, 1, 4, 64, dtype=torch.float64)
    v[0, 0, :, 0] = vals
    return q.to(dtype), k.to(dtype), v.to(dtype)


@pytest.mark.parametrize("nq", [1, 4])
def test_hand_example_f32(nq):
    say(f"hand example f32 nq={nq}")
    q, k, v = hand_example(nq, torch.float32)
    o, lse = run_forward(q, k, v, causal=False, scale=1.0)
    o = to_f64(o)
    assert np.max(np.abs(o[..., 0] - 29.0)) <= 1e-5
    assert np.max(np.abs(o[..., 1:])) == 0.0
    assert np.max(np.abs(to_f64(lse) - math.log(10.0))) <= 1e-5


@pytest.mark.parametrize("dtype", ["bf16", "f16"])
def test_hand_example_16bit(dtype):
    # In 16 bits ln(e_j) is rounded, so the exact answer is the oracle's on the
    # rounded inputs (close to, not exactly, 29); with 4 identical query rows
    # (prefill path) and one query row (decode path).
    for nq in (4, 1):
        say(f"hand example {dtype} nq={nq}")
        q, k, v = hand_example(nq, {"bf16": torch.bfloat16, "f16": torch.float16}[dtype])
        o, lse = run_forward(q, k, v, causal=False, scale=1.0)
        o_ref, lse_ref = full_oracle(q, k, v, False, 1.0)
        check_forward(o, lse, o_ref, lse_ref, dtype, f"hand {dtype} nq={nq}")
        assert abs(o_ref[0, 0, 0, 0] - 29.0) < 0.3


# ------------------------------------------------------------------ workloads

@pytest.mark.parametrize("name", ["c1", "c1c"])
def test_c1_f32(name):
    w = WORKLOADS[name]
    say(f"{name}: {w}")
    q, k, v, _ = make_inputs(w)
    o, lse = run_forward(q, k, v, w.causal, w.scale)
    o_ref, lse_ref = full_oracle(q, k, v, w.causal, w.scale)
    check_forward(o, lse, o_ref, lse_ref, "f32", name)


@pytest.mark.parametrize("name", ["c2", "c2c"])
def test_c2_forward(name):
    w = WORKLOADS[name]
    say(f"{name}: {w}")
    q, k, v, _ = make_inputs(w)
    o, lse = run_forward(q, k, v, w.causal, w.scale)
    o_ref, lse_ref = full_oracle(q, k, v, w.causal, w.scale)
    check_forward(o, lse, o_ref, lse_ref, w.dtype, name)


@pytest.mark.parametrize("name", ["c3", "c4", "c5g", "c5m"])
def test_full_size_forward_sampled_heads(name):
    """Full-size launch (as timed by the bench) into NaN-filled outputs:
    every element must be written and finite. The oracle computes complete
    heads, which are independent of the others: all 32 heads at c3 (the
    8-wave, 256-row workgroups over the whole grid), a sample elsewhere."""
    w = WORKLOADS[name]
    say(f"{name}: {w}")
    q, k, v, _ = make_inputs(w, with_grad=False)
    o, lse = forward_nan_filled(gpu(q), gpu(k), gpu(v), w.causal, w.scale)
    torch.cuda.synchronize()
    all_finite(f"{name} o", o)
    all_finite(f"{name} lse", lse)
    if name == "c3":
        heads = [(0, h) for h in range(w.Hq)]
    else:
        heads = sample_heads(w.B, w.Hq, 2 if w.Nq >= 8192 else 3)
    o, lse = o.cpu(), lse.cpu()
    for i in range(0, len(heads), 8):
        chunk = heads[i:i + 8]
        o_ref, lse_ref = oracle_heads_forward(q, k, v, w.causal, w.scale, chunk)
        o_s = torch.stack([o[b, h] for b, h in chunk])
        l_s = torch.stack([lse[b, h] for b, h in chunk])
        check_forward(o_s, l_s, o_ref, lse_ref, w.dtype, f"{name} heads {chunk}")


@pytest.mark.parametrize("causal", [False, True])
def test_long_ragged_forward_sampled_heads(causal):
    """256-row workgroups (N_q >= 4096 and enough of them to fill the GPU)
    with a ragged last query and key tile, causal and not."""
    w = WORKLOADS["c3"].replace(name="long_ragged", Hq=16, Hkv=16, Nq=4100, Nkv=4100,
                                causal=causal, seed=37)
    say(f"{w}")
    q, k, v, _ = make_inputs(w, with_grad=False)
    o, lse = run_forward(q, k, v, w.causal, w.scale)
    heads = [(0, 0), (0, w.Hq - 1)]
    o_ref, lse_ref = oracle_heads_forward(q, k, v, w.causal, w.scale, heads)
    o_s = torch.stack([o[b, h] for b, h in heads])
    l_s = torch.stack([lse[b, h] for b, h in heads])
    check_forward(o_s, l_s, o_ref, lse_ref, w.dtype, f"long ragged causal={causal}")
    assert torch.isfinite(o).all()


@pytest.mark.parametrize("name", ["c5dg", "c5dm"])
def test_decode_forward(name):
    w = WORKLOADS[name]
    say(f"{name}: {w}")
    q, k, v, _ = make_inputs(w)
    o, lse = forward_nan_filled(gpu(q), gpu(k), gpu(v), w.causal, w.scale)
    torch.cuda.synchronize()
    all_finite(f"{name} o", o)
    all_finite(f"{name} lse", lse)
    heads = [(0, 0), (w.B - 1, w.Hq - 1), (7, 13), (3, 30)]
    o_ref, lse_ref = oracle_heads_forward(q, k, v, w.causal, w.scale, heads)
    o_s = torch.stack([o[b, h] for b, h in heads])
    l_s = torch.stack([lse[b, h] for b, h in heads])
    check_forward(o_s, l_s, o_ref, lse_ref, w.dtype, f"{name} heads {heads}")


# ------------------------------------------------------------------ edge cases

EDGE = [
    # (B, Hq, Hkv, Nq, Nkv, d, causal)
    (1, 2, 2, 300, 300, 64, True),     # ragged tail, several tiles
    (1, 2, 2, 300, 300, 128, False),
    (2, 4, 2, 200, 333, 128, True),    # N_q < N_kv, bottom-right causal, GQA
    (1, 4, 1, 333, 200, 64, True),     # N_q > N_kv: leading rows see nothing (MQA)
    (1, 2, 2, 1, 1, 64, False),        # single query, single key
    (1, 2, 2, 5, 1, 128, False),       # single key: O = V0
    (1, 2, 2, 130, 7, 64, False),      # keys fewer than one tile
    (1, 1, 1, 2, 4, 128, True),
    (3, 6, 3, 65, 129, 64, True),
    (1, 2, 1, 1, 1000, 128, True),     # decode, ragged split
    (2, 4, 1, 1, 12763, 128, False),   # decode, 100 key-range splits: two merge rounds of 64, last group of 16 partial
    (2, 8, 2, 1, 64, 64, False),
    (2, 64, 16, 1000, 1000, 128, True),  # many 128-row workgroups, ragged last tile
    (4, 32, 32, 700, 900, 64, False),    # many workgroups, N_q < N_kv
]


@pytest.mark.parametrize("dtype", ["bf16", "f16", "f32"])
@pytest.mark.parametrize("case", EDGE, ids=[str(c) for c in EDGE])
def test_edge_cases(dtype, case):
    B, Hq, Hkv, nq, nkv, d, causal = case
    say(f"edge {dtype} {case}")
    q, k, v, _ = random_tensors((B, Hq, nq, d), (B, Hkv, nkv, d), dtype, seed=nq * 7 + nkv)
    scale = 1.0 / math.sqrt(d)
    o, lse = run_forward(q, k, v, causal, scale)
    o_ref, lse_ref = full_oracle(q, k, v, causal, scale)
    check_forward(o, lse, o_ref, lse_ref, dtype, str(case))


@pytest.mark.parametrize("dtype", ["bf16", "f32"])
def test_no_keys(dtype):
    """N_kv = 0: every row sees nothing -> O = 0, LSE = -inf."""
    say(f"no keys {dtype}")
    q, k, v, _ = random_tensors((1, 2, 70, 64), (1, 2, 0, 64), dtype, seed=3)
    o, lse = run_forward(q, k, v, False, 0.125)
    assert torch.all(o == 0)
    assert torch.all(torch.isneginf(lse))
    o_ref, lse_ref = oracle.attention_forward(to_f64(q), to_f64(k), to_f64(v), False, 0.125)
    assert np.all(o_ref == 0) and np.all(np.isneginf(lse_ref))


def test_gqa_equals_repeated_mha_bitwise():
    say("gqa vs repeated mha")
    q, k, v, _ = random_tensors((2, 8, 257, 128), (2, 2, 257, 128), "bf16", seed=5)
    o1, l1 = run_forward(q, k, v, True, 0.09)
    o2, l2 = run_forward(q, k.repeat_interleave(4, dim=1), v.repeat_interleave(4, dim=1), True, 0.09)
    assert torch.equal(o1, o2) and torch.equal(l1, l2)


def test_decode_equals_last_causal_row():
    """Decode of the last query == last row of a causal prefill with that query."""
    say("decode vs last causal row")
    q, k, v, _ = random_tensors((2, 8, 300, 128), (2, 2, 300, 128), "bf16", seed=6)
    o_full, l_full = run_forward(q, k, v, True, 0.09)
    o_dec, l_dec = run_forward(q[:, :, -1:].contiguous(), k, v, True, 0.09)
    diff = (o_full[:, :, -1:].float() - o_dec.float()).abs().max().item()
    assert diff <= 2e-2
    assert (l_full[:, :, -1:] - l_dec).abs().max().item() <= 1e-3


def test_forward_deterministic_and_overwrites():
    say("determinism")
    w = WORKLOADS["c2c"]
    q, k, v, _ = make_inputs(w)
    qg, kg, vg = gpu(q), gpu(k), gpu(v)
    o1, l1 = fa.forward(qg, kg, vg, causal=True)
    o2 = torch.full_like(o1, float("nan"))
    l2 = torch.full_like(l1, float("nan"))
    assert fa.fa_fwd(qg, kg, vg, o2, l2, None, w.scale, True) == 0
    torch.cuda.synchronize()
    assert torch.equal(o1, o2) and torch.equal(l1, l2)


@pytest.mark.parametrize("name", ["c4", "c2c"])
def test_forward_repeatable_bitwise(name):
    """The forward has no atomics: repeated launches (with other work between
    them changing the timing) must give identical bits. Guards the staging
    of key/value tiles in shared memory against read/overwrite races."""
    w = WORKLOADS[name]
    say(f"repeatability {name}")
    q, k, v, _ = make_inputs(w, with_grad=False)
    qg, kg, vg = gpu(q), gpu(k), gpu(v)
    o_ref, l_ref = fa.forward(qg, kg, vg, causal=w.causal)
    scratch = torch.empty(1 << 24, device="cuda")
    for i in range(6):
        scratch.normal_()
        o, lse = fa.forward(qg, kg, vg, causal=w.causal)
        assert torch.equal(o, o_ref) and torch.equal(lse, l_ref), f"launch {i} differs"
    torch.cuda.synchronize()
