"""GPU parity on seeded random shapes against the float64 oracle (every head).

The shapes are drawn once from a fixed seed: ragged N_q and N_kv,
log-uniform in [1, 1000) (N_q below and above N_kv; N_q = 1 takes the
decode path), MHA, GQA and MQA head ratios, d = 64 and 128, bf16 and fp16,
causal and not.
Each case checks the forward (O, LSE) and the backward (dQ, dK, dV) with the
same tolerances as the fixed cases.
"""

import math

import numpy as np
import pytest
import torch

import exact_attention_115_amd as fa
import oracle
from synth import random_tensors, to_f64
from tests.parity_util import check_forward, check_grads, gpu, say

pytestmark = [
    pytest.mark.gpu,
    pytest.mark.skipif(not torch.cuda.is_available(), reason="needs a GPU"),
]


def _cases(n=40, seed=2026):
    rng = np.random.default_rng(seed)

    def length():  # log-uniform in [1, 1000): single rows and keys come up too
        return int(np.exp(rng.uniform(0.0, np.log(1000.0))))

    out = []
    for i in range(n):
        hkv = int(rng.choice([1, 2, 3]))
        hq = hkv * int(rng.choice([1, 2, 4]))
        out.append((int(rng.integers(1, 3)), hq, hkv, length(), length(), int(rng.choice([64, 128])),
                    bool(rng.integers(0, 2)), str(rng.choice(["bf16", "f16"])), 1000 + i))
    return out


CASES = _cases()


@pytest.mark.parametrize("case", CASES, ids=["B{}Hq{}Hkv{}Nq{}Nkv{}d{}{}{}".format(
    *c[:6], "c" if c[6] else "n", c[7]) for c in CASES])
def test_random_shape_forward_backward(case):
    B, Hq, Hkv, Nq, Nkv, d, causal, dtype, seed = case
    label = f"B{B} Hq{Hq} Hkv{Hkv} Nq{Nq} Nkv{Nkv} d{d} causal={causal} {dtype}"
    say(label)
    scale = 1.0 / math.sqrt(d)
    q, k, v, do = random_tensors((B, Hq, Nq, d), (B, Hkv, Nkv, d), dtype, seed=seed, with_grad=True)
    qg, kg, vg, dog = gpu(q), gpu(k), gpu(v), gpu(do)
    o, lse = fa.forward(qg, kg, vg, causal=causal, scale=scale)
    dq, dk, dv = fa.backward(qg, kg, vg, o, lse, dog, causal=causal, scale=scale)
    torch.cuda.synchronize()
    q64, k64, v64, do64 = (to_f64(t) for t in (q, k, v, do))
    o_ref, lse_ref = oracle.attention_forward(q64, k64, v64, causal, scale)
    check_forward(o.cpu(), lse.cpu(), o_ref, lse_ref, dtype, label)
    g_ref = oracle.attention_backward(q64, k64, v64, do64, causal, scale)
    check_grads((dq.cpu(), dk.cpu(), dv.cpu()), g_ref, dtype, label,
                mags=oracle.attention_backward_magnitudes(q64, k64, v64, do64, causal, scale))
