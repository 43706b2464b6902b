"""GPU parity on seeded random shapes for the paths beside the plain
forward / backward: dropout (forward and backward), the paged-KV decode and
the FP8 forward, each against its float64 oracle.

The cases are drawn once from fixed seeds, like tests/test_parity_sweep.py:
ragged lengths log-uniform in [1, 700), MHA / GQA / MQA head ratios, causal
and not; for dropout also the probability, the generator seed and offset
(64-bit); for the paged decode the page size, the sequence lengths (empty
sequences included) and spare pages in the pool; for FP8 the three descale
factors. Each case uses the checks and bars of the path's own parity tests.
"""

import math

import numpy as np
import pytest
import torch

import exact_attention_115_amd as fa
import oracle
from oracle import dropout as drop
from synth import random_tensors, to_f64
from tests.parity_util import check_forward, gpu, say
from tests.test_parity_dropout import check_dropout_forward, check_dropout_grads, f32
from tests.test_parity_fp8 import check_fp8, e4m3_inputs
from tests.test_parity_paged import make_case, run_paged

pytestmark = [
    pytest.mark.gpu,
    pytest.mark.skipif(not torch.cuda.is_available(), reason="needs a GPU"),
]


def _length(rng, hi=700.0):
    return int(np.exp(rng.uniform(0.0, np.log(hi))))


def _heads(rng):
    hkv = int(rng.choice([1, 2, 3]))
    return hkv * int(rng.choice([1, 2, 4])), hkv


def _dropout_cases(n=16, seed=3031):
    rng = np.random.default_rng(seed)
    out = []
    for i in range(n):
        hq, hkv = _heads(rng)
        out.append((int(rng.integers(1, 3)), hq, hkv, _length(rng), _length(rng),
                    int(rng.choice([64, 128])), bool(rng.integers(0, 2)),
                    str(rng.choice(["bf16", "f16"])), round(float(rng.uniform(0.05, 0.9)), 3),
                    int(rng.integers(0, 2**63)) * 2 + int(rng.integers(0, 2)),
                    int(rng.integers(0, 2**62)), 3000 + i))
    return out


DROPOUT_CASES = _dropout_cases()


@pytest.mark.parametrize("case", DROPOUT_CASES, ids=["B{}Hq{}Hkv{}Nq{}Nkv{}d{}{}{}p{}".format(
    *c[:6], "c" if c[6] else "n", c[7], c[8]) for c in DROPOUT_CASES])
def test_random_shape_dropout(case):
    B, Hq, Hkv, Nq, Nkv, d, causal, dtype, p, seed, offset, data_seed = case
    label = f"dropout B{B} Hq{Hq} Hkv{Hkv} Nq{Nq} Nkv{Nkv} d{d} causal={causal} {dtype} p={p}"
    say(label)
    scale = 1.0 / math.sqrt(d)
    q, k, v, do = random_tensors((B, Hq, Nq, d), (B, Hkv, Nkv, d), dtype, seed=data_seed,
                                 with_grad=True)
    qg, kg, vg, dog = gpu(q), gpu(k), gpu(v), gpu(do)
    o, lse = fa.forward_dropout(qg, kg, vg, p, seed, offset, causal=causal, scale=scale)
    grads = fa.backward_dropout(qg, kg, vg, o, lse, dog, p, seed, offset, causal=causal,
                                scale=scale)
    torch.cuda.synchronize()
    o_ref, lse_ref = drop.attention_forward_dropout(to_f64(q), to_f64(k), to_f64(v), causal, scale,
                                                    f32(p), seed, offset)
    check_dropout_forward(o, lse, o_ref, lse_ref, dtype, p, label)
    check_dropout_grads(grads, q, k, v, do, causal, scale, p, seed, offset, dtype, label)


def _paged_cases(n=14, seed=3032):
    rng = np.random.default_rng(seed)
    out = []
    for i in range(n):
        hkv = int(rng.choice([1, 2, 4]))
        g = int(rng.choice([1, 2, 4, 8, 32]))
        B = int(rng.integers(1, 5))
        ps = int(rng.choice([64, 128, 256]))
        lens = [0 if rng.uniform() < 0.1 else _length(rng, 3000.0) for _ in range(B)]
        out.append((B, hkv * g, hkv, int(rng.choice([64, 128])), ps, lens,
                    str(rng.choice(["bf16", "f16"])), int(rng.integers(0, 4)), 3100 + i))
    return out


PAGED_CASES = _paged_cases()


@pytest.mark.parametrize("case", PAGED_CASES, ids=["B{}Hq{}Hkv{}d{}ps{}-{}-{}".format(
    c[0], c[1], c[2], c[3], c[4], "_".join(map(str, c[5])), c[6]) for c in PAGED_CASES])
def test_random_shape_paged_decode(case):
    B, Hq, Hkv, d, ps, lens, dtype, spare, seed = case
    label = f"paged B{B} Hq{Hq} Hkv{Hkv} d{d} page {ps} lens {lens} {dtype}"
    say(label)
    q, kp, vp, table, ln = make_case(B, Hq, Hkv, d, ps, lens, dtype, seed=seed, spare_pages=spare)
    scale = 1.0 / math.sqrt(d)
    o, lse = run_paged(q, kp, vp, table, ln, scale)
    o_ref, lse_ref = oracle.paged_decode_forward(to_f64(q), to_f64(kp), to_f64(vp), table, ln,
                                                 scale)
    check_forward(o, lse, o_ref, lse_ref, dtype, label)


def _fp8_cases(n=10, seed=3033):
    rng = np.random.default_rng(seed)
    out = []
    for i in range(n):
        hq, hkv = _heads(rng)
        descales = tuple(float(2.0 ** rng.integers(-3, 3) * rng.uniform(0.5, 1.0)) for _ in range(3))
        out.append((int(rng.integers(1, 3)), hq, hkv, _length(rng), _length(rng),
                    bool(rng.integers(0, 2)), descales, 3200 + i))
    return out


FP8_CASES = _fp8_cases()


@pytest.mark.parametrize("case", FP8_CASES, ids=["B{}Hq{}Hkv{}Nq{}Nkv{}{}".format(
    *c[:5], "c" if c[5] else "n") for c in FP8_CASES])
def test_random_shape_fp8_forward(case):
    B, Hq, Hkv, Nq, Nkv, causal, descales, seed = case
    label = f"fp8 B{B} Hq{Hq} Hkv{Hkv} Nq{Nq} Nkv{Nkv} causal={causal}"
    say(label)
    scale = 1.0 / math.sqrt(128)
    q8, k8, v8 = e4m3_inputs(B, Hq, Hkv, Nq, Nkv, seed=seed, descales=descales)
    o, lse = fa.forward_fp8(q8.cuda(), k8.cuda(), v8.cuda(), *descales, causal=causal, scale=scale)
    torch.cuda.synchronize()
    heads = [(b, h) for b in range(B) for h in range(Hq)]
    check_fp8(o.cpu(), lse.cpu(), q8, k8, v8, heads, causal, scale, descales, label)
