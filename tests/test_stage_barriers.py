"""The debug build with a stage barrier per pipeline step gives bit-identical
results (GPU).

libfa_stagesync.so is built from the same sources with -DFA_STAGE_BARRIERS:
every pipelined kernel waits for all of its copies and meets the other waves
of its workgroup at a barrier between issuing a step's copies and computing
that step (the decode kernel, whose waves pipeline independently, waits for
each copy as soon as it is issued). That changes when data arrives but not
one operation of the arithmetic, so each output must equal the normal
build's bit for bit. A buffer that a step reads before its copy has landed,
or that a copy overwrites while it is still being read, gives a different
result in one of the two builds. The normal build is also run twice to show
that it repeats itself bit for bit.
"""

import os

import numpy as np
import pytest
import torch

import exact_attention_115_amd as fa
from exact_attention_115_amd import _lib
from exact_attention_115_amd.build import STAGESYNC_LIB
from synth import random_tensors
from tests.parity_util import gpu, say
from tests.test_parity_fp8 import e4m3_inputs
from tests.test_parity_paged import make_case

pytestmark = [
    pytest.mark.gpu,
    pytest.mark.skipif(not torch.cuda.is_available(), reason="needs a GPU"),
    pytest.mark.skipif(not os.path.exists(STAGESYNC_LIB), reason="debug build missing"),
]


def _bits(t):
    """Integer view of a tensor's storage (NaN payloads and -0 compare exactly)."""
    t = t.contiguous()
    return t.view({1: torch.uint8, 2: torch.int16, 4: torch.int32}[t.element_size()])


def run_three(fn):
    """fn() with the normal library, again with it, then with the debug
    build; returns the three results (tuples of tensors)."""
    native = fa.load()
    debug = _lib.open_library(STAGESYNC_LIB)
    out = []
    for lib in (native, native, debug):
        _lib._lib = lib
        try:
            res = fn()
            torch.cuda.synchronize()
        finally:
            _lib._lib = native
        out.append(tuple(r.clone() for r in res))
    return out


def assert_bit_identical(label, results):
    base, again, debug = results
    for i, (a, b, c) in enumerate(zip(base, again, debug)):
        assert torch.equal(_bits(a), _bits(b)), f"{label}: output {i} differs between two runs"
        diff = (_bits(a) != _bits(c)).sum().item()
        assert diff == 0, f"{label}: output {i}: {diff} elements differ in the stage-barrier build"
    say(f"{label}: {len(base)} outputs bit-identical")


DT = {"bf16": torch.bfloat16, "f16": torch.float16}

PREFILL = [
    # (B, Hq, Hkv, Nq, Nkv, d, causal, dtype)
    (1, 32, 32, 4096, 4096, 128, True, "bf16"),   # 8-wave forward and dQ kernels
    (2, 16, 16, 1024, 1024, 64, False, "f16"),
    (1, 4, 2, 333, 517, 128, True, "bf16"),       # ragged, GQA
    (4, 32, 1, 2048, 2048, 128, True, "bf16"),    # MQA: split head group + reduce
    (2, 8, 8, 700, 300, 64, True, "f16"),         # rows that see no key
]


@pytest.mark.parametrize("case", PREFILL, ids=[str(c) for c in PREFILL])
def test_forward_and_backward(case):
    B, Hq, Hkv, Nq, Nkv, d, causal, dtype = case
    say(f"stage barriers fwd/bwd {case}")
    q, k, v, do = [gpu(t) for t in random_tensors((B, Hq, Nq, d), (B, Hkv, Nkv, d), dtype, 5,
                                                  with_grad=True)]
    assert_bit_identical(f"forward {case}",
                         run_three(lambda: fa.forward(q, k, v, causal=causal)))
    o, lse = fa.forward(q, k, v, causal=causal)
    assert_bit_identical(f"backward {case}",
                         run_three(lambda: fa.backward(q, k, v, o, lse, do, causal=causal)))


def test_dropout_forward_and_backward():
    B, Hq, Hkv, N, d = 2, 8, 4, 640, 128
    q, k, v, do = [gpu(t) for t in random_tensors((B, Hq, N, d), (B, Hkv, N, d), "bf16", 9,
                                                  with_grad=True)]
    assert_bit_identical("dropout forward", run_three(
        lambda: fa.forward_dropout(q, k, v, 0.15, seed=3, offset=7, causal=True)))
    o, lse = fa.forward_dropout(q, k, v, 0.15, seed=3, offset=7, causal=True)
    assert_bit_identical("dropout backward", run_three(
        lambda: fa.backward_dropout(q, k, v, o, lse, do, 0.15, seed=3, offset=7, causal=True)))


DECODE = [
    # (B, Hq, Hkv, Nkv, d)
    (16, 32, 8, 8192, 128),
    (16, 32, 1, 8192, 128),
    (2, 8, 2, 100 * 64 + 17, 64),   # many splits, ragged tail
]


@pytest.mark.parametrize("case", DECODE, ids=[str(c) for c in DECODE])
def test_decode(case):
    B, Hq, Hkv, Nkv, d = case
    say(f"stage barriers decode {case}")
    q, k, v, _ = [gpu(t) for t in random_tensors((B, Hq, 1, d), (B, Hkv, Nkv, d), "bf16", 11)]
    assert_bit_identical(f"decode {case}", run_three(lambda: fa.forward(q, k, v)))


def test_paged_decode():
    q, kp, vp, table, lens = make_case(3, 8, 2, 128, 64, [1, 700, 1280], "bf16", seed=13)
    q, kp, vp = gpu(q), gpu(kp), gpu(vp)
    t, ln = torch.from_numpy(table).cuda(), torch.from_numpy(lens).cuda()
    assert_bit_identical("paged decode", run_three(
        lambda: fa.forward_paged(q, kp, vp, t, ln, 1.0 / np.sqrt(128))))


@pytest.mark.parametrize("causal", [False, True])
def test_fp8_forward(causal):
    q8, k8, v8 = [t.cuda() for t in e4m3_inputs(1, 8, 8, 1024, 1024, seed=17)]
    assert_bit_identical(f"fp8 forward causal={causal}", run_three(
        lambda: fa.forward_fp8(q8, k8, v8, 0.5, 0.25, 2.0, causal=causal)))
