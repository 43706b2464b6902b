"""GPU test of fa_bwd_noalloc (the backward on the library's static scratch
buffer) against fa_bwd (the same kernels on a caller's workspace), through
the C ABI: two calls in a row, the second on a smaller problem, so the
second call runs on a buffer that still holds the first call's contents."""

import pytest
import torch

import exact_attention_115_amd as fa
from synth import random_tensors
from tests.parity_util import gpu, say

pytestmark = [
    pytest.mark.gpu,
    pytest.mark.skipif(not torch.cuda.is_available(), reason="needs a GPU"),
]

FA_ERR_SCRATCH = -9
SCRATCH_BYTES = 32 << 20


def noalloc(q, k, v, o, lse, do, dq, dk, dv, scale, causal):
    """fa_bwd_noalloc through the C ABI (ctypes binding, no workspace)."""
    return fa.fa_bwd_noalloc(q, k, v, o, lse, do, dq, dk, dv, scale, causal)


CASES = [
    # B, Hq, Hkv, Nq, Nkv, d, causal, dtype
    (2, 8, 2, 700, 900, 128, True, "bf16"),
    (1, 4, 4, 200, 130, 64, False, "f16"),     # smaller: the buffer holds the first call's data
    (1, 8, 1, 300, 300, 128, True, "bf16"),    # MQA: split head group, float32 partials in scratch
    (1, 2, 2, 64, 64, 64, True, "bf16"),
]


def test_noalloc_equals_fa_bwd_on_consecutive_calls():
    for case in CASES:
        B, Hq, Hkv, Nq, Nkv, d, causal, dtype = case
        say(f"fa_bwd_noalloc {case}")
        q, k, v, do = random_tensors((B, Hq, Nq, d), (B, Hkv, Nkv, d), dtype, seed=Nq + Nkv,
                                     with_grad=True)
        qg, kg, vg, dog = gpu(q), gpu(k), gpu(v), gpu(do)
        scale = d ** -0.5
        need = fa.fa_bwd_workspace_size(B, Hq, Hkv, Nq, Nkv, d, qg.dtype)
        assert 0 < need <= SCRATCH_BYTES
        o, lse = fa.forward(qg, kg, vg, causal=causal, scale=scale)
        ref = fa.backward(qg, kg, vg, o, lse, dog, causal=causal, scale=scale)
        got = [torch.full_like(t, float("nan")) for t in ref]
        assert noalloc(qg, kg, vg, o, lse, dog, *got, scale, causal) == 0
        torch.cuda.synchronize()
        for name, a, b in zip(("dq", "dk", "dv"), got, ref):
            assert torch.equal(a, b), f"{case}: {name} differs from fa_bwd"


def test_noalloc_refuses_problems_beyond_the_scratch():
    # Row terms alone: 2 * 4 B per query row -> 4.2 M rows need 32 MiB + 256 B.
    B, Hq, Hkv, Nq, Nkv, d = 1, 64, 64, 65540, 64, 64
    need = fa.fa_bwd_workspace_size(B, Hq, Hkv, Nq, Nkv, d, torch.bfloat16)
    assert need > SCRATCH_BYTES
    q = torch.zeros((B, Hq, Nq, d), dtype=torch.bfloat16, device="cuda")
    k = torch.zeros((B, Hkv, Nkv, d), dtype=torch.bfloat16, device="cuda")
    lse = torch.zeros((B, Hq, Nq), dtype=torch.float32, device="cuda")
    dq = torch.full_like(q, 7.0)
    dk, dv = torch.full_like(k, 7.0), torch.full_like(k, 7.0)
    st = noalloc(q, k, k.clone(), q.clone(), lse, q.clone(), dq, dk, dv, 0.1, True)
    torch.cuda.synchronize()
    assert st == FA_ERR_SCRATCH, st
    assert "static scratch" in fa.fa_strerror(st)
    assert torch.all(dq == 7.0) and torch.all(dk == 7.0) and torch.all(dv == 7.0)
