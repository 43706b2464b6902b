"""GPU parity at the largest sizes the library accepts.

One head's K (or V) is addressed with 32-bit byte offsets, and the calls
accept N_kv * d * 4 < 2^31: at d = 128 the largest key count is 4 194 303
(a 1 GiB K and a 1 GiB V for one kv head). These cases run the decode and
the tiled forward at exactly that size, and the backward at a million keys,
so that every per-head offset in the kernels comes close to its range, and
compare with the float64 oracle on the same seeded inputs.

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
from parity_util import check_forward, check_grads, gpu, oracle_heads_backward, say
from synth import random_tensors, to_f64

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
    (dq_ref, dk_ref, dv_ref), = oracle_heads_backward(q, k, v, do, True, 1.0, [(0, 0)])
    check_grads((dq[0].cpu(), dk[0, 0].cpu(), dv[0, 0].cpu()), (dq_ref, dk_ref, dv_ref), "bf16",
                f"backward N_kv={nkv}")
