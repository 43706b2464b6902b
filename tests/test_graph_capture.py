"""The entry points recorded into a HIP graph (GPU).

fa_fwd, fa_bwd, the decode path of fa_fwd and fa_bwd_noalloc only enqueue
kernels on the caller's stream: no allocation, no memset, no
synchronization. So they can be captured into a graph (here through
torch.cuda.graph, which captures the current stream) and replayed. Each test
captures once, then replays several times, each time after writing new
input values into the captured buffers with ordinary eager work and a
synchronization. Every replay must give bit for bit what eager calls of the
same entry points give on the same inputs (the kernels are deterministic).
"""

import math

import pytest
import torch

import exact_attention_115_amd as fa
from synth import random_device_tensor

pytestmark = [
    pytest.mark.gpu,
    pytest.mark.skipif(not torch.cuda.is_available(), reason="needs a GPU"),
]

REPLAYS = 3


def _fill(tensors, seed):
    for i, t in enumerate(tensors):
        t.copy_(random_device_tensor(t.shape, "bf16", seed * 16 + i))


def _ok(status, where):
    assert status == 0, f"{where}: {fa.fa_strerror(status)}"


def _capture(fn):
    """Capture fn() into a graph (after one eager warm-up call on a side
    stream, as torch asks before capture)."""
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        fn()
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        fn()
    torch.cuda.synchronize()
    return g


def test_forward_backward_replays_match_eager():
    B, Hq, Hkv, N, d, causal = 2, 8, 2, 1000, 128, True
    scale = 1.0 / math.sqrt(d)
    dev = "cuda"
    q = torch.empty((B, Hq, N, d), dtype=torch.bfloat16, device=dev)
    do = torch.empty_like(q)
    k = torch.empty((B, Hkv, N, d), dtype=torch.bfloat16, device=dev)
    v = torch.empty_like(k)
    o, dq = torch.empty_like(q), torch.empty_like(q)
    dk, dv = torch.empty_like(k), torch.empty_like(k)
    lse = torch.empty((B, Hq, N), dtype=torch.float32, device=dev)
    ws = torch.empty(fa.fa_bwd_workspace_size(B, Hq, Hkv, N, N, d, fa.FA_BF16), dtype=torch.uint8,
                     device=dev)
    _fill((q, k, v, do), 0)

    def step():
        _ok(fa.fa_fwd(q, k, v, o, lse, None, scale, causal), "fa_fwd")
        _ok(fa.fa_bwd(q, k, v, o, lse, do, dq, dk, dv, ws, scale, causal), "fa_bwd")

    g = _capture(step)
    for rep in range(REPLAYS):
        _fill((q, k, v, do), rep + 1)
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        o_e, lse_e = fa.forward(q, k, v, causal=causal, scale=scale)
        dq_e, dk_e, dv_e = fa.backward(q, k, v, o_e, lse_e, do, causal=causal, scale=scale)
        torch.cuda.synchronize()
        for name, a, b in (("o", o, o_e), ("lse", lse, lse_e), ("dq", dq, dq_e), ("dk", dk, dk_e),
                           ("dv", dv, dv_e)):
            assert torch.equal(a, b), f"replay {rep}: {name} differs from the eager call"


def test_decode_replays_match_eager():
    B, Hq, Hkv, Nkv, d = 4, 32, 8, 3000, 128
    scale = 1.0 / math.sqrt(d)
    dev = "cuda"
    q = torch.empty((B, Hq, 1, d), dtype=torch.bfloat16, device=dev)
    k = torch.empty((B, Hkv, Nkv, d), dtype=torch.bfloat16, device=dev)
    v = torch.empty_like(k)
    o = torch.empty_like(q)
    lse = torch.empty((B, Hq, 1), dtype=torch.float32, device=dev)
    ws = torch.empty(fa.fa_fwd_workspace_size(B, Hq, Hkv, 1, Nkv, d, fa.FA_BF16),
                     dtype=torch.uint8, device=dev)
    _fill((q, k, v), 10)
    g = _capture(lambda: _ok(fa.fa_fwd(q, k, v, o, lse, ws, scale, False), "fa_fwd decode"))
    for rep in range(REPLAYS):
        _fill((q, k, v), 11 + rep)
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        o_e, lse_e = fa.forward(q, k, v, scale=scale)
        torch.cuda.synchronize()
        assert torch.equal(o, o_e) and torch.equal(lse, lse_e), f"replay {rep}"


def test_noalloc_backward_replays_match_fa_bwd():
    """The allocation-free backward is meant for code under graph capture:
    captured here (after one eager call that looks up its scratch buffer),
    each replay equals fa_bwd with a caller workspace."""
    B, Hq, Hkv, N, d, causal = 1, 4, 4, 700, 64, False
    scale = 1.0 / math.sqrt(d)
    dev = "cuda"
    q = torch.empty((B, Hq, N, d), dtype=torch.bfloat16, device=dev)
    k, v, do = torch.empty_like(q), torch.empty_like(q), torch.empty_like(q)
    dq, dk, dv = torch.empty_like(q), torch.empty_like(q), torch.empty_like(q)
    _fill((q, k, v, do), 20)
    o, lse = fa.forward(q, k, v, causal=causal, scale=scale)
    g = _capture(lambda: _ok(fa.fa_bwd_noalloc(q, k, v, o, lse, do, dq, dk, dv, scale, causal),
                             "fa_bwd_noalloc"))
    for rep in range(REPLAYS):
        _fill((q, k, v, do), 21 + rep)
        o_new, lse_new = fa.forward(q, k, v, causal=causal, scale=scale)
        o.copy_(o_new)
        lse.copy_(lse_new)
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        ref = fa.backward(q, k, v, o, lse, do, causal=causal, scale=scale)
        torch.cuda.synchronize()
        for name, a, b in zip(("dq", "dk", "dv"), (dq, dk, dv), ref):
            assert torch.equal(a, b), f"replay {rep}: {name} differs from fa_bwd"
