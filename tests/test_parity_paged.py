"""GPU parity of decode over a paged K/V cache (fa_fwd_paged) against the
float64 oracle (the definition on each sequence's gathered keys)."""

import numpy as np
import pytest
import torch

import exact_attention_115_amd as fa
import oracle
from synth import random_tensors, to_f64
from tests.parity_util import check_forward, gpu, say

pytestmark = [
    pytest.mark.gpu,
    pytest.mark.skipif(not torch.cuda.is_available(), reason="needs a GPU"),
]

DT = {"bf16": torch.bfloat16, "f16": torch.float16}


def make_case(B, Hq, Hkv, d, page_size, lens, dtype, seed, spare_pages=3):
    """Random q and page pools, and a shuffled page table that gives each
    sequence the pages its length needs (unused table entries point at
    random pages too)."""
    g = np.random.default_rng(seed)
    max_pages = max(1, max(-(-n // page_size) for n in lens))
    num_pages = B * max_pages + spare_pages
    q, k_pages, v_pages, _ = random_tensors((B, Hq, 1, d), (num_pages, Hkv, page_size, d), dtype,
                                            seed)
    table = g.permutation(num_pages)[: B * max_pages].reshape(B, max_pages).astype(np.int32)
    return q, k_pages, v_pages, table, np.array(lens, dtype=np.int32)


def run_paged(q, k_pages, v_pages, table, lens, scale):
    o, lse = fa.forward_paged(gpu(q), gpu(k_pages), gpu(v_pages),
                              torch.from_numpy(table).cuda(), torch.from_numpy(lens).cuda(), scale)
    torch.cuda.synchronize()
    return o, lse


CASES = [
    # (B, Hq, Hkv, d, page_size, lens)
    (3, 8, 2, 128, 64, [1, 700, 1280]),
    (2, 32, 8, 64, 128, [0, 2000]),        # an empty sequence
    (2, 32, 1, 128, 256, [4096, 333]),     # MQA, group of 32 heads
    (4, 64, 1, 64, 64, [65, 64, 63, 1]),   # two groups of 32 heads per kv head
]


@pytest.mark.parametrize("dtype", ["bf16", "f16"])
@pytest.mark.parametrize("case", CASES, ids=[str(c) for c in CASES])
def test_paged_decode_matches_oracle(dtype, case):
    B, Hq, Hkv, d, ps, lens = case
    say(f"paged {case} {dtype}")
    q, kp, vp, table, ln = make_case(B, Hq, Hkv, d, ps, lens, dtype, seed=61)
    scale = 1.0 / np.sqrt(d)
    o, lse = run_paged(q, kp, vp, table, ln, scale)
    o_ref, lse_ref = oracle.paged_decode_forward(to_f64(q), to_f64(kp), to_f64(vp), table, ln, scale)
    check_forward(o, lse, o_ref, lse_ref, dtype, f"paged {case}")


def test_paged_full_size_sampled():
    """The decode shape of the pages' decode workload (B = 16, Hq = 32,
    Hkv = 8, up to 8192 keys, d = 128) with 128-key pages, random lengths."""
    g = np.random.default_rng(5)
    lens = [int(x) for x in g.integers(1, 8193, size=16)]
    lens[0] = 8192
    q, kp, vp, table, ln = make_case(16, 32, 8, 128, 128, lens, "bf16", seed=62)
    scale = 1.0 / np.sqrt(128)
    o, lse = run_paged(q, kp, vp, table, ln, scale)
    rows = [0, 5, 15]
    o_ref, lse_ref = oracle.paged_decode_forward(to_f64(q[rows]), to_f64(kp), to_f64(vp), table[rows],
                                                 ln[rows], scale)
    check_forward(o[rows], lse[rows], o_ref, lse_ref, "bf16", "paged full size")
    assert torch.isfinite(o).all()


def test_identity_table_equals_contiguous_decode_bitwise():
    """With pages laid out in order and every sequence full, paged decode
    runs the same arithmetic as the contiguous decode."""
    B, Hq, Hkv, d, ps, mp = 4, 32, 8, 128, 128, 16
    q, k, v = random_tensors((B, Hq, 1, d), (B, Hkv, ps * mp, d), "bf16", 63)[:3]
    # Contiguous [B, Hkv, N, d] -> pool [B * mp, Hkv, ps, d], page b*mp + p.
    kp = k.reshape(B, Hkv, mp, ps, d).permute(0, 2, 1, 3, 4).reshape(B * mp, Hkv, ps, d).contiguous()
    vp = v.reshape(B, Hkv, mp, ps, d).permute(0, 2, 1, 3, 4).reshape(B * mp, Hkv, ps, d).contiguous()
    table = np.arange(B * mp, dtype=np.int32).reshape(B, mp)
    ln = np.full(B, ps * mp, dtype=np.int32)
    o_p, lse_p = run_paged(q, kp, vp, table, ln, 0.1)
    o_c, lse_c = fa.forward(gpu(q), gpu(k), gpu(v), causal=False, scale=0.1)
    torch.cuda.synchronize()
    assert torch.equal(o_p, o_c)
    assert torch.equal(lse_p, lse_c)


def test_out_of_range_entries_drop_their_keys():
    """A table entry outside [0, num_pages) (too large or negative) names no
    page: its keys are dropped from the attention (never read, never scored),
    against the oracle with those keys removed; a sequence whose every entry
    is out of range gets O = 0, LSE = -inf."""
    B, Hq, Hkv, d, ps = 3, 8, 2, 64, 64
    q, kp, vp, table, ln = make_case(B, Hq, Hkv, d, ps, [3 * ps, 2 * ps + 7, 4 * ps], "bf16",
                                     seed=64)
    bad = table.copy()
    bad[0, 1] = 1 << 20
    bad[1, 0] = -5
    bad[2, :] = kp.shape[0]
    o_bad, lse_bad = run_paged(q, kp, vp, bad, ln, 0.125)
    o_ref, lse_ref = oracle.paged_decode_forward(to_f64(q), to_f64(kp), to_f64(vp), bad,
                                                 ln, 0.125)
    check_forward(o_bad[:2].cpu(), lse_bad[:2].cpu(), o_ref[:2], lse_ref[:2], "bf16",
                  "out-of-range entries")
    assert torch.all(o_bad[2] == 0) and torch.all(torch.isneginf(lse_bad[2]))
