"""CPU tests of the Python binding's shape checks: every tensor a call reads
or writes must have the shape the sizes passed to the library imply, or the
call raises ValueError before any GPU work (a short v, o, lse, dO or
seq_lens would otherwise let the kernels run past the caller's buffers)."""

import pytest
import torch

import exact_attention_115_amd as fa

B, Hq, Hkv, Nq, Nkv, d = 2, 4, 2, 33, 40, 64


def t(*shape, dtype=torch.bfloat16):
    return torch.zeros(shape, dtype=dtype)


def fwd_args():
    return dict(q=t(B, Hq, Nq, d), k=t(B, Hkv, Nkv, d), v=t(B, Hkv, Nkv, d), o=t(B, Hq, Nq, d),
                lse=t(B, Hq, Nq, dtype=torch.float32))


def bwd_args():
    a = fwd_args()
    a.update(do=t(B, Hq, Nq, d), dq=t(B, Hq, Nq, d), dk=t(B, Hkv, Nkv, d), dv=t(B, Hkv, Nkv, d))
    return a


def call_fwd(a):
    return fa.fa_fwd(a["q"], a["k"], a["v"], a["o"], a["lse"], None, 0.125, True)


def call_bwd(a):
    return fa.fa_bwd(a["q"], a["k"], a["v"], a["o"], a["lse"], a["do"], a["dq"], a["dk"], a["dv"],
                     None, 0.125, True)


def test_matching_shapes_pass_the_shape_checks():
    # Correct shapes get past the shape checks and stop at the device check.
    with pytest.raises(ValueError, match="GPU tensor"):
        call_fwd(fwd_args())
    with pytest.raises(ValueError, match="GPU tensor"):
        call_bwd(bwd_args())


@pytest.mark.parametrize("name,shape", [
    ("v", (B, Hkv, Nkv - 1, d)),       # fewer keys in v than in k
    ("o", (B, Hq, Nq - 1, d)),
    ("lse", (B, Hq, Nq - 1)),
    ("lse", (B * Hq * Nq,)),
])
def test_forward_shape_mismatch_raises(name, shape):
    a = fwd_args()
    a[name] = t(*shape, dtype=a[name].dtype)
    with pytest.raises(ValueError, match=f"{name} has shape"):
        call_fwd(a)
    if name != "v":
        with pytest.raises(ValueError, match=f"{name} has shape"):
            fa.fa_fwd_dropout(a["q"], a["k"], a["v"], a["o"], a["lse"], None, 0.125, True, 0.1, 1)


@pytest.mark.parametrize("name,shape", [
    ("v", (B, Hkv, Nkv + 1, d)),
    ("o", (B, Hq, Nq, d // 2)),
    ("do", (B, Hq, Nq - 1, d)),
    ("dq", (B, Hq - 1, Nq, d)),
    ("dk", (B, Hkv, Nkv - 1, d)),
    ("dv", (B - 1, Hkv, Nkv, d)),
    ("lse", (B, Hq, Nq + 1)),
])
def test_backward_shape_mismatch_raises(name, shape):
    a = bwd_args()
    a[name] = t(*shape, dtype=a[name].dtype)
    with pytest.raises(ValueError, match=f"{name} has shape"):
        call_bwd(a)
    with pytest.raises(ValueError, match=f"{name} has shape"):
        fa.fa_bwd_stage(1, a["q"], a["k"], a["v"], a["o"], a["lse"], a["do"], a["dq"], a["dk"],
                        a["dv"], None, 0.125, True)
    with pytest.raises(ValueError, match=f"{name} has shape"):
        fa.fa_bwd_dropout(a["q"], a["k"], a["v"], a["o"], a["lse"], a["do"], a["dq"], a["dk"],
                          a["dv"], None, 0.125, True, 0.2, 3)


def test_paged_shape_mismatch_raises():
    q = t(3, 4, 1, d)
    kp = t(10, 2, 64, d)
    table = torch.zeros((3, 5), dtype=torch.int32)
    lens = torch.zeros(3, dtype=torch.int32)
    o = t(3, 4, 1, d)
    lse = t(3, 4, 1, dtype=torch.float32)
    with pytest.raises(ValueError, match="seq_lens has shape"):
        fa.fa_fwd_paged(q, kp, kp, table, lens[:2], o, lse, None, 0.1)
    with pytest.raises(ValueError, match="o has shape"):
        fa.fa_fwd_paged(q, kp, kp, table, lens, o[:2], lse, None, 0.1)
    with pytest.raises(ValueError, match="lse has"):
        fa.fa_fwd_paged(q, kp, kp, table, lens, o, lse[:2], None, 0.1)
    with pytest.raises(ValueError, match="same shape"):
        fa.fa_fwd_paged(q, kp, kp[:9], table, lens, o, lse, None, 0.1)
    with pytest.raises(ValueError, match="GPU tensor"):
        fa.fa_fwd_paged(q, kp, kp, table, lens, o, lse, None, 0.1)


def test_fp8_shape_mismatch_raises():
    q8 = torch.zeros((1, 2, 16, 128), dtype=torch.uint8)
    k8 = torch.zeros((1, 2, 20, 128), dtype=torch.uint8)
    o = t(1, 2, 16, 128)
    lse = t(1, 2, 16, dtype=torch.float32)
    with pytest.raises(ValueError, match="v has shape"):
        fa.fa_fwd_fp8(q8, k8, k8[:, :, :19], o, lse, 0.1, True)
    with pytest.raises(ValueError, match="o has shape"):
        fa.fa_fwd_fp8(q8, k8, k8, o[:, :1], lse, 0.1, True)
    with pytest.raises(ValueError, match="lse has shape"):
        fa.fa_fwd_fp8(q8, k8, k8, o, lse[..., :3], 0.1, True)
