"""C-ABI checks that need no GPU: the library loads, exports every symbol the
header declares, sizes workspaces as documented, and rejects bad arguments on
the host before any HIP call (so these run on a machine without a GPU)."""

import ctypes
import os
import re

import pytest

import exact_attention_115_amd as fa

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "fa.h")

pytestmark = pytest.mark.skipif(not os.path.exists(fa.LIB_PATH), reason="libfa.so not built")

# The library the checks below call: libfa.so through ctypes, unless another
# module (test_abi_sanitized.py) installs a stand-in with the same entry points.
BACKEND = {"lib": None}


def lib():
    return BACKEND["lib"] or fa.load()


def declared_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(fa_\w+)\s*\(", text)))


def test_exports_every_declared_symbol():
    lib = fa.load()
    names = declared_functions()
    assert {"fa_fwd", "fa_bwd", "fa_bwd_stage", "fa_strerror", "fa_version",
            "fa_fwd_workspace_size", "fa_bwd_workspace_size"} <= set(names)
    for n in names:
        assert hasattr(lib, n), n


def test_version_and_strerror():
    assert lib().fa_version() >= 100
    for code in [0, -1, -2, -3, -4, -5, -6, -7, -8, -9]:
        s = lib().fa_strerror(code).decode()
        assert s and s != "unknown status"
    assert lib().fa_strerror(-99).decode() == "unknown status"


def _align(x, a=256):
    return (x + a - 1) // a * a


def test_workspace_sizes():
    lib_ = lib()
    # Prefill forward needs none; float32 needs none.
    assert lib_.fa_fwd_workspace_size(1, 32, 32, 4096, 4096, 128, fa.FA_BF16) == 0
    assert lib_.fa_fwd_workspace_size(1, 1, 1, 1, 256, 64, fa.FA_F32) == 0
    # Decode: per split one float32 row (d values) plus one LSE per query head.
    ws = lib_.fa_fwd_workspace_size(16, 32, 8, 1, 8192, 128, fa.FA_BF16)
    assert ws > 0 and ws % 256 == 0
    rows = ws // (129 * 4)
    assert rows % (16 * 32) == 0
    # Backward: the float32 row terms D and LSE log2(e), linear in N.
    for B, Hq, Hkv, N, d in [(1, 32, 32, 4096, 128), (2, 16, 16, 1024, 64), (4, 32, 8, 2048, 128)]:
        want = 2 * _align(B * Hq * N * 4)
        assert lib_.fa_bwd_workspace_size(B, Hq, Hkv, N, N, d, fa.FA_BF16) == want
    # MQA with few key blocks: the head group is split over s workgroups, which
    # adds float32 partial dK and dV planes (s of each), s a divisor of G.
    B, Hq, Hkv, N, d = 4, 32, 1, 2048, 128
    base = 2 * _align(B * Hq * N * 4)
    extra = lib_.fa_bwd_workspace_size(B, Hq, Hkv, N, N, d, fa.FA_BF16) - base
    plane = B * Hkv * N * d * 4
    assert extra > 0 and extra % (2 * plane) == 0
    s = extra // (2 * plane)
    assert s > 1 and (Hq // Hkv) % s == 0
    assert lib_.fa_bwd_workspace_size(1, 1, 1, 10, 10, 64, fa.FA_F32) == 0
    # Invalid problems report 0.
    assert lib_.fa_bwd_workspace_size(1, 3, 2, 10, 10, 64, fa.FA_BF16) == 0
    assert lib_.fa_fwd_workspace_size(1, 2, 2, 1, 10, 96, fa.FA_BF16) == 0


# Fake, 256-byte aligned, never dereferenced device addresses: every call below
# must be rejected by the host-side checks before anything is enqueued.
BASE = 1 << 40


def P(i, off=0):
    return ctypes.c_void_p(BASE + i * (1 << 32) + off)


def fwd(q=P(1), k=P(2), v=P(3), o=P(4), lse=P(5), ws=None, ws_bytes=0, B=1, Hq=2, Hkv=2, Nq=64,
        Nkv=64, d=64, scale=0.125, causal=0, dt=fa.FA_BF16):
    return lib().fa_fwd(q, k, v, o, lse, ws, ws_bytes, B, Hq, Hkv, Nq, Nkv, d, scale, causal,
                            dt, None)


def bwd(q=P(1), k=P(2), v=P(3), o=P(4), lse=P(5), do=P(6), dq=P(7), dk=P(8), dv=P(9), ws=P(10),
        ws_bytes=1 << 30, B=1, Hq=2, Hkv=2, Nq=64, Nkv=64, d=64, scale=0.125, causal=0,
        dt=fa.FA_BF16, stage=None):
    args = (q, k, v, o, lse, do, dq, dk, dv, ws, ws_bytes, B, Hq, Hkv, Nq, Nkv, d, scale, causal, dt,
            None)
    if stage is None:
        return lib().fa_bwd(*args)
    return lib().fa_bwd_stage(stage, *args)


def test_fwd_rejects_bad_arguments():
    assert fwd(q=None) == -1
    assert fwd(lse=None) == -1
    assert fwd(Hq=3, Hkv=2) == -2
    assert fwd(Hkv=0) == -2
    assert fwd(Nq=-1) == -2
    assert fwd(d=96) == -3
    assert fwd(d=32) == -3
    assert fwd(dt=7) == -3
    assert fwd(q=P(1, 8)) == -4
    assert fwd(lse=P(5, 4)) == -4
    assert fwd(scale=0.0) == -6
    assert fwd(scale=-1.0) == -6
    assert fwd(scale=float("nan")) == -6
    assert fwd(scale=float("inf")) == -6
    assert fwd(causal=2) == -6
    assert fwd(o=P(1)) == -8          # output aliases q
    assert fwd(lse=P(4, 1024)) == -8  # lse inside o


def test_size_limits_are_enforced():
    """One head's K (or V) is addressed with 32-bit byte offsets: the calls
    accept N_kv * d * 4 < 2^31 (N_kv <= 4194303 at d = 128, 8388607 at
    d = 64) and B * Hq * N_q, B * Hkv * N_kv < 2^31; beyond that they return
    FA_ERR_UNSUPPORTED before touching any pointer."""
    assert fwd(Nkv=(1 << 31) // (128 * 4), d=128) == -3
    assert fwd(Nkv=(1 << 31) // (64 * 4), d=64) == -3
    assert fwd(Nq=1, Nkv=(1 << 31) // (128 * 4), d=128, ws=P(10), ws_bytes=1 << 30) == -3
    assert fwd(B=1, Hq=2, Hkv=2, Nq=1 << 30) == -3
    assert fwd(B=2, Hq=2, Hkv=1, Nkv=1 << 30) == -3
    assert bwd(Nkv=(1 << 31) // (128 * 4), d=128) == -3
    assert bwd(B=1, Hq=2, Hkv=2, Nq=1 << 30) == -3


def test_extreme_sizes_are_refused_without_overflow():
    """Sizes near INT_MAX in every argument: the size checks must refuse
    them without overflowing their own arithmetic (the sanitized replay of
    this module turns any signed overflow into a failure)."""
    M = (1 << 31) - 1
    lib_ = lib()
    for B, Hq, Hkv, Nq, Nkv in [(M, M, 1, M, 1), (M, M, M, M, M), (1, M, 1, M, M), (M, 1, 1, 1, M),
                                (M, M, 1, 1, 1)]:
        for d in (64, 128):
            assert fwd(B=B, Hq=Hq, Hkv=Hkv, Nq=Nq, Nkv=Nkv, d=d) == -3, (B, Hq, Hkv, Nq, Nkv, d)
            assert fwd(B=B, Hq=Hq, Hkv=Hkv, Nq=1, Nkv=Nkv, d=d, ws=P(10),
                       ws_bytes=1 << 40) in (-3, 0), (B, Hq, Hkv, Nkv, d)
            assert bwd(B=B, Hq=Hq, Hkv=Hkv, Nq=Nq, Nkv=Nkv, d=d) == -3, (B, Hq, Hkv, Nq, Nkv, d)
            for dt in (fa.FA_BF16, fa.FA_F32):
                assert lib_.fa_fwd_workspace_size(B, Hq, Hkv, Nq, Nkv, d, dt) == 0
                assert lib_.fa_bwd_workspace_size(B, Hq, Hkv, Nq, Nkv, d, dt) == 0
            assert lib_.fa_fwd_paged_workspace_size(B, Hq, Hkv, 64 * (M // 64), M, d,
                                                    fa.FA_BF16) == 0
            assert paged(B=B, Hq=Hq, Hkv=Hkv, num_pages=M, page_size=64 * (M // 64),
                         max_pages=M, d=d) == -3
    assert lib_.fa_dropout_mask(P(1), M, M, M, M, 0.5, 1, 0, None) == -3
    assert fwd_drop(B=M, Hq=M, Hkv=1, Nq=M, Nkv=M) == -3
    assert bwd_noalloc(B=M, Hq=M, Hkv=1, Nq=M, Nkv=M) == -3
    assert lib_.fa_bwd_dropout(P(1), P(2), P(3), P(4), P(5), P(6), P(7), P(8), P(9), P(10),
                               1 << 40, M, M, 1, M, M, 64, 0.125, 0, 0.1, 7, 0, fa.FA_BF16,
                               None) == -3
    assert lib_.fa_fwd_fp8(P(1), P(2), P(3), P(4), P(5), M, M, 1, M, M, 128, 0.1, 0, 1.0, 1.0,
                           1.0, None) == -3


def test_fwd_decode_needs_workspace():
    assert fwd(Nq=1, Nkv=8192, ws=None) == -1
    need = lib().fa_fwd_workspace_size(1, 2, 2, 1, 8192, 64, fa.FA_BF16)
    assert fwd(Nq=1, Nkv=8192, ws=P(10), ws_bytes=need - 1) == -5
    assert fwd(Nq=1, Nkv=8192, ws=P(10, 16), ws_bytes=need) == -4


def test_fwd_empty_problems_are_noops():
    assert fwd(Nq=0) == 0
    assert fwd(B=0) == 0
    assert fwd(Hq=0, Hkv=0) == 0


def test_bwd_rejects_bad_arguments():
    assert bwd(dt=fa.FA_F32) == -3
    assert bwd(do=None) == -1
    assert bwd(dk=None) == -1
    assert bwd(ws=None) == -1
    need = lib().fa_bwd_workspace_size(1, 2, 2, 64, 64, 64, fa.FA_BF16)
    assert need > 0 and bwd(ws_bytes=need - 1) == -5
    assert bwd(ws=P(10, 64)) == -4
    assert bwd(dq=P(7, 2)) == -4
    assert bwd(Hq=4, Hkv=3) == -2
    assert bwd(scale=0.0) == -6
    assert bwd(dq=P(1)) == -8          # dq aliases q
    assert bwd(dv=P(8)) == -8          # dv aliases dk
    assert bwd(ws=P(6)) == -8          # workspace aliases dO
    assert bwd(stage=3) == -3
    assert bwd(stage=-1) == -3
    assert bwd(B=0) == 0


def paged(q=P(1), kp=P(2), vp=P(3), table=P(4), lens=P(5), o=P(6), lse=P(7), ws=P(8),
          ws_bytes=1 << 30, B=2, Hq=4, Hkv=2, num_pages=8, page_size=64, max_pages=4, d=64,
          scale=0.125, dt=fa.FA_BF16):
    return lib().fa_fwd_paged(q, kp, vp, table, lens, o, lse, ws, ws_bytes, B, Hq, Hkv,
                                  num_pages, page_size, max_pages, d, scale, dt, None)


def test_paged_workspace_matches_contiguous_decode():
    lib_ = lib()
    for B, Hq, Hkv, ps, mp, d in [(16, 32, 8, 128, 64, 128), (3, 8, 2, 64, 20, 64), (2, 32, 1, 256, 8, 128)]:
        want = lib_.fa_fwd_workspace_size(B, Hq, Hkv, 1, ps * mp, d, fa.FA_BF16)
        assert lib_.fa_fwd_paged_workspace_size(B, Hq, Hkv, ps, mp, d, fa.FA_BF16) == want > 0
    assert lib_.fa_fwd_paged_workspace_size(2, 4, 2, 96, 4, 64, fa.FA_BF16) == 0   # page size
    assert lib_.fa_fwd_paged_workspace_size(2, 4, 2, 64, 4, 64, fa.FA_F32) == 0    # dtype


def test_paged_rejects_bad_arguments():
    assert paged(page_size=96) == -3          # not a multiple of 64
    assert paged(page_size=0) == -3
    assert paged(dt=fa.FA_F32) == -3
    assert paged(d=96) == -3
    assert paged(max_pages=0) == -2
    assert paged(num_pages=0) == -2
    assert paged(Hq=3) == -2
    assert paged(page_size=-64) == -2
    assert paged(table=None) == -1
    assert paged(lens=None) == -1
    assert paged(ws=None) == -1
    assert paged(lens=P(5, 2)) == -4          # int32 array not 4-byte aligned
    assert paged(q=P(1, 8)) == -4
    assert paged(ws=P(8, 16)) == -4
    need = lib().fa_fwd_paged_workspace_size(2, 4, 2, 64, 4, 64, fa.FA_BF16)
    assert paged(ws_bytes=need - 1) == -5
    assert paged(scale=0.0) == -6
    assert paged(o=P(1)) == -8                # output aliases q
    assert paged(ws=P(4)) == -8               # workspace aliases the page table
    assert paged(B=0) == 0                    # nothing to do


def fwd_drop(p=0.1, seed=1, offset=0, **kw):
    a = dict(q=P(1), k=P(2), v=P(3), o=P(4), lse=P(5), ws=None, ws_bytes=0, B=1, Hq=2, Hkv=2,
             Nq=64, Nkv=64, d=64, scale=0.125, causal=0, dt=fa.FA_BF16)
    a.update(kw)
    return lib().fa_fwd_dropout(a["q"], a["k"], a["v"], a["o"], a["lse"], a["ws"],
                                    a["ws_bytes"], a["B"], a["Hq"], a["Hkv"], a["Nq"], a["Nkv"],
                                    a["d"], a["scale"], a["causal"], p, seed, offset, a["dt"], None)


def test_fwd_dropout_rejects_bad_arguments():
    for p in (-0.1, 1.0, 1.5, float("nan"), float("inf")):
        assert fwd_drop(p=p) == -6, p
    assert fwd_drop(dt=fa.FA_F32) == -3
    assert fwd_drop(q=None) == -1
    assert fwd_drop(d=96) == -3
    assert fwd_drop(Hq=3, Hkv=2) == -2
    assert fwd_drop(scale=0.0) == -6
    assert fwd_drop(o=P(1)) == -8
    assert fwd_drop(Nq=0) == 0            # empty problem: nothing enqueued
    assert fwd_drop(Nq=0, p=2.0) == -6    # but the probability is still checked


def test_dropout_mask_rejects_bad_arguments():
    lib_ = lib()
    assert lib_.fa_dropout_mask(P(1), 1, 2, 3, 4, 1.0, 1, 0, None) == -6
    assert lib_.fa_dropout_mask(P(1), 1, 2, 3, 4, float("nan"), 1, 0, None) == -6
    assert lib_.fa_dropout_mask(P(1), -1, 2, 3, 4, 0.5, 1, 0, None) == -2
    assert lib_.fa_dropout_mask(None, 1, 2, 3, 4, 0.5, 1, 0, None) == -1
    assert lib_.fa_dropout_mask(None, 1, 2, 0, 4, 0.5, 1, 0, None) == 0
    assert lib_.fa_dropout_mask(P(1), 1 << 16, 1 << 16, 1, 1, 0.5, 1, 0, None) == -3


def test_bwd_dropout_rejects_bad_arguments():
    lib_ = lib()

    def call(p=0.1, **kw):
        a = dict(q=P(1), k=P(2), v=P(3), o=P(4), lse=P(5), do=P(6), dq=P(7), dk=P(8), dv=P(9),
                 ws=P(10), ws_bytes=1 << 30, B=1, Hq=2, Hkv=2, Nq=64, Nkv=64, d=64, scale=0.125,
                 causal=0, dt=fa.FA_BF16)
        a.update(kw)
        return lib_.fa_bwd_dropout(a["q"], a["k"], a["v"], a["o"], a["lse"], a["do"], a["dq"],
                                  a["dk"], a["dv"], a["ws"], a["ws_bytes"], a["B"], a["Hq"],
                                  a["Hkv"], a["Nq"], a["Nkv"], a["d"], a["scale"], a["causal"], p,
                                  7, 0, a["dt"], None)

    for p in (-0.5, 1.0, float("nan")):
        assert call(p=p) == -6, p
    assert call(dt=fa.FA_F32) == -3
    assert call(do=None) == -1
    assert call(ws=None) == -1
    assert call(dq=P(1)) == -8
    assert call(B=0) == 0


def test_fwd_fp8_rejects_bad_arguments():
    lib_ = lib()

    def call(**kw):
        a = dict(q=P(1), k=P(2), v=P(3), o=P(4), lse=P(5), B=1, Hq=2, Hkv=2, Nq=64, Nkv=64, d=128,
                 scale=0.1, causal=0, dq=1.0, dk=1.0, dv=1.0)
        a.update(kw)
        return lib_.fa_fwd_fp8(a["q"], a["k"], a["v"], a["o"], a["lse"], a["B"], a["Hq"], a["Hkv"],
                              a["Nq"], a["Nkv"], a["d"], a["scale"], a["causal"], a["dq"], a["dk"],
                              a["dv"], None)

    assert call(d=64) == -3
    assert call(d=96) == -3
    for x in (0.0, -1.0, float("nan"), float("inf")):
        assert call(dq=x) == -6 and call(dk=x) == -6 and call(dv=x) == -6
    assert call(scale=0.0) == -6
    assert call(q=None) == -1
    assert call(Hq=3, Hkv=2) == -2
    assert call(q=P(1, 8)) == -4
    assert call(o=P(1)) == -8
    assert call(Nq=0) == 0


def bwd_noalloc(q=P(1), k=P(2), v=P(3), o=P(4), lse=P(5), do=P(6), dq=P(7), dk=P(8), dv=P(9),
                B=1, Hq=2, Hkv=2, Nq=64, Nkv=64, d=64, scale=0.125, causal=0, dt=fa.FA_BF16):
    return lib().fa_bwd_noalloc(q, k, v, o, lse, do, dq, dk, dv, B, Hq, Hkv, Nq, Nkv, d, scale,
                                    causal, dt, None)


def test_bwd_noalloc_rejects_bad_arguments_before_any_hip_call():
    """fa_bwd_noalloc checks its arguments like fa_bwd (there is no workspace
    argument) and refuses a problem whose workspace exceeds the static
    scratch buffer, all before looking the buffer up (no HIP call)."""
    assert bwd_noalloc(dt=fa.FA_F32) == -3
    assert bwd_noalloc(do=None) == -1
    assert bwd_noalloc(dq=P(7, 2)) == -4
    assert bwd_noalloc(Hq=4, Hkv=3) == -2
    assert bwd_noalloc(scale=float("nan")) == -6
    assert bwd_noalloc(dq=P(1)) == -8
    assert bwd_noalloc(B=0) == 0
    lib_ = lib()
    scratch = 32 << 20
    # 2 float32 row terms per query row: 4 Mi + 64 rows need just over 32 MiB.
    B, Hq, Hkv, Nq, Nkv, d = 1, 64, 64, 65540, 64, 64
    assert lib_.fa_bwd_workspace_size(B, Hq, Hkv, Nq, Nkv, d, fa.FA_BF16) > scratch
    assert bwd_noalloc(B=B, Hq=Hq, Hkv=Hkv, Nq=Nq, Nkv=Nkv, d=d) == -9
    assert "static scratch" in lib_.fa_strerror(-9).decode()
