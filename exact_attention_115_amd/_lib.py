"""ctypes binding of libfa.so (argument marshalling only).

Each C entry point of include/fa.h has a Python function of the same name
that takes torch tensors, checks device / dtype / contiguity / shape, and
passes raw device pointers, sizes and the current HIP stream through. Every
step of the computation runs in the library's kernels; PyTorch provides only
device memory and the stream. If the library is missing this module raises:
there is no fallback path.
"""

from __future__ import annotations

import ctypes
import math
import os

import torch

_PKG = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_PKG, "libfa.so")

FA_F32, FA_F16, FA_BF16 = 0, 1, 2
FA_OK = 0
STATUS_NAMES = {
    0: "FA_OK", -1: "FA_ERR_NULLPTR", -2: "FA_ERR_SHAPE", -3: "FA_ERR_UNSUPPORTED",
    -4: "FA_ERR_ALIGNMENT", -5: "FA_ERR_WORKSPACE", -6: "FA_ERR_SCALE", -7: "FA_ERR_HIP",
    -8: "FA_ERR_OVERLAP", -9: "FA_ERR_SCRATCH",
}
_DT = {torch.float32: FA_F32, torch.float16: FA_F16, torch.bfloat16: FA_BF16}

_lib = None


class FAError(RuntimeError):
    def __init__(self, status: int, where: str):
        self.status = status
        super().__init__(f"{where}: {STATUS_NAMES.get(status, status)} ({fa_strerror(status)})")


def load() -> ctypes.CDLL:
    """Load libfa.so once; raise if it has not been built."""
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(LIB_PATH):
        raise RuntimeError(
            f"{LIB_PATH} is missing: build it with exact_attention_115_amd.build.build() "
            "(there is no fallback implementation)")
    _lib = open_library(LIB_PATH)
    return _lib


def open_library(path: str) -> ctypes.CDLL:
    """Open a build of the library at ``path`` with the C signatures of
    include/fa.h declared (load() uses it for libfa.so)."""
    lib = ctypes.CDLL(path)
    vp, i, sz, f = ctypes.c_void_p, ctypes.c_int, ctypes.c_size_t, ctypes.c_float
    shape = [i, i, i, i, i, i]
    lib.fa_fwd_workspace_size.argtypes = shape + [i]
    lib.fa_fwd_workspace_size.restype = sz
    lib.fa_bwd_workspace_size.argtypes = shape + [i]
    lib.fa_bwd_workspace_size.restype = sz
    lib.fa_fwd.argtypes = [vp, vp, vp, vp, vp, vp, sz] + shape + [f, i, i, vp]
    lib.fa_fwd.restype = i
    bwd = [vp] * 9 + [vp, sz] + shape + [f, i, i, vp]
    lib.fa_bwd.argtypes = bwd
    lib.fa_bwd.restype = i
    lib.fa_bwd_stage.argtypes = [i] + bwd
    lib.fa_bwd_stage.restype = i
    lib.fa_bwd_noalloc.argtypes = [vp] * 9 + shape + [f, i, i, vp]
    lib.fa_bwd_noalloc.restype = i
    lib.fa_strerror.argtypes = [i]
    lib.fa_strerror.restype = ctypes.c_char_p
    lib.fa_version.argtypes = []
    lib.fa_version.restype = i
    lib.fa_fwd_paged_workspace_size.argtypes = [i, i, i, i, i, i, i]
    lib.fa_fwd_paged_workspace_size.restype = sz
    lib.fa_fwd_paged.argtypes = [vp] * 8 + [sz] + [i] * 7 + [f, i, vp]
    lib.fa_fwd_paged.restype = i
    u64 = ctypes.c_uint64
    lib.fa_fwd_dropout.argtypes = [vp, vp, vp, vp, vp, vp, sz] + shape + [f, i, f, u64, u64, i, vp]
    lib.fa_fwd_dropout.restype = i
    lib.fa_bwd_dropout.argtypes = bwd[:-2] + [f, u64, u64, i, vp]
    lib.fa_bwd_dropout.restype = i
    lib.fa_dropout_mask.argtypes = [vp, i, i, i, i, f, u64, u64, vp]
    lib.fa_fwd_fp8.argtypes = [vp] * 5 + shape + [f, i, f, f, f, vp]
    lib.fa_fwd_fp8.restype = i
    lib.fa_dropout_mask.restype = i
    return lib


def fa_strerror(status: int) -> str:
    return load().fa_strerror(int(status)).decode()


def fa_version() -> int:
    return load().fa_version()


def _dtype_code(t: torch.Tensor) -> int:
    if t.dtype not in _DT:
        raise TypeError(f"unsupported dtype {t.dtype}")
    return _DT[t.dtype]


def _ptr(t):
    return None if t is None else ctypes.c_void_p(t.data_ptr())


def _stream(stream):
    if stream is None:
        stream = torch.cuda.current_stream()
    return ctypes.c_void_p(stream.cuda_stream)


def _dims(q: torch.Tensor, k: torch.Tensor):
    if q.dim() != 4 or k.dim() != 4:
        raise ValueError("q, k, v must be 4-D [batch, heads, sequence, head_dim]")
    B, Hq, Nq, d = q.shape
    Bk, Hkv, Nkv, dk = k.shape
    if Bk != B or dk != d:
        raise ValueError(f"shape mismatch q {tuple(q.shape)} vs k {tuple(k.shape)}")
    return B, Hq, Hkv, Nq, Nkv, d


def _shape(name, t, shape):
    """Raise ValueError unless tensor t (if given) has exactly this shape."""
    if t is not None and tuple(t.shape) != tuple(shape):
        raise ValueError(f"{name} has shape {tuple(t.shape)}, expected {tuple(shape)}")


def _fwd_shapes(q, k, v, o, lse):
    """Shapes of a forward call: v like k, o like q, lse [B, Hq, N_q]."""
    B, Hq, Hkv, Nq, Nkv, d = _dims(q, k)
    _shape("v", v, k.shape)
    _shape("o", o, q.shape)
    _shape("lse", lse, (B, Hq, Nq))
    return B, Hq, Hkv, Nq, Nkv, d


def _check(ts, dtype=None):
    for name, t in ts.items():
        if t is None:
            continue
        if not t.is_cuda:
            raise ValueError(f"{name} must be a GPU tensor")
        if not t.is_contiguous():
            raise ValueError(f"{name} must be contiguous")
        if dtype is not None and t.dtype != dtype:
            raise TypeError(f"{name} has dtype {t.dtype}, expected {dtype}")


def fa_fwd_workspace_size(B, Hq, Hkv, Nq, Nkv, d, dtype) -> int:
    code = dtype if isinstance(dtype, int) else _DT[dtype]
    return int(load().fa_fwd_workspace_size(B, Hq, Hkv, Nq, Nkv, d, code))


def fa_bwd_workspace_size(B, Hq, Hkv, Nq, Nkv, d, dtype) -> int:
    code = dtype if isinstance(dtype, int) else _DT[dtype]
    return int(load().fa_bwd_workspace_size(B, Hq, Hkv, Nq, Nkv, d, code))


def fa_fwd(q, k, v, o, lse, workspace, scale: float, causal: bool, stream=None) -> int:
    """Call fa_fwd on tensors; returns the status code (no exception)."""
    B, Hq, Hkv, Nq, Nkv, d = _fwd_shapes(q, k, v, o, lse)
    _check({"q": q, "k": k, "v": v, "o": o}, q.dtype)
    _check({"lse": lse}, torch.float32)
    _check({"workspace": workspace})
    ws_bytes = 0 if workspace is None else workspace.numel() * workspace.element_size()
    return load().fa_fwd(_ptr(q), _ptr(k), _ptr(v), _ptr(o), _ptr(lse), _ptr(workspace), ws_bytes,
                         B, Hq, Hkv, Nq, Nkv, d, float(scale), int(bool(causal)), _dtype_code(q),
                         _stream(stream))


def _bwd_args(q, k, v, o, lse, do, dq, dk, dv, workspace, scale, causal, stream):
    B, Hq, Hkv, Nq, Nkv, d = _fwd_shapes(q, k, v, o, lse)
    _shape("do", do, q.shape)
    _shape("dq", dq, q.shape)
    _shape("dk", dk, k.shape)
    _shape("dv", dv, k.shape)
    _check({"q": q, "k": k, "v": v, "o": o, "do": do, "dq": dq, "dk": dk, "dv": dv}, q.dtype)
    _check({"lse": lse}, torch.float32)
    _check({"workspace": workspace})
    ws_bytes = 0 if workspace is None else workspace.numel() * workspace.element_size()
    return (_ptr(q), _ptr(k), _ptr(v), _ptr(o), _ptr(lse), _ptr(do), _ptr(dq), _ptr(dk), _ptr(dv),
            _ptr(workspace), ws_bytes, B, Hq, Hkv, Nq, Nkv, d, float(scale), int(bool(causal)),
            _dtype_code(q), _stream(stream))


def fa_bwd(q, k, v, o, lse, do, dq, dk, dv, workspace, scale: float, causal: bool, stream=None) -> int:
    """Call fa_bwd on tensors; returns the status code (no exception)."""
    return load().fa_bwd(*_bwd_args(q, k, v, o, lse, do, dq, dk, dv, workspace, scale, causal, stream))


def fa_bwd_stage(stage: int, q, k, v, o, lse, do, dq, dk, dv, workspace, scale: float, causal: bool,
                 stream=None) -> int:
    """Call fa_bwd_stage on tensors; returns the status code (no exception)."""
    return load().fa_bwd_stage(int(stage), *_bwd_args(q, k, v, o, lse, do, dq, dk, dv, workspace,
                                                      scale, causal, stream))


def fa_bwd_noalloc(q, k, v, o, lse, do, dq, dk, dv, scale: float, causal: bool, stream=None) -> int:
    """Call fa_bwd_noalloc (the backward on the library's static scratch
    buffer, no workspace argument); returns the status code (no exception)."""
    args = _bwd_args(q, k, v, o, lse, do, dq, dk, dv, None, scale, causal, stream)
    return load().fa_bwd_noalloc(*args[:9], *args[11:])


def _workspace(nbytes: int, device) -> torch.Tensor | None:
    if nbytes == 0:
        return None
    return torch.empty(nbytes, dtype=torch.uint8, device=device)


def _default_scale(d: int, scale):
    return 1.0 / math.sqrt(d) if scale is None else float(scale)


def forward(q, k, v, causal: bool = False, scale: float | None = None, stream=None):
    """O, LSE = attention(q, k, v). Allocates o, lse and the workspace."""
    B, Hq, Hkv, Nq, Nkv, d = _dims(q, k)
    o = torch.empty_like(q)
    lse = torch.empty((B, Hq, Nq), dtype=torch.float32, device=q.device)
    ws = _workspace(fa_fwd_workspace_size(B, Hq, Hkv, Nq, Nkv, d, q.dtype), q.device)
    st = fa_fwd(q, k, v, o, lse, ws, _default_scale(d, scale), causal, stream)
    if st != FA_OK:
        raise FAError(st, "fa_fwd")
    return o, lse


def backward(q, k, v, o, lse, do, causal: bool = False, scale: float | None = None, stream=None):
    """dq, dk, dv of sum(do * O). Allocates the gradients and the workspace."""
    B, Hq, Hkv, Nq, Nkv, d = _dims(q, k)
    dq, dk, dv = torch.empty_like(q), torch.empty_like(k), torch.empty_like(v)
    ws = _workspace(fa_bwd_workspace_size(B, Hq, Hkv, Nq, Nkv, d, q.dtype), q.device)
    st = fa_bwd(q, k, v, o, lse, do, dq, dk, dv, ws, _default_scale(d, scale), causal, stream)
    if st != FA_OK:
        raise FAError(st, "fa_bwd")
    return dq, dk, dv


def fa_fwd_paged_workspace_size(B, Hq, Hkv, page_size, max_pages, d, dtype) -> int:
    code = dtype if isinstance(dtype, int) else _DT[dtype]
    return int(load().fa_fwd_paged_workspace_size(B, Hq, Hkv, page_size, max_pages, d, code))


def _paged_dims(q, k_pages, page_table):
    if q.dim() != 4 or q.shape[2] != 1:
        raise ValueError("q must be [batch, heads, 1, head_dim]")
    if k_pages.dim() != 4:
        raise ValueError("k_pages, v_pages must be [num_pages, kv_heads, page_size, head_dim]")
    if page_table.dim() != 2 or page_table.shape[0] != q.shape[0]:
        raise ValueError("page_table must be [batch, max_pages]")
    B, Hq, _, d = q.shape
    num_pages, Hkv, page_size, dk = k_pages.shape
    if dk != d:
        raise ValueError(f"head_dim mismatch q {tuple(q.shape)} vs k_pages {tuple(k_pages.shape)}")
    return B, Hq, Hkv, num_pages, page_size, page_table.shape[1], d


def fa_fwd_paged(q, k_pages, v_pages, page_table, seq_lens, o, lse, workspace, scale: float,
                 stream=None) -> int:
    """Call fa_fwd_paged on tensors; returns the status code (no exception)."""
    if v_pages.shape != k_pages.shape:
        raise ValueError("k_pages and v_pages must have the same shape")
    B, Hq, Hkv, num_pages, page_size, max_pages, d = _paged_dims(q, k_pages, page_table)
    _shape("seq_lens", seq_lens, (B,))
    _shape("o", o, q.shape)
    if lse is not None and lse.numel() != B * Hq:
        raise ValueError(f"lse has {lse.numel()} elements, expected B * Hq = {B * Hq}")
    _check({"q": q, "k_pages": k_pages, "v_pages": v_pages, "o": o}, q.dtype)
    _check({"page_table": page_table, "seq_lens": seq_lens}, torch.int32)
    _check({"lse": lse}, torch.float32)
    _check({"workspace": workspace})
    ws_bytes = 0 if workspace is None else workspace.numel() * workspace.element_size()
    return load().fa_fwd_paged(_ptr(q), _ptr(k_pages), _ptr(v_pages), _ptr(page_table),
                               _ptr(seq_lens), _ptr(o), _ptr(lse), _ptr(workspace), ws_bytes, B, Hq,
                               Hkv, num_pages, page_size, max_pages, d, float(scale),
                               _dtype_code(q), _stream(stream))


def forward_paged(q, k_pages, v_pages, page_table, seq_lens, scale: float | None = None,
                  stream=None):
    """Decode over a paged K/V cache: O [B, Hq, 1, d], LSE [B, Hq, 1].
    Allocates o, lse and the workspace."""
    B, Hq, Hkv, num_pages, page_size, max_pages, d = _paged_dims(q, k_pages, page_table)
    o = torch.empty_like(q)
    lse = torch.empty((B, Hq, 1), dtype=torch.float32, device=q.device)
    ws = _workspace(fa_fwd_paged_workspace_size(B, Hq, Hkv, page_size, max_pages, d, q.dtype),
                    q.device)
    st = fa_fwd_paged(q, k_pages, v_pages, page_table, seq_lens, o, lse, ws,
                      _default_scale(d, scale), stream)
    if st != FA_OK:
        raise FAError(st, "fa_fwd_paged")
    return o, lse


# ------------------------------------------------------------------ dropout

def fa_fwd_dropout(q, k, v, o, lse, workspace, scale: float, causal: bool, dropout_p: float,
                   seed: int, offset: int = 0, stream=None) -> int:
    """Call fa_fwd_dropout on tensors; returns the status code (no exception)."""
    B, Hq, Hkv, Nq, Nkv, d = _fwd_shapes(q, k, v, o, lse)
    _check({"q": q, "k": k, "v": v, "o": o}, q.dtype)
    _check({"lse": lse}, torch.float32)
    _check({"workspace": workspace})
    ws_bytes = 0 if workspace is None else workspace.numel() * workspace.element_size()
    return load().fa_fwd_dropout(_ptr(q), _ptr(k), _ptr(v), _ptr(o), _ptr(lse), _ptr(workspace),
                                 ws_bytes, B, Hq, Hkv, Nq, Nkv, d, float(scale),
                                 int(bool(causal)), float(dropout_p), int(seed), int(offset),
                                 _dtype_code(q), _stream(stream))


def forward_dropout(q, k, v, dropout_p: float, seed: int, offset: int = 0, causal: bool = False,
                    scale: float | None = None, stream=None):
    """O, LSE of attention with dropout on P (see fa_fwd_dropout in fa.h).
    Allocates o, lse and the workspace."""
    B, Hq, Hkv, Nq, Nkv, d = _dims(q, k)
    o = torch.empty_like(q)
    lse = torch.empty((B, Hq, Nq), dtype=torch.float32, device=q.device)
    ws = _workspace(fa_fwd_workspace_size(B, Hq, Hkv, Nq, Nkv, d, q.dtype), q.device)
    st = fa_fwd_dropout(q, k, v, o, lse, ws, _default_scale(d, scale), causal, dropout_p, seed,
                        offset, stream)
    if st != FA_OK:
        raise FAError(st, "fa_fwd_dropout")
    return o, lse


def fa_bwd_dropout(q, k, v, o, lse, do, dq, dk, dv, workspace, scale: float, causal: bool,
                   dropout_p: float, seed: int, offset: int = 0, stream=None) -> int:
    """Call fa_bwd_dropout on tensors; returns the status code (no exception)."""
    args = _bwd_args(q, k, v, o, lse, do, dq, dk, dv, workspace, scale, causal, stream)
    return load().fa_bwd_dropout(*args[:-2], float(dropout_p), int(seed), int(offset), *args[-2:])


def backward_dropout(q, k, v, o, lse, do, dropout_p: float, seed: int, offset: int = 0,
                     causal: bool = False, scale: float | None = None, stream=None):
    """dq, dk, dv for forward_dropout with the same (dropout_p, seed, offset)."""
    B, Hq, Hkv, Nq, Nkv, d = _dims(q, k)
    dq, dk, dv = torch.empty_like(q), torch.empty_like(k), torch.empty_like(v)
    ws = _workspace(fa_bwd_workspace_size(B, Hq, Hkv, Nq, Nkv, d, q.dtype), q.device)
    st = fa_bwd_dropout(q, k, v, o, lse, do, dq, dk, dv, ws, _default_scale(d, scale), causal,
                        dropout_p, seed, offset, stream)
    if st != FA_OK:
        raise FAError(st, "fa_bwd_dropout")
    return dq, dk, dv


def fa_dropout_mask(keep, B: int, Hq: int, Nq: int, Nkv: int, dropout_p: float, seed: int,
                    offset: int = 0, stream=None) -> int:
    """Call fa_dropout_mask into a uint8 tensor [B, Hq, Nq, Nkv]; returns the status."""
    _check({"keep": keep}, torch.uint8)
    if keep is not None and keep.numel() < B * Hq * Nq * Nkv:
        raise ValueError("keep is smaller than B * Hq * Nq * Nkv bytes")
    return load().fa_dropout_mask(_ptr(keep), int(B), int(Hq), int(Nq), int(Nkv),
                                  float(dropout_p), int(seed), int(offset), _stream(stream))


def dropout_mask(B: int, Hq: int, Nq: int, Nkv: int, dropout_p: float, seed: int, offset: int = 0,
                 device="cuda", stream=None):
    """The keep mask of fa_fwd_dropout as a uint8 tensor [B, Hq, Nq, Nkv] (1 = kept)."""
    keep = torch.empty((B, Hq, Nq, Nkv), dtype=torch.uint8, device=device)
    st = fa_dropout_mask(keep, B, Hq, Nq, Nkv, dropout_p, seed, offset, stream)
    if st != FA_OK:
        raise FAError(st, "fa_dropout_mask")
    return keep


# ---------------------------------------------------------------------- fp8

_FP8_TYPES = (torch.uint8,) + ((torch.float8_e4m3fn,) if hasattr(torch, "float8_e4m3fn") else ())


def fa_fwd_fp8(q8, k8, v8, o, lse, scale: float, causal: bool, descale_q: float = 1.0,
               descale_k: float = 1.0, descale_v: float = 1.0, stream=None) -> int:
    """Call fa_fwd_fp8 (E4M3 codes as uint8 or float8_e4m3fn tensors, o bf16);
    returns the status code (no exception)."""
    B, Hq, Hkv, Nq, Nkv, d = _fwd_shapes(q8, k8, v8, o, lse)
    for name, t in {"q8": q8, "k8": k8, "v8": v8}.items():
        _check({name: t})
        if t.dtype not in _FP8_TYPES:
            raise TypeError(f"{name} must hold E4M3 codes (uint8 or float8_e4m3fn), not {t.dtype}")
    _check({"o": o}, torch.bfloat16)
    _check({"lse": lse}, torch.float32)
    return load().fa_fwd_fp8(_ptr(q8), _ptr(k8), _ptr(v8), _ptr(o), _ptr(lse), B, Hq, Hkv, Nq,
                             Nkv, d, float(scale), int(bool(causal)), float(descale_q),
                             float(descale_k), float(descale_v), _stream(stream))


def forward_fp8(q8, k8, v8, descale_q: float = 1.0, descale_k: float = 1.0, descale_v: float = 1.0,
                causal: bool = False, scale: float | None = None, stream=None):
    """O (bf16), LSE of attention over E4M3 inputs (see fa_fwd_fp8 in fa.h)."""
    B, Hq, Hkv, Nq, Nkv, d = _dims(q8, k8)
    o = torch.empty((B, Hq, Nq, d), dtype=torch.bfloat16, device=q8.device)
    lse = torch.empty((B, Hq, Nq), dtype=torch.float32, device=q8.device)
    st = fa_fwd_fp8(q8, k8, v8, o, lse, _default_scale(d, scale), causal, descale_q, descale_k,
                    descale_v, stream)
    if st != FA_OK:
        raise FAError(st, "fa_fwd_fp8")
    return o, lse
