"""Thin ctypes binding of libattn_mi355x.so (include/attn.h).

Argument marshalling only: shapes, strides, device pointers and the current
HIP stream go to the C ABI; every step of the computation runs in the
library's HIP kernels.  torch is used for device memory and streams.  There is
no fallback: if the library is missing, every call raises.

    o, lse = fwd(q, k, v, causal=False, offset=0, seqlens_q=None, seqlens_k=None)
    dq, dk, dv = bwd(q, k, v, o, lse, do, causal=..., offset=..., ...)

Tensors are [B, H, n, d] with unit stride in d (any batch/head/row strides that
are multiples of 8 elements), dtype torch.bfloat16 or torch.float32, on the GPU.
``offset`` is one causal offset for every sequence or a list of B of them.
Packed ("varlen") sequences: pass cu_seqlens_q / cu_seqlens_k (B + 1 row
offsets) and tensors [total_rows, H, d]; lse is then [H_q, total_q_rows].
"""

from __future__ import annotations

import ctypes
import os
from typing import Optional, Sequence

PKG = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(PKG, "libattn_mi355x.so")

OK = 0
INVALID_ARG = 1
EMPTY_ROW = 2
UNSUPPORTED = 3
WORKSPACE = 4
HIP = 5
F32 = 0
BF16 = 1

# every symbol the header declares
EXPORTS = ("attn_validate", "attn_bwd_workspace_size", "attn_fwd", "attn_bwd", "attn_bwd_gs_workspace_size",
           "attn_bwd_gs", "attn_bwd_gs_stage", "attn_bwd_noalloc",
           "attn_bwd_dq", "attn_bwd_dkdv", "attn_fwd_splitkv_workspace_size", "attn_fwd_splitkv",
           "attn_rope_apply", "attn_fwd_rope_workspace_size", "attn_fwd_rope",
           "attn_bwd_rope_workspace_size", "attn_bwd_rope", "attn_gemm_create", "attn_gemm_destroy",
           "attn_linear_fwd", "attn_linear_bwd",
           "attn_self_attention_fwd", "attn_self_attention_bwd_workspace_size", "attn_self_attention_bwd",
           "attn_status_string", "attn_version")


class AttnError(RuntimeError):
    def __init__(self, status: int, what: str = ""):
        self.status = status
        msg = status_string(status) if _lib_or_none() else f"status {status}"
        super().__init__(f"{what}: {msg} (status {status})" if what else f"{msg} (status {status})")


class Mask(ctypes.Structure):
    _fields_ = [("causal", ctypes.c_int32), ("reserved", ctypes.c_int32),
                ("causal_offset", ctypes.c_int64),
                ("seqlens_q", ctypes.POINTER(ctypes.c_int32)),
                ("seqlens_k", ctypes.POINTER(ctypes.c_int32)),
                ("causal_offsets", ctypes.POINTER(ctypes.c_int64))]


class Problem(ctypes.Structure):
    _fields_ = [("B", ctypes.c_int32), ("H_q", ctypes.c_int32), ("H_kv", ctypes.c_int32),
                ("n_q", ctypes.c_int32), ("n_k", ctypes.c_int32),
                ("d_h", ctypes.c_int32), ("d_v", ctypes.c_int32), ("dtype", ctypes.c_int32),
                ("q_stride", ctypes.c_int64 * 3), ("k_stride", ctypes.c_int64 * 3),
                ("v_stride", ctypes.c_int64 * 3), ("o_stride", ctypes.c_int64 * 3),
                ("cu_seqlens_q", ctypes.POINTER(ctypes.c_int32)),
                ("cu_seqlens_k", ctypes.POINTER(ctypes.c_int32))]


class Linear(ctypes.Structure):
    _fields_ = [("rows", ctypes.c_int32), ("d_in", ctypes.c_int32), ("d_out", ctypes.c_int32),
                ("dtype", ctypes.c_int32), ("ld_x", ctypes.c_int64), ("ld_w", ctypes.c_int64),
                ("ld_y", ctypes.c_int64)]


class Rope(ctypes.Structure):
    _fields_ = [("cos_sin", ctypes.c_void_p), ("n_pos", ctypes.c_int32), ("reserved", ctypes.c_int32)]


_LIB = None


def _lib_or_none():
    return _LIB


def lib():
    """Load the library (once).  Raises if it has not been built."""
    global _LIB
    if _LIB is not None:
        return _LIB
    if not os.path.exists(LIB_PATH):
        raise RuntimeError(f"{LIB_PATH} is missing: build it with "
                           "`python -m exact_masked_scaled_amd.build` (there is no fallback path)")
    L = ctypes.CDLL(LIB_PATH)
    P, M = ctypes.POINTER(Problem), ctypes.POINTER(Mask)
    vp = ctypes.c_void_p
    L.attn_validate.argtypes = [P, M]
    L.attn_validate.restype = ctypes.c_int
    L.attn_bwd_workspace_size.argtypes = [P]
    L.attn_bwd_workspace_size.restype = ctypes.c_size_t
    L.attn_fwd.argtypes = [P, M, vp, vp, vp, vp, vp, vp]
    L.attn_fwd.restype = ctypes.c_int
    L.attn_bwd.argtypes = [P, M, vp, vp, vp, vp, vp, vp, vp, vp, vp, vp, ctypes.c_size_t, vp]
    L.attn_bwd.restype = ctypes.c_int
    L.attn_bwd_gs_workspace_size.argtypes = [P]
    L.attn_bwd_gs_workspace_size.restype = ctypes.c_size_t
    L.attn_bwd_gs.argtypes = [P, M, vp, vp, vp, vp, vp, vp, vp, vp, vp, vp, ctypes.c_size_t, vp]
    L.attn_bwd_gs.restype = ctypes.c_int
    L.attn_bwd_gs_stage.argtypes = [P, M, vp, vp, vp, vp, vp, vp, vp, vp, vp, vp, ctypes.c_size_t, ctypes.c_int32, vp]
    L.attn_bwd_gs_stage.restype = ctypes.c_int
    L.attn_bwd_noalloc.argtypes = [P, M, vp, vp, vp, vp, vp, vp, vp, vp, vp, vp]
    L.attn_bwd_noalloc.restype = ctypes.c_int
    L.attn_bwd_dq.argtypes = [P, M, vp, vp, vp, vp, vp, vp, vp, vp, ctypes.c_size_t, vp]
    L.attn_bwd_dq.restype = ctypes.c_int
    L.attn_bwd_dkdv.argtypes = [P, M, vp, vp, vp, vp, vp, vp, vp, vp, ctypes.c_size_t, vp]
    L.attn_bwd_dkdv.restype = ctypes.c_int
    L.attn_fwd_splitkv_workspace_size.argtypes = [P, ctypes.c_int32]
    L.attn_fwd_splitkv_workspace_size.restype = ctypes.c_size_t
    L.attn_fwd_splitkv.argtypes = [P, M, vp, vp, vp, vp, vp, ctypes.c_int32, vp, ctypes.c_size_t, vp]
    L.attn_fwd_splitkv.restype = ctypes.c_int
    R = ctypes.POINTER(Rope)
    L.attn_rope_apply.argtypes = [P, M, R, ctypes.c_int32, ctypes.c_int32, vp, vp, vp]
    L.attn_rope_apply.restype = ctypes.c_int
    L.attn_fwd_rope_workspace_size.argtypes = [P]
    L.attn_fwd_rope_workspace_size.restype = ctypes.c_size_t
    L.attn_fwd_rope.argtypes = [P, M, R, vp, vp, vp, vp, vp, vp, ctypes.c_size_t, vp]
    L.attn_fwd_rope.restype = ctypes.c_int
    L.attn_bwd_rope_workspace_size.argtypes = [P]
    L.attn_bwd_rope_workspace_size.restype = ctypes.c_size_t
    L.attn_bwd_rope.argtypes = [P, M, R, vp, vp, vp, vp, vp, vp, vp, vp, vp, vp, ctypes.c_size_t, vp]
    L.attn_bwd_rope.restype = ctypes.c_int
    LP = ctypes.POINTER(Linear)
    L.attn_gemm_create.argtypes = [ctypes.POINTER(vp)]
    L.attn_gemm_create.restype = ctypes.c_int
    L.attn_gemm_destroy.argtypes = [vp]
    L.attn_gemm_destroy.restype = ctypes.c_int
    L.attn_linear_fwd.argtypes = [LP, vp, vp, vp, vp, vp]
    L.attn_linear_fwd.restype = ctypes.c_int
    L.attn_linear_bwd.argtypes = [LP, vp, vp, vp, vp, vp, vp, ctypes.c_int32, vp]
    L.attn_linear_bwd.restype = ctypes.c_int
    L.attn_self_attention_fwd.argtypes = [P, M, vp, ctypes.c_int32, vp, vp, vp, vp, vp, vp]
    L.attn_self_attention_fwd.restype = ctypes.c_int
    L.attn_self_attention_bwd_workspace_size.argtypes = [P]
    L.attn_self_attention_bwd_workspace_size.restype = ctypes.c_size_t
    L.attn_self_attention_bwd.argtypes = [P, M, vp, ctypes.c_int32, vp, vp, vp, vp, vp, vp, vp, vp, vp,
                                          ctypes.c_size_t, vp]
    L.attn_self_attention_bwd.restype = ctypes.c_int
    L.attn_status_string.argtypes = [ctypes.c_int]
    L.attn_status_string.restype = ctypes.c_char_p
    L.attn_version.argtypes = []
    L.attn_version.restype = ctypes.c_int32
    _LIB = L
    return L


def status_string(status: int) -> str:
    return lib().attn_status_string(int(status)).decode()


# ---------------------------------------------------------------------------
# problem / mask construction (plain integers; usable without a GPU)
# ---------------------------------------------------------------------------

def _i32_array(vals):
    arr = (ctypes.c_int32 * len(vals))(*[int(x) for x in vals])
    return arr, ctypes.cast(arr, ctypes.POINTER(ctypes.c_int32))


def make_problem(B, H_q, H_kv, n_q, n_k, d_h, d_v, dtype, q_stride=None, k_stride=None,
                 v_stride=None, o_stride=None, cu_seqlens_q=None, cu_seqlens_k=None) -> Problem:
    """With cu_seqlens_q / cu_seqlens_k (B + 1 row offsets each) the problem is in
    the packed layout: default strides are then those of contiguous
    [total_rows, H, d] tensors (batch stride 0).  The returned Problem keeps
    its host arrays alive (attribute ``_keep``)."""
    packed = cu_seqlens_q is not None or cu_seqlens_k is not None

    def contig(H, n, d):
        return (0, d, H * d) if packed else (H * n * d, n * d, d)
    p = Problem()
    p.B, p.H_q, p.H_kv, p.n_q, p.n_k, p.d_h, p.d_v, p.dtype = B, H_q, H_kv, n_q, n_k, d_h, d_v, dtype
    p.q_stride[:] = q_stride or contig(H_q, n_q, d_h)
    p.k_stride[:] = k_stride or contig(H_kv, n_k, d_h)
    p.v_stride[:] = v_stride or contig(H_kv, n_k, d_v)
    p.o_stride[:] = o_stride or contig(H_q, n_q, d_v)
    p._keep = []
    for name, cu in (("cu_seqlens_q", cu_seqlens_q), ("cu_seqlens_k", cu_seqlens_k)):
        if cu is None:
            setattr(p, name, None)
        else:
            arr, ptr = _i32_array(cu)
            p._keep.append(arr)
            setattr(p, name, ptr)
    return p


def make_mask(causal=False, offset=0, seqlens_q: Optional[Sequence[int]] = None,
              seqlens_k: Optional[Sequence[int]] = None):
    """Returns (Mask, keepalive) -- the host arrays must outlive the call.
    ``offset``: one causal offset, or a sequence of per-sequence offsets."""
    m = Mask()
    m.causal = 1 if causal else 0
    m.reserved = 0
    keep = []
    if isinstance(offset, (int,)) or (hasattr(offset, "ndim") and offset.ndim == 0):
        m.causal_offset = int(offset)
        m.causal_offsets = None
    else:
        m.causal_offset = 0
        arr = (ctypes.c_int64 * len(offset))(*[int(x) for x in offset])
        keep.append(arr)
        m.causal_offsets = ctypes.cast(arr, ctypes.POINTER(ctypes.c_int64))
    for name, lens in (("seqlens_q", seqlens_q), ("seqlens_k", seqlens_k)):
        if lens is None:
            setattr(m, name, None)
        else:
            arr = (ctypes.c_int32 * len(lens))(*[int(x) for x in lens])
            keep.append(arr)
            setattr(m, name, ctypes.cast(arr, ctypes.POINTER(ctypes.c_int32)))
    return m, keep


def validate(prob: Problem, mask: Mask) -> int:
    return int(lib().attn_validate(ctypes.byref(prob), ctypes.byref(mask)))


def workspace_size(prob: Problem) -> int:
    return int(lib().attn_bwd_workspace_size(ctypes.byref(prob)))


def gs_workspace_size(prob: Problem) -> int:
    return int(lib().attn_bwd_gs_workspace_size(ctypes.byref(prob)))


# ---------------------------------------------------------------------------
# torch entry points
# ---------------------------------------------------------------------------

def _torch():
    import torch
    return torch


def _dtype_code(t) -> int:
    torch = _torch()
    if t.dtype == torch.bfloat16:
        return BF16
    if t.dtype == torch.float32:
        return F32
    raise TypeError(f"unsupported dtype {t.dtype}")


def _check4(name, t, dtype, ndim=4):
    if t.dim() != ndim:
        raise ValueError(f"{name} must be " + ("[B, H, n, d]" if ndim == 4 else "[rows, H, d]"))
    if t.dtype != dtype:
        raise TypeError(f"{name} has dtype {t.dtype}, expected {dtype}")
    if not t.is_cuda:
        raise ValueError(f"{name} must be a GPU tensor")
    if t.shape[-1] > 0 and t.stride(-1) != 1:
        raise ValueError(f"{name} must have unit stride in its last dimension")


def _strides(t):
    """ABI strides (batch, head, row): [B, H, n, d] tensors directly, packed
    [rows, H, d] tensors with batch stride 0."""
    if t.dim() == 3:
        return (0, int(t.stride(1)), int(t.stride(0)))
    return tuple(int(s) for s in t.stride()[:3])


def _ptr(t):
    return ctypes.c_void_p(t.data_ptr()) if t is not None and t.numel() > 0 else ctypes.c_void_p(0)


def _packed_lengths(cu):
    cu = [int(x) for x in cu]
    return cu, [cu[i + 1] - cu[i] for i in range(len(cu) - 1)]


def _problem_from(q, k, v, o_like_stride=None, cu_seqlens_q=None, cu_seqlens_k=None,
                  max_seqlen_q=None, max_seqlen_k=None):
    if cu_seqlens_q is None and cu_seqlens_k is None:
        B, H_q, n_q, d_h = q.shape
        _, H_kv, n_k, d_v = v.shape
        return make_problem(B, H_q, H_kv, n_q, n_k, d_h, d_v, _dtype_code(q), _strides(q), _strides(k),
                            _strides(v), o_like_stride)
    if cu_seqlens_q is None or cu_seqlens_k is None:
        raise ValueError("the packed layout needs both cu_seqlens_q and cu_seqlens_k")
    cu_q, lq = _packed_lengths(cu_seqlens_q)
    cu_k, lk = _packed_lengths(cu_seqlens_k)
    if len(cu_q) != len(cu_k) or len(cu_q) < 1:
        raise ValueError("cu_seqlens_q and cu_seqlens_k must both hold B + 1 offsets")
    _, H_q, d_h = q.shape
    _, H_kv, d_v = v.shape
    n_q = int(max_seqlen_q) if max_seqlen_q is not None else max(lq, default=0)
    n_k = int(max_seqlen_k) if max_seqlen_k is not None else max(lk, default=0)
    return make_problem(len(cu_q) - 1, H_q, H_kv, n_q, n_k, d_h, d_v, _dtype_code(q), _strides(q),
                        _strides(k), _strides(v), o_like_stride, cu_q, cu_k)


def _stream(stream):
    torch = _torch()
    s = stream if stream is not None else torch.cuda.current_stream()
    return ctypes.c_void_p(s.cuda_stream)


def fwd(q, k, v, *, causal=False, offset=0, seqlens_q=None, seqlens_k=None, out=None, lse=None,
        stream=None, cu_seqlens_q=None, cu_seqlens_k=None, max_seqlen_q=None, max_seqlen_k=None):
    """O (dtype of q) and float32 lse: [B,H_q,n_q,d_v] and [B,H_q,n_q], or in
    the packed layout [total_q,H_q,d_v] and [H_q,total_q]."""
    torch = _torch()
    packed = cu_seqlens_q is not None or cu_seqlens_k is not None
    nd = 3 if packed else 4
    for name, t in (("q", q), ("k", k), ("v", v)):
        _check4(name, t, q.dtype, nd)
    d_v = v.shape[-1]
    if packed:
        total_q, H_q, _ = q.shape
        o_shape, lse_shape = (total_q, H_q, d_v), (H_q, total_q)
    else:
        B, H_q, n_q, _ = q.shape
        o_shape, lse_shape = (B, H_q, n_q, d_v), (B, H_q, n_q)
    if out is None:
        out = torch.empty(*o_shape, dtype=q.dtype, device=q.device)
    if lse is None:
        lse = torch.empty(*lse_shape, dtype=torch.float32, device=q.device)
    _check4("out", out, q.dtype, nd)
    if not lse.is_contiguous() or lse.dtype != torch.float32 or tuple(lse.shape) != lse_shape:
        raise ValueError(f"lse must be contiguous float32 of shape {lse_shape}")
    prob = _problem_from(q, k, v, _strides(out), cu_seqlens_q, cu_seqlens_k, max_seqlen_q, max_seqlen_k)
    mask, keep = make_mask(causal, offset, seqlens_q, seqlens_k)
    st = lib().attn_fwd(ctypes.byref(prob), ctypes.byref(mask), _ptr(q), _ptr(k), _ptr(v), _ptr(out),
                        _ptr(lse), _stream(stream))
    del keep
    if st != OK:
        raise AttnError(st, "attn_fwd")
    return out, lse


def splitkv_workspace_size(prob: Problem, num_splits: int = 0) -> int:
    return int(lib().attn_fwd_splitkv_workspace_size(ctypes.byref(prob), int(num_splits)))


def fwd_splitkv(q, k, v, *, num_splits=0, causal=False, offset=0, seqlens_q=None, seqlens_k=None,
                out=None, lse=None, workspace=None, stream=None, cu_seqlens_q=None, cu_seqlens_k=None,
                max_seqlen_q=None, max_seqlen_k=None):
    """The forward split over the keys (attn_fwd_splitkv): same results as
    fwd(); num_splits <= 0 lets the library choose."""
    torch = _torch()
    packed = cu_seqlens_q is not None or cu_seqlens_k is not None
    nd = 3 if packed else 4
    for name, t in (("q", q), ("k", k), ("v", v)):
        _check4(name, t, q.dtype, nd)
    d_v = v.shape[-1]
    if packed:
        total_q, H_q, _ = q.shape
        o_shape, lse_shape = (total_q, H_q, d_v), (H_q, total_q)
    else:
        B, H_q, n_q, _ = q.shape
        o_shape, lse_shape = (B, H_q, n_q, d_v), (B, H_q, n_q)
    if out is None:
        out = torch.empty(*o_shape, dtype=q.dtype, device=q.device)
    if lse is None:
        lse = torch.empty(*lse_shape, dtype=torch.float32, device=q.device)
    _check4("out", out, q.dtype, nd)
    if not lse.is_contiguous() or lse.dtype != torch.float32 or tuple(lse.shape) != lse_shape:
        raise ValueError(f"lse must be contiguous float32 of shape {lse_shape}")
    prob = _problem_from(q, k, v, _strides(out), cu_seqlens_q, cu_seqlens_k, max_seqlen_q, max_seqlen_k)
    need = splitkv_workspace_size(prob, num_splits)
    if workspace is None:
        workspace = torch.empty(max(need, 1), dtype=torch.uint8, device=q.device)
    mask, keep = make_mask(causal, offset, seqlens_q, seqlens_k)
    st = lib().attn_fwd_splitkv(ctypes.byref(prob), ctypes.byref(mask), _ptr(q), _ptr(k), _ptr(v), _ptr(out),
                                _ptr(lse), int(num_splits), _ptr(workspace), ctypes.c_size_t(workspace.numel()),
                                _stream(stream))
    del keep
    if st != OK:
        raise AttnError(st, "attn_fwd_splitkv")
    return out, lse


def bwd(q, k, v, o, lse, do, *, causal=False, offset=0, seqlens_q=None, seqlens_k=None,
        dq=None, dk=None, dv=None, workspace=None, stream=None, cu_seqlens_q=None, cu_seqlens_k=None,
        max_seqlen_q=None, max_seqlen_k=None, keep_gs=False):
    """G_Q, G_K, G_V.  ``do`` must have the strides of ``o``; outputs are
    allocated contiguous unless given (then with the strides of q / k / v).
    ``keep_gs`` calls attn_bwd_gs (G_S kept in the workspace) instead of
    attn_bwd."""
    torch = _torch()
    nd = 3 if (cu_seqlens_q is not None or cu_seqlens_k is not None) else 4
    for name, t in (("q", q), ("k", k), ("v", v), ("o", o), ("do", do)):
        _check4(name, t, q.dtype, nd)
    if do.stride() != o.stride():
        raise ValueError("do must have the strides of o")
    if dq is None:
        dq = torch.empty_like(q, memory_format=torch.contiguous_format)
        if dq.stride() != q.stride():
            raise ValueError("q must be contiguous when dq is not given")
    if dk is None:
        dk = torch.empty_like(k)
        if dk.stride() != k.stride():
            raise ValueError("k must be contiguous when dk is not given")
    if dv is None:
        dv = torch.empty_like(v)
        if dv.stride() != v.stride():
            raise ValueError("v must be contiguous when dv is not given")
    prob = _problem_from(q, k, v, _strides(o), cu_seqlens_q, cu_seqlens_k, max_seqlen_q, max_seqlen_k)
    need = gs_workspace_size(prob) if keep_gs else workspace_size(prob)
    if workspace is None:
        workspace = torch.empty(max(need, 1), dtype=torch.uint8, device=q.device)
    mask, keep = make_mask(causal, offset, seqlens_q, seqlens_k)
    fn = lib().attn_bwd_gs if keep_gs else lib().attn_bwd
    st = fn(ctypes.byref(prob), ctypes.byref(mask), _ptr(q), _ptr(k), _ptr(v), _ptr(o),
            _ptr(lse), _ptr(do), _ptr(dq), _ptr(dk), _ptr(dv), _ptr(workspace),
            ctypes.c_size_t(workspace.numel()), _stream(stream))
    del keep
    if st != OK:
        raise AttnError(st, "attn_bwd_gs" if keep_gs else "attn_bwd")
    return dq, dk, dv


def bwd_noalloc(q, k, v, o, lse, do, *, causal=False, offset=0, seqlens_q=None, seqlens_k=None,
                dq, dk, dv, stream=None, cu_seqlens_q=None, cu_seqlens_k=None, max_seqlen_q=None,
                max_seqlen_k=None):
    """attn_bwd_noalloc: the backward with the library's fixed device
    workspace; the caller passes every output (nothing is allocated)."""
    nd = 3 if (cu_seqlens_q is not None or cu_seqlens_k is not None) else 4
    for name, t in (("q", q), ("k", k), ("v", v), ("o", o), ("do", do), ("dq", dq), ("dk", dk), ("dv", dv)):
        _check4(name, t, q.dtype, nd)
    if do.stride() != o.stride() or dq.stride() != q.stride() or dk.stride() != k.stride() \
            or dv.stride() != v.stride():
        raise ValueError("do, dq, dk, dv must have the strides of o, q, k, v")
    prob = _problem_from(q, k, v, _strides(o), cu_seqlens_q, cu_seqlens_k, max_seqlen_q, max_seqlen_k)
    mask, keep = make_mask(causal, offset, seqlens_q, seqlens_k)
    st = lib().attn_bwd_noalloc(ctypes.byref(prob), ctypes.byref(mask), _ptr(q), _ptr(k), _ptr(v), _ptr(o),
                                _ptr(lse), _ptr(do), _ptr(dq), _ptr(dk), _ptr(dv), _stream(stream))
    del keep
    if st != OK:
        raise AttnError(st, "attn_bwd_noalloc")
    return dq, dk, dv


NOALLOC_MAX_WORKSPACE = 64 << 20  # ATTN_BWD_NOALLOC_MAX_WORKSPACE


class StagedBackward:
    """The backward's ABI passes bound to fixed tensors, for callers that
    time or schedule them separately: dq() then dkdv() equals one bwd();
    gs_stage(0), (1), (2) equals one bwd(keep_gs=True)."""

    def __init__(self, q, k, v, o, lse, do, dq, dk, dv, workspace, *, causal=False, offset=0,
                 seqlens_q=None, seqlens_k=None, cu_seqlens_q=None, cu_seqlens_k=None,
                 max_seqlen_q=None, max_seqlen_k=None):
        nd = 3 if (cu_seqlens_q is not None or cu_seqlens_k is not None) else 4
        for name, t in (("q", q), ("k", k), ("v", v), ("o", o), ("do", do), ("dq", dq),
                        ("dk", dk), ("dv", dv)):
            _check4(name, t, q.dtype, nd)
        if do.stride() != o.stride() or dq.stride() != q.stride() or dk.stride() != k.stride() \
                or dv.stride() != v.stride():
            raise ValueError("gradient strides must match their tensors")
        self.prob = _problem_from(q, k, v, _strides(o), cu_seqlens_q, cu_seqlens_k, max_seqlen_q,
                                  max_seqlen_k)
        self.mask, self._keep = make_mask(causal, offset, seqlens_q, seqlens_k)
        self.t = (q, k, v, o, lse, do, dq, dk, dv, workspace)
        self.ws = _ptr(workspace)
        self.ws_bytes = ctypes.c_size_t(workspace.numel())

    def _check(self, st, what):
        if st != OK:
            raise AttnError(st, what)

    def dq(self, stream=None):
        q, k, v, o, lse, do, dq, dk, dv, ws = self.t
        self._check(lib().attn_bwd_dq(ctypes.byref(self.prob), ctypes.byref(self.mask), _ptr(q), _ptr(k),
                                      _ptr(v), _ptr(o), _ptr(lse), _ptr(do), _ptr(dq), self.ws,
                                      self.ws_bytes, _stream(stream)), "attn_bwd_dq")

    def dkdv(self, stream=None):
        q, k, v, o, lse, do, dq, dk, dv, ws = self.t
        self._check(lib().attn_bwd_dkdv(ctypes.byref(self.prob), ctypes.byref(self.mask), _ptr(q),
                                        _ptr(k), _ptr(v), _ptr(lse), _ptr(do), _ptr(dk), _ptr(dv),
                                        self.ws, self.ws_bytes, _stream(stream)), "attn_bwd_dkdv")

    def gs_stage(self, stage, stream=None):
        """Stage 0, 1 or 2 of attn_bwd_gs (the workspace must hold
        gs_workspace_size bytes)."""
        q, k, v, o, lse, do, dq, dk, dv, ws = self.t
        self._check(lib().attn_bwd_gs_stage(ctypes.byref(self.prob), ctypes.byref(self.mask), _ptr(q), _ptr(k),
                                            _ptr(v), _ptr(o), _ptr(lse), _ptr(do), _ptr(dq), _ptr(dk), _ptr(dv),
                                            self.ws, self.ws_bytes, ctypes.c_int32(stage), _stream(stream)),
                    "attn_bwd_gs_stage")


# ---------------------------------------------------------------------------
# rotary positions
# ---------------------------------------------------------------------------
def make_rope(cos_sin, n_pos: Optional[int] = None) -> Rope:
    """cos_sin: contiguous float32 GPU tensor [n_pos, d_h / 2, 2] of (cos, sin),
    or an integer device address with n_pos given (host-side checks only)."""
    if isinstance(cos_sin, int) or cos_sin is None:
        return Rope(ctypes.c_void_p(cos_sin or 0), int(n_pos or 0), 0)
    torch = _torch()
    if cos_sin.dtype != torch.float32 or not cos_sin.is_contiguous() or cos_sin.dim() != 3 \
            or cos_sin.shape[-1] != 2:
        raise ValueError("cos_sin must be a contiguous float32 [n_pos, d_h/2, 2] tensor")
    return Rope(ctypes.c_void_p(cos_sin.data_ptr()), int(cos_sin.shape[0]), 0)


def rope_workspace_size(prob: Problem, backward: bool) -> int:
    fn = lib().attn_bwd_rope_workspace_size if backward else lib().attn_fwd_rope_workspace_size
    return int(fn(ctypes.byref(prob)))


def rope_apply(q, k, v, cos_sin, *, operand="q", inverse=False, out=None, causal=False, offset=0,
               seqlens_q=None, seqlens_k=None, stream=None, cu_seqlens_q=None, cu_seqlens_k=None,
               max_seqlen_q=None, max_seqlen_k=None):
    """attn_rope_apply: q or k (operand "q" / "k") turned by its positions
    (inverse: turned back).  ``out`` (default: a new tensor) must have the
    strides of the input; it may be the input itself."""
    torch = _torch()
    nd = 3 if (cu_seqlens_q is not None or cu_seqlens_k is not None) else 4
    for name, t in (("q", q), ("k", k), ("v", v)):
        _check4(name, t, q.dtype, nd)
    x = q if operand == "q" else k
    if out is None:
        out = torch.empty_like(x)
    if out.stride() != x.stride() or out.shape != x.shape:
        raise ValueError("out must have the shape and strides of the input")
    prob = _problem_from(q, k, v, None, cu_seqlens_q, cu_seqlens_k, max_seqlen_q, max_seqlen_k)
    mask, keep = make_mask(causal, offset, seqlens_q, seqlens_k)
    rope = make_rope(cos_sin)
    st = lib().attn_rope_apply(ctypes.byref(prob), ctypes.byref(mask), ctypes.byref(rope),
                               0 if operand == "q" else 1, 1 if inverse else 0, _ptr(x), _ptr(out),
                               _stream(stream))
    del keep
    if st != OK:
        raise AttnError(st, "attn_rope_apply")
    return out


def fwd_rope(q, k, v, cos_sin, *, causal=False, offset=0, seqlens_q=None, seqlens_k=None, out=None,
             lse=None, workspace=None, stream=None, cu_seqlens_q=None, cu_seqlens_k=None,
             max_seqlen_q=None, max_seqlen_k=None):
    """attn_fwd_rope: O and lse of attention on the rotated q and k."""
    torch = _torch()
    packed = cu_seqlens_q is not None or cu_seqlens_k is not None
    nd = 3 if packed else 4
    for name, t in (("q", q), ("k", k), ("v", v)):
        _check4(name, t, q.dtype, nd)
    d_v = v.shape[-1]
    if packed:
        total_q, H_q, _ = q.shape
        o_shape, lse_shape = (total_q, H_q, d_v), (H_q, total_q)
    else:
        B, H_q, n_q, _ = q.shape
        o_shape, lse_shape = (B, H_q, n_q, d_v), (B, H_q, n_q)
    if out is None:
        out = torch.empty(*o_shape, dtype=q.dtype, device=q.device)
    if lse is None:
        lse = torch.empty(*lse_shape, dtype=torch.float32, device=q.device)
    _check4("out", out, q.dtype, nd)
    if not lse.is_contiguous() or lse.dtype != torch.float32 or tuple(lse.shape) != lse_shape:
        raise ValueError(f"lse must be contiguous float32 of shape {lse_shape}")
    prob = _problem_from(q, k, v, _strides(out), cu_seqlens_q, cu_seqlens_k, max_seqlen_q, max_seqlen_k)
    need = rope_workspace_size(prob, backward=False)
    if workspace is None:
        workspace = torch.empty(max(need, 1), dtype=torch.uint8, device=q.device)
    mask, keep = make_mask(causal, offset, seqlens_q, seqlens_k)
    rope = make_rope(cos_sin)
    st = lib().attn_fwd_rope(ctypes.byref(prob), ctypes.byref(mask), ctypes.byref(rope), _ptr(q), _ptr(k),
                             _ptr(v), _ptr(out), _ptr(lse), _ptr(workspace), ctypes.c_size_t(workspace.numel()),
                             _stream(stream))
    del keep
    if st != OK:
        raise AttnError(st, "attn_fwd_rope")
    return out, lse


def bwd_rope(q, k, v, o, lse, do, cos_sin, *, causal=False, offset=0, seqlens_q=None, seqlens_k=None,
             dq=None, dk=None, dv=None, workspace=None, stream=None, cu_seqlens_q=None, cu_seqlens_k=None,
             max_seqlen_q=None, max_seqlen_k=None):
    """attn_bwd_rope: G_Q, G_K (turned back to the unrotated inputs) and G_V."""
    torch = _torch()
    nd = 3 if (cu_seqlens_q is not None or cu_seqlens_k is not None) else 4
    for name, t in (("q", q), ("k", k), ("v", v), ("o", o), ("do", do)):
        _check4(name, t, q.dtype, nd)
    if do.stride() != o.stride():
        raise ValueError("do must have the strides of o")
    dq = torch.empty_like(q) if dq is None else dq
    dk = torch.empty_like(k) if dk is None else dk
    dv = torch.empty_like(v) if dv is None else dv
    if dq.stride() != q.stride() or dk.stride() != k.stride() or dv.stride() != v.stride():
        raise ValueError("gradient strides must match their tensors")
    prob = _problem_from(q, k, v, _strides(o), cu_seqlens_q, cu_seqlens_k, max_seqlen_q, max_seqlen_k)
    need = rope_workspace_size(prob, backward=True)
    if workspace is None:
        workspace = torch.empty(max(need, 1), dtype=torch.uint8, device=q.device)
    mask, keep = make_mask(causal, offset, seqlens_q, seqlens_k)
    rope = make_rope(cos_sin)
    st = lib().attn_bwd_rope(ctypes.byref(prob), ctypes.byref(mask), ctypes.byref(rope), _ptr(q), _ptr(k),
                             _ptr(v), _ptr(o), _ptr(lse), _ptr(do), _ptr(dq), _ptr(dk), _ptr(dv),
                             _ptr(workspace), ctypes.c_size_t(workspace.numel()), _stream(stream))
    del keep
    if st != OK:
        raise AttnError(st, "attn_bwd_rope")
    return dq, dk, dv


# ---------------------------------------------------------------------------
# projections
# ---------------------------------------------------------------------------
class GemmContext:
    """A caller-owned GEMM context (attn_gemm_create) for the projection
    calls, bound to the device current when it is made; destroyed by close()
    or when collected."""

    def __init__(self):
        h = ctypes.c_void_p()
        st = lib().attn_gemm_create(ctypes.byref(h))
        if st != OK:
            raise AttnError(st, "attn_gemm_create")
        self.handle = h

    def close(self):
        if self.handle is not None and self.handle.value:
            lib().attn_gemm_destroy(self.handle)
        self.handle = None

    def __del__(self):
        try:
            self.close()
        except Exception:  # interpreter shutdown
            pass


_DEFAULT_GEMM = {}


def gemm_context(device=None) -> GemmContext:
    """This process's default context for `device` (the current one when
    None), made on first use: the caller side, not the library, keeps it."""
    torch = _torch()
    dev = torch.cuda.current_device() if device is None else int(device)
    ctx = _DEFAULT_GEMM.get(dev)
    if ctx is None:
        with torch.cuda.device(dev):
            ctx = GemmContext()
        _DEFAULT_GEMM[dev] = ctx
    return ctx


def _gemm_of(ctx, t):
    return (ctx if ctx is not None else gemm_context(t.device.index)).handle


def _check2(name, t, dtype):
    if t.dim() != 2 or t.dtype != dtype or not t.is_cuda or (t.shape[1] > 0 and t.stride(1) != 1):
        raise ValueError(f"{name} must be a 2-D GPU tensor of {dtype} with unit column stride")


def make_linear(rows, d_in, d_out, dtype, ld_x=None, ld_w=None, ld_y=None) -> Linear:
    return Linear(int(rows), int(d_in), int(d_out), int(dtype), int(ld_x if ld_x is not None else d_in),
                  int(ld_w if ld_w is not None else d_out), int(ld_y if ld_y is not None else d_out))


def _linear_of(x, w, y_stride0=None) -> Linear:
    return make_linear(x.shape[0], x.shape[1], w.shape[1], _dtype_code(x), x.stride(0), w.stride(0),
                       y_stride0 if y_stride0 is not None else w.shape[1])


def linear_fwd(x, w, *, out=None, stream=None, gemm=None):
    """attn_linear_fwd: Y = X W for 2-D x [rows, d_in], w [d_in, d_out].
    gemm: a GemmContext (default: gemm_context() of x's device)."""
    torch = _torch()
    _check2("x", x, x.dtype)
    _check2("w", w, x.dtype)
    if out is None:
        out = torch.empty(x.shape[0], w.shape[1], dtype=x.dtype, device=x.device)
    _check2("out", out, x.dtype)
    lin = _linear_of(x, w, out.stride(0))
    st = lib().attn_linear_fwd(ctypes.byref(lin), _gemm_of(gemm, x), _ptr(x), _ptr(w), _ptr(out), _stream(stream))
    if st != OK:
        raise AttnError(st, "attn_linear_fwd")
    return out


def linear_bwd(x, w, gy, *, gx=None, gw=None, accumulate=False, want_gx=True, want_gw=True, stream=None,
               gemm=None):
    """attn_linear_bwd: G_X = G_Y W^T and G_W = X^T G_Y (accumulate: added)."""
    torch = _torch()
    for n_, t in (("x", x), ("w", w), ("gy", gy)):
        _check2(n_, t, x.dtype)
    if want_gx and gx is None:
        gx = torch.empty_like(x)
    if want_gw and gw is None:
        gw = torch.empty_like(w)
    if gx is not None and gx.stride() != x.stride():
        raise ValueError("gx must have the strides of x")
    if gw is not None and gw.stride() != w.stride():
        raise ValueError("gw must have the strides of w")
    lin = _linear_of(x, w, gy.stride(0))
    st = lib().attn_linear_bwd(ctypes.byref(lin), _gemm_of(gemm, x), _ptr(x), _ptr(w), _ptr(gy),
                               _ptr(gx) if gx is not None else None,
                               _ptr(gw) if gw is not None else None, 1 if accumulate else 0, _stream(stream))
    if st != OK:
        raise AttnError(st, "attn_linear_bwd")
    return gx, gw


def _self_problem(x, w, H_q, H_kv, d_h, d_v, o_stride, cu_seqlens, max_seqlen):
    if cu_seqlens is None:
        B, n, _ = x.shape
        return make_problem(B, H_q, H_kv, n, n, d_h, d_v, _dtype_code(x), o_stride=o_stride)
    cu, lens = _packed_lengths(cu_seqlens)
    n = int(max_seqlen) if max_seqlen is not None else max(lens, default=0)
    # the q/k/v strides are the column blocks of qkv, set by the library
    return make_problem(len(cu) - 1, H_q, H_kv, n, n, d_h, d_v, _dtype_code(x), None, None, None, o_stride, cu, cu)


def self_attention_fwd(x, w_qkv, *, H_q, H_kv, d_h, d_v, causal=False, offset=0, seqlens_q=None, seqlens_k=None,
                       qkv=None, out=None, lse=None, stream=None, cu_seqlens=None, max_seqlen=None, gemm=None):
    """attn_self_attention_fwd: x [B, n, d_model] (or packed [rows, d_model]
    with cu_seqlens), w_qkv [d_model, H_q d_h + H_kv d_h + H_kv d_v].
    Returns qkv [rows, C], O and lse (shapes as fwd())."""
    torch = _torch()
    packed = cu_seqlens is not None
    if x.dim() != (2 if packed else 3) or not x.is_contiguous() or not w_qkv.is_contiguous():
        raise ValueError("x ([B, n, d_model] or packed [rows, d_model]) and w_qkv must be contiguous")
    rows = x.shape[0] if packed else x.shape[0] * x.shape[1]
    C = H_q * d_h + H_kv * d_h + H_kv * d_v
    if qkv is None:
        qkv = torch.empty(rows, C, dtype=x.dtype, device=x.device)
    if packed:
        o_shape, lse_shape = (rows, H_q, d_v), (H_q, rows)
    else:
        o_shape, lse_shape = (x.shape[0], H_q, x.shape[1], d_v), (x.shape[0], H_q, x.shape[1])
    if out is None:
        out = torch.empty(*o_shape, dtype=x.dtype, device=x.device)
    if lse is None:
        lse = torch.empty(*lse_shape, dtype=torch.float32, device=x.device)
    prob = _self_problem(x, w_qkv, H_q, H_kv, d_h, d_v, _strides(out), cu_seqlens, max_seqlen)
    mask, keep = make_mask(causal, offset, seqlens_q, seqlens_k)
    st = lib().attn_self_attention_fwd(ctypes.byref(prob), ctypes.byref(mask), _gemm_of(gemm, x), int(x.shape[-1]),
                                       _ptr(x),
                                       _ptr(w_qkv), _ptr(qkv), _ptr(out), _ptr(lse), _stream(stream))
    del keep
    if st != OK:
        raise AttnError(st, "attn_self_attention_fwd")
    return qkv, out, lse


def self_attention_bwd(x, w_qkv, qkv, o, lse, do, *, H_q, H_kv, d_h, d_v, causal=False, offset=0, seqlens_q=None,
                       seqlens_k=None, gx=None, gw=None, workspace=None, stream=None, cu_seqlens=None,
                       max_seqlen=None, gemm=None):
    """attn_self_attention_bwd: G_X (shape of x) and G_W (shape of w_qkv)."""
    torch = _torch()
    if do.stride() != o.stride():
        raise ValueError("do must have the strides of o")
    gx = torch.empty_like(x) if gx is None else gx
    gw = torch.empty_like(w_qkv) if gw is None else gw
    prob = _self_problem(x, w_qkv, H_q, H_kv, d_h, d_v, _strides(o), cu_seqlens, max_seqlen)
    need = int(lib().attn_self_attention_bwd_workspace_size(ctypes.byref(prob)))
    if workspace is None:
        workspace = torch.empty(max(need, 1), dtype=torch.uint8, device=x.device)
    mask, keep = make_mask(causal, offset, seqlens_q, seqlens_k)
    st = lib().attn_self_attention_bwd(ctypes.byref(prob), ctypes.byref(mask), _gemm_of(gemm, x), int(x.shape[-1]),
                                       _ptr(x),
                                       _ptr(w_qkv), _ptr(qkv), _ptr(o), _ptr(lse), _ptr(do), _ptr(gx), _ptr(gw),
                                       _ptr(workspace), ctypes.c_size_t(workspace.numel()), _stream(stream))
    del keep
    if st != OK:
        raise AttnError(st, "attn_self_attention_bwd")
    return gx, gw


def self_attention_workspace_size(prob: Problem) -> int:
    return int(lib().attn_self_attention_bwd_workspace_size(ctypes.byref(prob)))
