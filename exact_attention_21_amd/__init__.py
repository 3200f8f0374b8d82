"""Python binding of the gfx950 fused-attention library (libfa.so).

Argument marshalling only: tensors are checked for device, dtype, shape and
contiguity, their data pointers and torch's current HIP stream are handed to
the C ABI declared in include/fa.h, and every step of the computation runs in
the library's kernels.  There is no fallback: if libfa.so is missing or the
device is not gfx950 the calls raise.

Names mirror the C ABI: fa_fwd, fa_bwd (and its stages fa_bwd_preprocess,
fa_bwd_dkdv, fa_bwd_dq, fa_bwd_dq_preprocess), fa_bwd_noalloc, fa_fwd_padded, fa_bwd_padded, fa_fwd_dropout,
fa_bwd_dropout, fa_fwd_splitkv, fa_fwd_splitkv_workspace_size,
fa_bwd_workspace_size, fa_fwd_plan, fa_bwd_plan, fa_status_str.
fwd(), bwd(), fwd_padded(), bwd_padded(), fwd_dropout(), bwd_dropout() and
fwd_splitkv() are conveniences that allocate the outputs (and workspaces) with
torch and call the corresponding entry point.
"""
from __future__ import annotations

import ctypes
import math
import os

_PKG = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_PKG, "libfa.so")

FA_F16, FA_BF16 = 0, 1
_lib = None


class FaError(RuntimeError):
    def __init__(self, fn: str, status: int):
        super().__init__(f"{fn} failed with status {status}: {fa_status_str(status)}")
        self.status = status


class fa_plan_t(ctypes.Structure):
    _fields_ = [("block_m", ctypes.c_int), ("block_n", ctypes.c_int), ("threads", ctypes.c_int),
                ("grid", ctypes.c_int), ("lds_bytes", ctypes.c_int), ("xcd_grouped", ctypes.c_int)]


def lib() -> ctypes.CDLL:
    """Load libfa.so (built by exact_attention_21_amd.build); raises if absent."""
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            raise ImportError(f"{LIB_PATH} is missing: build it with `python -m exact_attention_21_amd.build`")
        L = ctypes.CDLL(LIB_PATH)
        vp, I, F, Z = ctypes.c_void_p, ctypes.c_int, ctypes.c_float, ctypes.c_size_t
        L.fa_fwd.argtypes = [vp, vp, vp, vp, vp, I, I, I, I, F, I, I, vp]
        L.fa_fwd.restype = I
        L.fa_bwd.argtypes = [vp, vp, vp, vp, vp, vp, vp, vp, vp, I, I, I, I, F, I, I, vp, Z, vp]
        L.fa_bwd.restype = I
        L.fa_bwd_preprocess.argtypes = [vp, vp, vp, I, I, I, I, I, vp, Z, vp]
        L.fa_bwd_preprocess.restype = I
        L.fa_bwd_dkdv.argtypes = [vp, vp, vp, vp, vp, vp, I, I, I, I, F, I, I, vp, Z, vp]
        L.fa_bwd_dkdv.restype = I
        L.fa_bwd_dq.argtypes = [vp, vp, vp, vp, vp, I, I, I, I, F, I, I, vp, Z, vp]
        L.fa_bwd_dq.restype = I
        L.fa_bwd_dq_preprocess.argtypes = [vp, vp, vp, vp, vp, vp, vp, I, I, I, I, F, I, I, vp, Z, vp]
        L.fa_bwd_dq_preprocess.restype = I
        L.fa_fwd_padded.argtypes = [vp, vp, vp, vp, vp, vp, vp, I, I, I, I, I, F, I, I, vp]
        L.fa_fwd_padded.restype = I
        L.fa_bwd_noalloc.argtypes = [vp, vp, vp, vp, vp, vp, vp, vp, vp, I, I, I, I, F, I, I, vp]
        L.fa_bwd_noalloc.restype = I
        L.fa_bwd_padded.argtypes = [vp, vp, vp, vp, vp, vp, vp, vp, vp, vp, vp, I, I, I, I, I, F, I, I,
                                    vp, Z, vp]
        L.fa_bwd_padded.restype = I
        U64, U32 = ctypes.c_uint64, ctypes.c_uint32
        L.fa_fwd_dropout.argtypes = [vp, vp, vp, vp, vp, vp, vp, I, I, I, I, I, F, I, F, U64, U32, I, vp]
        L.fa_fwd_dropout.restype = I
        L.fa_bwd_dropout.argtypes = [vp, vp, vp, vp, vp, vp, vp, vp, vp, vp, vp, I, I, I, I, I, F, I, F,
                                     U64, U32, I, vp, Z, vp]
        L.fa_bwd_dropout.restype = I
        L.fa_fwd_splitkv.argtypes = [vp, vp, vp, vp, vp, vp, vp, I, I, I, I, I, F, I, I, vp, Z, vp]
        L.fa_fwd_splitkv.restype = I
        L.fa_fwd_splitkv_workspace_size.argtypes = [I, I, I, I, I]
        L.fa_fwd_splitkv_workspace_size.restype = Z
        L.fa_bwd_workspace_size.argtypes = [I, I, I, I]
        L.fa_bwd_workspace_size.restype = Z
        L.fa_fwd_plan.argtypes = [I, I, I, I, I, I, ctypes.POINTER(fa_plan_t)]
        L.fa_fwd_plan.restype = I
        L.fa_bwd_plan.argtypes = [I, I, I, I, I, I, ctypes.POINTER(fa_plan_t)]
        L.fa_bwd_plan.restype = I
        L.fa_status_str.argtypes = [I]
        L.fa_status_str.restype = ctypes.c_char_p
        _lib = L
    return _lib


def fa_status_str(status: int) -> str:
    return lib().fa_status_str(int(status)).decode()


def _dtype_code(t) -> int:
    import torch
    if t.dtype == torch.float16:
        return FA_F16
    if t.dtype == torch.bfloat16:
        return FA_BF16
    raise TypeError(f"only float16 / bfloat16 tensors are supported, got {t.dtype}")


def _check_qkv_like(name, t, ref):
    """t is a contiguous GPU tensor with ref's device, dtype and shape (checked
    before any pointer reaches the library: a host pointer handed to a kernel
    would fault the GPU instead of raising)."""
    if not t.is_cuda:
        raise ValueError(f"{name} must be a GPU tensor")
    if t.device != ref.device or t.dtype != ref.dtype or t.shape != ref.shape:
        raise ValueError(f"{name} must match q in device, dtype and shape")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous [B, H, N, d]")


def _check_lse(lse, shape, ref):
    """lse is a contiguous float32 GPU tensor of the given shape on ref's device."""
    import torch
    if not lse.is_cuda or lse.device != ref.device:
        raise ValueError("lse must be a GPU tensor on q's device")
    if lse.dtype != torch.float32 or tuple(lse.shape) != tuple(shape) or not lse.is_contiguous():
        raise ValueError(f"lse must be contiguous float32 {list(shape)}")


def _stream(stream):
    import torch
    if stream is None:
        return ctypes.c_void_p(torch.cuda.current_stream().cuda_stream)
    if isinstance(stream, int):
        return ctypes.c_void_p(stream)
    return ctypes.c_void_p(stream.cuda_stream)


def _ptr(t):
    return ctypes.c_void_p(t.data_ptr())


def default_scale(d: int) -> float:
    return 1.0 / math.sqrt(d)


def fa_fwd_plan(B, H, N, d, causal, dtype) -> fa_plan_t:
    plan = fa_plan_t()
    rc = lib().fa_fwd_plan(B, H, N, d, int(causal), int(dtype), ctypes.byref(plan))
    if rc:
        raise FaError("fa_fwd_plan", rc)
    return plan


def fa_bwd_plan(B, H, N, d, causal, dtype) -> fa_plan_t:
    plan = fa_plan_t()
    rc = lib().fa_bwd_plan(B, H, N, d, int(causal), int(dtype), ctypes.byref(plan))
    if rc:
        raise FaError("fa_bwd_plan", rc)
    return plan


def fa_bwd_workspace_size(B, H, N, d) -> int:
    return int(lib().fa_bwd_workspace_size(B, H, N, d))


def fa_fwd(q, k, v, o, lse, scale: float, causal: bool, stream=None) -> None:
    """Forward into caller-provided o ([B,H,N,d], q's dtype) and lse ([B,H,N] fp32)."""
    import torch
    if q.dim() != 4:
        raise ValueError("q must be [B, H, N, d]")
    B, H, N, d = q.shape
    for name, t in (("q", q), ("k", k), ("v", v), ("o", o)):
        _check_qkv_like(name, t, q)
    _check_lse(lse, (B, H, N), q)
    rc = lib().fa_fwd(_ptr(q), _ptr(k), _ptr(v), _ptr(o), _ptr(lse), B, H, N, d, float(scale),
                      int(bool(causal)), _dtype_code(q), _stream(stream))
    if rc:
        raise FaError("fa_fwd", rc)


def fa_bwd(q, k, v, o, dout, lse, dq, dk, dv, scale: float, causal: bool, workspace,
           stream=None) -> None:
    """Backward into caller-provided dq, dk, dv; workspace is a uint8 device tensor."""
    import torch
    B, H, N, d = q.shape
    for name, t in (("k", k), ("v", v), ("o", o), ("dout", dout), ("dq", dq), ("dk", dk), ("dv", dv)):
        _check_qkv_like(name, t, q)
    _check_lse(lse, (B, H, N), q)
    rc = lib().fa_bwd(_ptr(q), _ptr(k), _ptr(v), _ptr(o), _ptr(dout), _ptr(lse), _ptr(dq), _ptr(dk),
                      _ptr(dv), B, H, N, d, float(scale), int(bool(causal)), _dtype_code(q),
                      *_ws(workspace, q), _stream(stream))
    if rc:
        raise FaError("fa_bwd", rc)


FA_BWD_NOALLOC_MAX_ROWS = 4194304  # include/fa.h


def fa_bwd_noalloc(q, k, v, o, dout, lse, dq, dk, dv, scale: float, causal: bool,
                   stream=None) -> None:
    """fa_bwd without a workspace: the row statistics live in the library's static
    per-GPU scratch (B*H*N <= FA_BWD_NOALLOC_MAX_ROWS).  Allocates nothing; calls
    that overlap on one GPU race (see include/fa.h)."""
    B, H, N, d = q.shape
    for name, t in (("q", q), ("k", k), ("v", v), ("o", o), ("dout", dout), ("dq", dq), ("dk", dk),
                    ("dv", dv)):
        _check_qkv_like(name, t, q)
    _check_lse(lse, (B, H, N), q)
    rc = lib().fa_bwd_noalloc(_ptr(q), _ptr(k), _ptr(v), _ptr(o), _ptr(dout), _ptr(lse), _ptr(dq),
                              _ptr(dk), _ptr(dv), B, H, N, d, float(scale), int(bool(causal)),
                              _dtype_code(q), _stream(stream))
    if rc:
        raise FaError("fa_bwd_noalloc", rc)


def _ws(workspace, q):
    if not workspace.is_cuda or not workspace.is_contiguous() or workspace.device != q.device:
        raise ValueError("workspace must be a contiguous GPU tensor on q's device")
    return _ptr(workspace), ctypes.c_size_t(workspace.numel() * workspace.element_size())


def fa_bwd_preprocess(o, dout, lse, workspace, stream=None) -> None:
    """Stage 1 of fa_bwd: D = rowsum(dO * O) and LSE * log2(e) into the workspace."""
    import torch
    B, H, N, d = o.shape
    _check_qkv_like("o", o, o)
    _check_qkv_like("dout", dout, o)
    _check_lse(lse, (B, H, N), o)
    rc = lib().fa_bwd_preprocess(_ptr(o), _ptr(dout), _ptr(lse), B, H, N, d, _dtype_code(o),
                                 *_ws(workspace, o), _stream(stream))
    if rc:
        raise FaError("fa_bwd_preprocess", rc)


def fa_bwd_dkdv(q, k, v, dout, dk, dv, scale: float, causal: bool, workspace, stream=None) -> None:
    """Stage 2 of fa_bwd: dK and dV (needs the preprocessed workspace)."""
    B, H, N, d = q.shape
    for name, t in (("k", k), ("v", v), ("dout", dout), ("dk", dk), ("dv", dv)):
        _check_qkv_like(name, t, q)
    rc = lib().fa_bwd_dkdv(_ptr(q), _ptr(k), _ptr(v), _ptr(dout), _ptr(dk), _ptr(dv), B, H, N, d,
                           float(scale), int(bool(causal)), _dtype_code(q), *_ws(workspace, q),
                           _stream(stream))
    if rc:
        raise FaError("fa_bwd_dkdv", rc)


def fa_bwd_dq(q, k, v, dout, dq, scale: float, causal: bool, workspace, stream=None) -> None:
    """Stage 3 of fa_bwd: dQ (needs the preprocessed workspace)."""
    B, H, N, d = q.shape
    for name, t in (("k", k), ("v", v), ("dout", dout), ("dq", dq)):
        _check_qkv_like(name, t, q)
    rc = lib().fa_bwd_dq(_ptr(q), _ptr(k), _ptr(v), _ptr(dout), _ptr(dq), B, H, N, d,
                         float(scale), int(bool(causal)), _dtype_code(q), *_ws(workspace, q),
                         _stream(stream))
    if rc:
        raise FaError("fa_bwd_dq", rc)


def fa_bwd_dq_preprocess(q, k, v, o, dout, lse, dq, scale: float, causal: bool, workspace,
                         stream=None) -> None:
    """fa_bwd_dq that also writes the row statistics fa_bwd_dkdv reads (no preprocessed workspace needed)."""
    import torch
    B, H, N, d = q.shape
    for name, t in (("k", k), ("v", v), ("o", o), ("dout", dout), ("dq", dq)):
        _check_qkv_like(name, t, q)
    _check_lse(lse, (B, H, N), q)
    rc = lib().fa_bwd_dq_preprocess(_ptr(q), _ptr(k), _ptr(v), _ptr(o), _ptr(dout), _ptr(lse), _ptr(dq),
                                    B, H, N, d, float(scale), int(bool(causal)), _dtype_code(q),
                                    *_ws(workspace, q), _stream(stream))
    if rc:
        raise FaError("fa_bwd_dq_preprocess", rc)


def fwd(q, k, v, causal: bool = False, scale: float | None = None):
    """Returns (o, lse) for q, k, v of shape [B, H, N, d]."""
    import torch
    B, H, N, d = q.shape
    o = torch.empty_like(q)
    lse = torch.empty((B, H, N), dtype=torch.float32, device=q.device)
    fa_fwd(q, k, v, o, lse, default_scale(d) if scale is None else scale, causal)
    return o, lse


def bwd(q, k, v, o, dout, lse, causal: bool = False, scale: float | None = None, workspace=None):
    """Returns (dq, dk, dv); o and lse are the forward's outputs."""
    import torch
    B, H, N, d = q.shape
    dq, dk, dv = torch.empty_like(q), torch.empty_like(q), torch.empty_like(q)
    if workspace is None:
        workspace = torch.empty(fa_bwd_workspace_size(B, H, N, d), dtype=torch.uint8, device=q.device)
    fa_bwd(q, k, v, o, dout, lse, dq, dk, dv, default_scale(d) if scale is None else scale, causal,
           workspace)
    return dq, dk, dv


def _lens_ptr(lens, B, device):
    """Device int32 [B] length array (or NULL)."""
    import torch
    if lens is None:
        return ctypes.c_void_p(None)
    if not (isinstance(lens, torch.Tensor) and lens.is_cuda and lens.dtype == torch.int32
            and lens.device == device and lens.is_contiguous() and tuple(lens.shape) == (B,)):
        raise ValueError("sequence lengths must be a contiguous int32 [B] tensor on q's device")
    return _ptr(lens)


def _check_padded(q, k, v):
    if q.dim() != 4 or k.dim() != 4:
        raise ValueError("q must be [B, H, Nq, d] and k, v [B, H, Nk, d]")
    B, H, Nq, d = q.shape
    Nk = k.shape[2]
    if not q.is_cuda:
        raise ValueError("q must be a GPU tensor")
    for name, t in (("k", k), ("v", v)):
        if not t.is_cuda or t.device != q.device or t.dtype != q.dtype or tuple(t.shape) != (B, H, Nk, d):
            raise ValueError(f"{name} must be [B, H, Nk, d] with q's device and dtype")
        if not t.is_contiguous():
            raise ValueError(f"{name} must be contiguous")
    if not q.is_contiguous():
        raise ValueError("q must be contiguous")
    return B, H, Nq, Nk, d


def fa_fwd_padded(q, k, v, o, lse, seqlens_q, seqlens_k, scale: float, causal: bool,
                  stream=None) -> None:
    """Forward over padded batches / cross-attention into caller-provided o and lse.
    seqlens_q, seqlens_k: device int32 [B] valid lengths, or None (all valid)."""
    import torch
    B, H, Nq, Nk, d = _check_padded(q, k, v)
    _check_qkv_like("o", o, q)
    _check_lse(lse, (B, H, Nq), q)
    rc = lib().fa_fwd_padded(_ptr(q), _ptr(k), _ptr(v), _ptr(o), _ptr(lse),
                             _lens_ptr(seqlens_q, B, q.device), _lens_ptr(seqlens_k, B, q.device),
                             B, H, Nq, Nk, d, float(scale), int(bool(causal)), _dtype_code(q),
                             _stream(stream))
    if rc:
        raise FaError("fa_fwd_padded", rc)


def fa_bwd_padded(q, k, v, o, dout, lse, dq, dk, dv, seqlens_q, seqlens_k, scale: float,
                  causal: bool, workspace, stream=None) -> None:
    """Backward of fa_fwd_padded into caller-provided dq, dk, dv."""
    import torch
    B, H, Nq, Nk, d = _check_padded(q, k, v)
    for name, t in (("o", o), ("dout", dout), ("dq", dq)):
        _check_qkv_like(name, t, q)
    for name, t in (("dk", dk), ("dv", dv)):
        _check_qkv_like(name, t, k)
    _check_lse(lse, (B, H, Nq), q)
    rc = lib().fa_bwd_padded(_ptr(q), _ptr(k), _ptr(v), _ptr(o), _ptr(dout), _ptr(lse), _ptr(dq),
                             _ptr(dk), _ptr(dv), _lens_ptr(seqlens_q, B, q.device),
                             _lens_ptr(seqlens_k, B, q.device), B, H, Nq, Nk, d, float(scale),
                             int(bool(causal)), _dtype_code(q), *_ws(workspace, q), _stream(stream))
    if rc:
        raise FaError("fa_bwd_padded", rc)


def fwd_padded(q, k, v, seqlens_q=None, seqlens_k=None, causal: bool = False,
               scale: float | None = None):
    """Returns (o, lse) for q [B, H, Nq, d], k, v [B, H, Nk, d] and per-batch valid lengths."""
    import torch
    B, H, Nq, d = q.shape
    o = torch.empty_like(q)
    lse = torch.empty((B, H, Nq), dtype=torch.float32, device=q.device)
    fa_fwd_padded(q, k, v, o, lse, seqlens_q, seqlens_k, default_scale(d) if scale is None else scale,
                  causal)
    return o, lse


def bwd_padded(q, k, v, o, dout, lse, seqlens_q=None, seqlens_k=None, causal: bool = False,
               scale: float | None = None, workspace=None):
    """Returns (dq, dk, dv) of fwd_padded."""
    import torch
    B, H, Nq, d = q.shape
    dq, dk, dv = torch.empty_like(q), torch.empty_like(k), torch.empty_like(k)
    if workspace is None:
        workspace = torch.empty(fa_bwd_workspace_size(B, H, Nq, d), dtype=torch.uint8, device=q.device)
    fa_bwd_padded(q, k, v, o, dout, lse, dq, dk, dv, seqlens_q, seqlens_k,
                  default_scale(d) if scale is None else scale, causal, workspace)
    return dq, dk, dv


def dropout_threshold(p: float) -> int:
    """The 8-bit drop threshold the library uses for probability p: round(256 p)."""
    return int(round(float(p) * 256.0))


def fa_fwd_dropout(q, k, v, o, lse, seqlens_q, seqlens_k, scale: float, causal: bool,
                   dropout_p: float, seed: int, offset: int, stream=None) -> None:
    """fa_fwd_padded with dropout on the attention weights (see include/fa.h)."""
    import torch
    B, H, Nq, Nk, d = _check_padded(q, k, v)
    _check_qkv_like("o", o, q)
    _check_lse(lse, (B, H, Nq), q)
    rc = lib().fa_fwd_dropout(_ptr(q), _ptr(k), _ptr(v), _ptr(o), _ptr(lse),
                              _lens_ptr(seqlens_q, B, q.device), _lens_ptr(seqlens_k, B, q.device),
                              B, H, Nq, Nk, d, float(scale), int(bool(causal)), float(dropout_p),
                              int(seed) & ((1 << 64) - 1), int(offset) & 0xFFFFFFFF, _dtype_code(q),
                              _stream(stream))
    if rc:
        raise FaError("fa_fwd_dropout", rc)


def fa_bwd_dropout(q, k, v, o, dout, lse, dq, dk, dv, seqlens_q, seqlens_k, scale: float,
                   causal: bool, dropout_p: float, seed: int, offset: int, workspace,
                   stream=None) -> None:
    """Backward of fa_fwd_dropout (same dropout_p, seed and offset)."""
    import torch
    B, H, Nq, Nk, d = _check_padded(q, k, v)
    for name, t in (("o", o), ("dout", dout), ("dq", dq)):
        _check_qkv_like(name, t, q)
    for name, t in (("dk", dk), ("dv", dv)):
        _check_qkv_like(name, t, k)
    _check_lse(lse, (B, H, Nq), q)
    rc = lib().fa_bwd_dropout(_ptr(q), _ptr(k), _ptr(v), _ptr(o), _ptr(dout), _ptr(lse), _ptr(dq),
                              _ptr(dk), _ptr(dv), _lens_ptr(seqlens_q, B, q.device),
                              _lens_ptr(seqlens_k, B, q.device), B, H, Nq, Nk, d, float(scale),
                              int(bool(causal)), float(dropout_p), int(seed) & ((1 << 64) - 1),
                              int(offset) & 0xFFFFFFFF, _dtype_code(q), *_ws(workspace, q),
                              _stream(stream))
    if rc:
        raise FaError("fa_bwd_dropout", rc)


def fwd_dropout(q, k, v, dropout_p: float, seed: int, offset: int = 0, seqlens_q=None,
                seqlens_k=None, causal: bool = False, scale: float | None = None):
    """Returns (o, lse) with dropout on the attention weights."""
    import torch
    B, H, Nq, d = q.shape
    o = torch.empty_like(q)
    lse = torch.empty((B, H, Nq), dtype=torch.float32, device=q.device)
    fa_fwd_dropout(q, k, v, o, lse, seqlens_q, seqlens_k, default_scale(d) if scale is None else scale,
                   causal, dropout_p, seed, offset)
    return o, lse


def bwd_dropout(q, k, v, o, dout, lse, dropout_p: float, seed: int, offset: int = 0,
                seqlens_q=None, seqlens_k=None, causal: bool = False, scale: float | None = None,
                workspace=None):
    """Returns (dq, dk, dv) of fwd_dropout."""
    import torch
    B, H, Nq, d = q.shape
    dq, dk, dv = torch.empty_like(q), torch.empty_like(k), torch.empty_like(k)
    if workspace is None:
        workspace = torch.empty(fa_bwd_workspace_size(B, H, Nq, d), dtype=torch.uint8, device=q.device)
    fa_bwd_dropout(q, k, v, o, dout, lse, dq, dk, dv, seqlens_q, seqlens_k,
                   default_scale(d) if scale is None else scale, causal, dropout_p, seed, offset,
                   workspace)
    return dq, dk, dv


def fa_fwd_splitkv_workspace_size(B, H, Nq, Nk, d) -> int:
    return int(lib().fa_fwd_splitkv_workspace_size(B, H, Nq, Nk, d))


def fa_fwd_splitkv(q, k, v, o, lse, seqlens_q, seqlens_k, scale: float, causal: bool, workspace,
                   stream=None) -> None:
    """fa_fwd_padded's result computed split over key blocks (few queries, long K/V)."""
    import torch
    B, H, Nq, Nk, d = _check_padded(q, k, v)
    _check_qkv_like("o", o, q)
    _check_lse(lse, (B, H, Nq), q)
    rc = lib().fa_fwd_splitkv(_ptr(q), _ptr(k), _ptr(v), _ptr(o), _ptr(lse),
                              _lens_ptr(seqlens_q, B, q.device), _lens_ptr(seqlens_k, B, q.device),
                              B, H, Nq, Nk, d, float(scale), int(bool(causal)), _dtype_code(q),
                              *_ws(workspace, q), _stream(stream))
    if rc:
        raise FaError("fa_fwd_splitkv", rc)


def fwd_splitkv(q, k, v, seqlens_q=None, seqlens_k=None, causal: bool = False,
                scale: float | None = None, workspace=None):
    """Returns (o, lse) like fwd_padded, computed split over key blocks."""
    import torch
    B, H, Nq, d = q.shape
    Nk = k.shape[2]
    o = torch.empty_like(q)
    lse = torch.empty((B, H, Nq), dtype=torch.float32, device=q.device)
    if workspace is None:
        workspace = torch.empty(fa_fwd_splitkv_workspace_size(B, H, Nq, Nk, d), dtype=torch.uint8,
                                device=q.device)
    fa_fwd_splitkv(q, k, v, o, lse, seqlens_q, seqlens_k, default_scale(d) if scale is None else scale,
                   causal, workspace)
    return o, lse
