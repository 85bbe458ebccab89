"""MI355X-native IO-aware attention: fused attention forward, split-KV decode, backward, the
one-pass row softmax, and the fused GELU / bias-GELU-dropout elementwise chains.

A thin binding over the C ABI of ``include/fa.h`` (``libfa_mi355x.so``).  The functions carry the
same names as the C entry points and only marshal arguments: torch supplies device memory and the
current stream, every step of the computation runs in the library's HIP kernels.  There is no CPU
fallback; importing this package fails if the library has not been built.
"""
from __future__ import annotations

import math

import torch

from . import _lib
from ._lib import (FA_ERR_ALIGN, FA_ERR_CAUSAL_TQ_GT_TK, FA_ERR_HEAD_DIM, FA_ERR_HIP,  # noqa: F401
                   FA_ERR_NULL, FA_ERR_PROB, FA_ERR_SCALE, FA_ERR_SCRATCH, FA_ERR_SHAPE,
                   FA_ERR_SPLITS, FA_ERR_WORKSPACE, FA_NOALLOC_SCRATCH_BYTES, FA_OK, LIB_PATH)

__all__ = ["fa_fwd", "fa_fwd_o32", "fa_fwd_strided", "fa_validate_fwd_strided", "fa_decode", "fa_decode_noalloc", "fa_decode_workspace_size", "fa_decode_strided", "fa_validate_decode_strided", "fa_bwd",
           "fa_bwd_f32", "fa_bwd_workspace_size", "fa_validate_fwd", "fa_validate_decode",
           "fa_validate_bwd", "fa_bwd_strided", "fa_validate_bwd_strided", "fa_softmax_rows", "fa_validate_softmax", "fa_gelu_f32",
           "fa_gelu_bf16", "fa_bias_gelu_dropout_bf16", "fa_validate_gelu",
           "fa_validate_bias_gelu_dropout", "fa_status_str", "fa_last_hip_error", "FaError",
           "LIB_PATH"]


class FaError(RuntimeError):
    """A nonzero status returned by the library."""

    def __init__(self, status: int):
        self.status = status
        msg = fa_status_str(status)
        if status == FA_ERR_HIP:
            msg += f" (hipError_t {fa_last_hip_error()})"
        super().__init__(msg)


def fa_status_str(status: int) -> str:
    return _lib.lib.fa_status_str(int(status)).decode()


def fa_last_hip_error() -> int:
    return int(_lib.lib.fa_last_hip_error())


def fa_decode_workspace_size(B: int, h: int, d_head: int, num_splits: int) -> int:
    return int(_lib.lib.fa_decode_workspace_size(B, h, d_head, num_splits))


def fa_bwd_workspace_size(B: int, h: int, Tq: int) -> int:
    return int(_lib.lib.fa_bwd_workspace_size(B, h, Tq))


def _check_tensor(name, t, dtype, ndim):
    if not isinstance(t, torch.Tensor):
        raise TypeError(f"{name} must be a torch.Tensor")
    if t.device.type != "cuda":
        raise ValueError(f"{name} must be on a GPU device, got {t.device}")
    if t.dtype != dtype:
        raise ValueError(f"{name} must be {dtype}, got {t.dtype}")
    if t.dim() != ndim:
        raise ValueError(f"{name} must have {ndim} dimensions, got shape {tuple(t.shape)}")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous (the kernels read raw row-major memory)")


def _stream_handle(stream, device):
    s = torch.cuda.current_stream(device) if stream is None else stream
    return ctypes_void(s.cuda_stream)


def ctypes_void(x):
    import ctypes
    return ctypes.c_void_p(int(x))


def _default_scale(d):
    return 1.0 / math.sqrt(d)


def _fwd(entry, out_dtype, q, k, v, causal, scale, o, lse, stream):
    _check_tensor("q", q, torch.bfloat16, 4)
    _check_tensor("k", k, torch.bfloat16, 4)
    _check_tensor("v", v, torch.bfloat16, 4)
    B, h, Tq, d = q.shape
    Tk = k.shape[2]
    if tuple(k.shape) != (B, h, Tk, d) or tuple(v.shape) != (B, h, Tk, d):
        raise ValueError(f"shape mismatch: q {tuple(q.shape)}, k {tuple(k.shape)}, v {tuple(v.shape)}")
    if not (q.device == k.device == v.device):
        raise ValueError("q, k and v must be on the same device")
    if o is None:
        o = torch.empty((B, h, Tq, d), dtype=out_dtype, device=q.device)
    if lse is None:
        lse = torch.empty((B, h, Tq), dtype=torch.float32, device=q.device)
    _check_tensor("o", o, out_dtype, 4)
    _check_tensor("lse", lse, torch.float32, 3)
    if tuple(o.shape) != (B, h, Tq, d) or tuple(lse.shape) != (B, h, Tq):
        raise ValueError("output shapes do not match the inputs")
    scale = _default_scale(d) if scale is None else float(scale)
    st = entry(q.data_ptr(), k.data_ptr(), v.data_ptr(), o.data_ptr(), lse.data_ptr(),
               B, h, Tq, Tk, d, int(bool(causal)), scale, _stream_handle(stream, q.device))
    if st != FA_OK:
        raise FaError(st)
    return o, lse


def fa_fwd(q, k, v, *, causal: bool, scale: float | None = None, o=None, lse=None, stream=None):
    """Attention forward.  q [B,h,Tq,d], k/v [B,h,Tk,d] bf16 on the GPU -> (o bf16, lse fp32).

    Enqueued on ``stream`` (default: torch's current stream); outputs are allocated with
    ``torch.empty`` unless given.  ``scale`` defaults to 1/sqrt(d).
    """
    return _fwd(_lib.lib.fa_fwd, torch.bfloat16, q, k, v, causal, scale, o, lse, stream)


def fa_fwd_o32(q, k, v, *, causal: bool, scale: float | None = None, o=None, lse=None,
               stream=None):
    """Same kernel as :func:`fa_fwd` with an fp32 O (parity diagnostics)."""
    return _fwd(_lib.lib.fa_fwd_o32, torch.float32, q, k, v, causal, scale, o, lse, stream)


def _strides3(name, t):
    """(batch, head, row) element strides of a 4-D [B, h, T, d] view with a contiguous last dim."""
    import ctypes
    if not isinstance(t, torch.Tensor) or t.device.type != "cuda" or t.dim() != 4:
        raise ValueError(f"{name} must be a 4-D GPU tensor [B, h, T, d]")
    if t.stride(3) != 1:
        raise ValueError(f"{name}: the last dimension must be contiguous")
    return (ctypes.c_int64 * 3)(t.stride(0), t.stride(1), t.stride(2))


def fa_fwd_strided(q, k, v, *, causal: bool, scale: float | None = None, o=None, lse=None,
                   stream=None):
    """Attention forward on strided [B, h, T, d] views (e.g. ``x.transpose(1, 2)`` of a
    [B, T, h, d] tensor): q, k, v bf16 with a contiguous last dimension -> (o, lse).

    ``o`` defaults to a contiguous [B, h, Tq, d] bf16 tensor and may be any such view; ``lse`` is
    contiguous [B, h, Tq] fp32.
    """
    for name, t in (("q", q), ("k", k), ("v", v)):
        if not isinstance(t, torch.Tensor) or t.dtype != torch.bfloat16:
            raise ValueError(f"{name} must be a bf16 tensor")
    B, h, Tq, d = q.shape
    Tk = k.shape[2]
    if tuple(k.shape) != (B, h, Tk, d) or tuple(v.shape) != (B, h, Tk, d):
        raise ValueError(f"shape mismatch: q {tuple(q.shape)}, k {tuple(k.shape)}, v {tuple(v.shape)}")
    if o is None:
        o = torch.empty((B, h, Tq, d), dtype=torch.bfloat16, device=q.device)
    if lse is None:
        lse = torch.empty((B, h, Tq), dtype=torch.float32, device=q.device)
    if o.dtype != torch.bfloat16 or tuple(o.shape) != (B, h, Tq, d):
        raise ValueError("o must be a bf16 [B, h, Tq, d] view")
    _check_tensor("lse", lse, torch.float32, 3)
    if len({t.device for t in (q, k, v, o, lse)}) != 1:
        raise ValueError("all tensors must be on the same device")
    scale = _default_scale(d) if scale is None else float(scale)
    st = _lib.lib.fa_fwd_strided(q.data_ptr(), k.data_ptr(), v.data_ptr(), o.data_ptr(),
                                 lse.data_ptr(), B, h, Tq, Tk, d, _strides3("q", q),
                                 _strides3("k", k), _strides3("v", v), _strides3("o", o),
                                 int(bool(causal)), scale, _stream_handle(stream, q.device))
    if st != FA_OK:
        raise FaError(st)
    return o, lse


def fa_validate_fwd_strided(q_ptr, k_ptr, v_ptr, o_ptr, lse_ptr, B, h, Tq, Tk, d_head, q_strides,
                            k_strides, v_strides, o_strides, causal, scale):
    """Host-only argument check of fa_fwd_strided (raw addresses; strides as 3-sequences)."""
    import ctypes
    arr = [None if s_ is None else (ctypes.c_int64 * 3)(*s_)
           for s_ in (q_strides, k_strides, v_strides, o_strides)]
    return int(_lib.lib.fa_validate_fwd_strided(q_ptr, k_ptr, v_ptr, o_ptr, lse_ptr, B, h, Tq, Tk,
                                                d_head, *arr, int(causal), float(scale)))


def fa_decode(q, k, v, *, num_splits: int, scale: float | None = None, o=None, lse=None,
              workspace=None, stream=None):
    """Split-KV decode.  q [B,h,d], k/v [B,h,Tk,d] bf16 -> (o [B,h,d] bf16, lse [B,h] fp32).

    ``workspace`` (a uint8 GPU tensor of at least fa_decode_workspace_size bytes) is allocated
    with ``torch.empty`` unless given.
    """
    _check_tensor("q", q, torch.bfloat16, 3)
    _check_tensor("k", k, torch.bfloat16, 4)
    _check_tensor("v", v, torch.bfloat16, 4)
    B, h, d = q.shape
    Tk = k.shape[2]
    if tuple(k.shape) != (B, h, Tk, d) or tuple(v.shape) != (B, h, Tk, d):
        raise ValueError(f"shape mismatch: q {tuple(q.shape)}, k {tuple(k.shape)}, v {tuple(v.shape)}")
    if o is None:
        o = torch.empty((B, h, d), dtype=torch.bfloat16, device=q.device)
    if lse is None:
        lse = torch.empty((B, h), dtype=torch.float32, device=q.device)
    _check_tensor("o", o, torch.bfloat16, 3)
    _check_tensor("lse", lse, torch.float32, 2)
    need = fa_decode_workspace_size(B, h, d, num_splits)
    if workspace is None:
        workspace = torch.empty(max(need, 16), dtype=torch.uint8, device=q.device)
    _check_tensor("workspace", workspace, torch.uint8, 1)
    scale = _default_scale(d) if scale is None else float(scale)
    st = _lib.lib.fa_decode(q.data_ptr(), k.data_ptr(), v.data_ptr(), o.data_ptr(), lse.data_ptr(),
                            B, h, Tk, d, scale, int(num_splits), workspace.data_ptr(),
                            workspace.numel(), _stream_handle(stream, q.device))
    if st != FA_OK:
        raise FaError(st)
    return o, lse


def fa_decode_noalloc(q, k, v, *, num_splits: int, scale: float | None = None, o=None,
                      lse=None, stream=None):
    """:func:`fa_decode` with the partials in the library's static per-GPU array instead of a
    workspace: the library allocates nothing (pass ``o`` and ``lse`` for an allocation-free
    call).  Calls that overlap on one GPU race on that array.  FA_ERR_SCRATCH when the partials,
    fa_decode_workspace_size(B, h, d, num_splits) bytes, exceed FA_NOALLOC_SCRATCH_BYTES."""
    _check_tensor("q", q, torch.bfloat16, 3)
    _check_tensor("k", k, torch.bfloat16, 4)
    _check_tensor("v", v, torch.bfloat16, 4)
    B, h, d = q.shape
    Tk = k.shape[2]
    if tuple(k.shape) != (B, h, Tk, d) or tuple(v.shape) != (B, h, Tk, d):
        raise ValueError(f"shape mismatch: q {tuple(q.shape)}, k {tuple(k.shape)}, v {tuple(v.shape)}")
    if o is None:
        o = torch.empty((B, h, d), dtype=torch.bfloat16, device=q.device)
    if lse is None:
        lse = torch.empty((B, h), dtype=torch.float32, device=q.device)
    _check_tensor("o", o, torch.bfloat16, 3)
    _check_tensor("lse", lse, torch.float32, 2)
    scale = _default_scale(d) if scale is None else float(scale)
    st = _lib.lib.fa_decode_noalloc(q.data_ptr(), k.data_ptr(), v.data_ptr(), o.data_ptr(),
                                    lse.data_ptr(), B, h, Tk, d, scale, int(num_splits),
                                    _stream_handle(stream, q.device))
    if st != FA_OK:
        raise FaError(st)
    return o, lse


def _strides2(name, t):
    """(batch, head) element strides of a 3-D [B, h, d] view with a contiguous last dim."""
    import ctypes
    if not isinstance(t, torch.Tensor) or t.device.type != "cuda" or t.dim() != 3:
        raise ValueError(f"{name} must be a 3-D GPU tensor [B, h, d]")
    if t.stride(2) != 1:
        raise ValueError(f"{name}: the last dimension must be contiguous")
    return (ctypes.c_int64 * 2)(t.stride(0), t.stride(1))


def fa_decode_strided(q, k, v, *, num_splits: int, scale: float | None = None, o=None, lse=None,
                      workspace=None, stream=None):
    """Split-KV decode on strided views and any head dim d <= 128 that is a multiple of 8:
    q [B,h,d], k/v [B,h,Tk,d] bf16 views (e.g. ``cache.transpose(1, 2)`` of a [B,Tk,h,d] KV
    cache) with a contiguous last dimension -> (o [B,h,d] bf16, lse [B,h] fp32).

    ``o`` defaults to a contiguous tensor and may be any such view; ``lse`` is contiguous.
    """
    for name, t, nd in (("q", q, 3), ("k", k, 4), ("v", v, 4)):
        if not isinstance(t, torch.Tensor) or t.dtype != torch.bfloat16 or t.dim() != nd:
            raise ValueError(f"{name} must be a {nd}-D bf16 tensor")
    B, h, d = q.shape
    Tk = k.shape[2]
    if tuple(k.shape) != (B, h, Tk, d) or tuple(v.shape) != (B, h, Tk, d):
        raise ValueError(f"shape mismatch: q {tuple(q.shape)}, k {tuple(k.shape)}, v {tuple(v.shape)}")
    if o is None:
        o = torch.empty((B, h, d), dtype=torch.bfloat16, device=q.device)
    if lse is None:
        lse = torch.empty((B, h), dtype=torch.float32, device=q.device)
    if o.dtype != torch.bfloat16 or tuple(o.shape) != (B, h, d):
        raise ValueError("o must be a bf16 [B, h, d] view")
    _check_tensor("lse", lse, torch.float32, 2)
    need = fa_decode_workspace_size(B, h, d, num_splits)
    if workspace is None:
        workspace = torch.empty(max(need, 16), dtype=torch.uint8, device=q.device)
    _check_tensor("workspace", workspace, torch.uint8, 1)
    if len({t.device for t in (q, k, v, o, lse, workspace)}) != 1:
        raise ValueError("all tensors must be on the same device")
    scale = _default_scale(d) if scale is None else float(scale)
    st = _lib.lib.fa_decode_strided(q.data_ptr(), k.data_ptr(), v.data_ptr(), o.data_ptr(),
                                    lse.data_ptr(), B, h, Tk, d, _strides2("q", q),
                                    _strides3("k", k), _strides3("v", v), _strides2("o", o),
                                    scale, int(num_splits), workspace.data_ptr(),
                                    workspace.numel(), _stream_handle(stream, q.device))
    if st != FA_OK:
        raise FaError(st)
    return o, lse


def fa_validate_decode_strided(q_ptr, k_ptr, v_ptr, o_ptr, lse_ptr, B, h, Tk, d_head, q_strides,
                               k_strides, v_strides, o_strides, scale, num_splits, ws_ptr,
                               ws_bytes):
    """Host-only argument check of fa_decode_strided (raw addresses; q / o strides as
    2-sequences, k / v strides as 3-sequences, or None)."""
    import ctypes
    arr = [None if s_ is None else (ctypes.c_int64 * len(s_))(*s_)
           for s_ in (q_strides, k_strides, v_strides, o_strides)]
    return int(_lib.lib.fa_validate_decode_strided(q_ptr, k_ptr, v_ptr, o_ptr, lse_ptr, B, h, Tk,
                                                   d_head, *arr, float(scale), int(num_splits),
                                                   ws_ptr, ws_bytes))


def _bwd(entry, out_dtype, q, k, v, o, do, lse, causal, scale, dq, dk, dv, workspace, stream):
    for name, t in (("q", q), ("k", k), ("v", v), ("o", o), ("do", do)):
        _check_tensor(name, t, torch.bfloat16, 4)
    B, h, Tq, d = q.shape
    Tk = k.shape[2]
    if (tuple(k.shape) != (B, h, Tk, d) or tuple(v.shape) != (B, h, Tk, d) or
            tuple(o.shape) != (B, h, Tq, d) or tuple(do.shape) != (B, h, Tq, d)):
        raise ValueError(f"shape mismatch: q {tuple(q.shape)}, k {tuple(k.shape)}, "
                         f"v {tuple(v.shape)}, o {tuple(o.shape)}, do {tuple(do.shape)}")
    _check_tensor("lse", lse, torch.float32, 3)
    if tuple(lse.shape) != (B, h, Tq):
        raise ValueError(f"lse must be [B, h, Tq], got {tuple(lse.shape)}")
    if len({t.device for t in (q, k, v, o, do, lse)}) != 1:
        raise ValueError("all inputs must be on the same device")
    if dq is None:
        dq = torch.empty((B, h, Tq, d), dtype=out_dtype, device=q.device)
    if dk is None:
        dk = torch.empty((B, h, Tk, d), dtype=out_dtype, device=q.device)
    if dv is None:
        dv = torch.empty((B, h, Tk, d), dtype=out_dtype, device=q.device)
    for name, t, shape in (("dq", dq, (B, h, Tq, d)), ("dk", dk, (B, h, Tk, d)),
                           ("dv", dv, (B, h, Tk, d))):
        _check_tensor(name, t, out_dtype, 4)
        if tuple(t.shape) != shape:
            raise ValueError(f"{name} must have shape {shape}, got {tuple(t.shape)}")
    need = fa_bwd_workspace_size(B, h, Tq)
    if workspace is None:
        workspace = torch.empty(max(need, 16), dtype=torch.uint8, device=q.device)
    _check_tensor("workspace", workspace, torch.uint8, 1)
    scale = _default_scale(d) if scale is None else float(scale)
    st = entry(q.data_ptr(), k.data_ptr(), v.data_ptr(), o.data_ptr(), do.data_ptr(),
               lse.data_ptr(), dq.data_ptr(), dk.data_ptr(), dv.data_ptr(), B, h, Tq, Tk, d,
               int(bool(causal)), scale, workspace.data_ptr(), workspace.numel(),
               _stream_handle(stream, q.device))
    if st != FA_OK:
        raise FaError(st)
    return dq, dk, dv


def fa_bwd(q, k, v, o, do, lse, *, causal: bool, scale: float | None = None, dq=None, dk=None,
           dv=None, workspace=None, stream=None):
    """Attention backward -> (dq, dk, dv) bf16, the gradients of sum(do * o).

    q, o, do [B,h,Tq,d] and k, v [B,h,Tk,d] bf16, lse [B,h,Tq] fp32: o and lse are
    :func:`fa_fwd`'s outputs for the same q, k, v, causal and scale.  ``workspace`` (a uint8 GPU
    tensor of at least fa_bwd_workspace_size bytes) and the outputs are allocated with
    ``torch.empty`` unless given.
    """
    return _bwd(_lib.lib.fa_bwd, torch.bfloat16, q, k, v, o, do, lse, causal, scale, dq, dk, dv,
                workspace, stream)


def fa_bwd_f32(q, k, v, o, do, lse, *, causal: bool, scale: float | None = None, dq=None,
               dk=None, dv=None, workspace=None, stream=None):
    """Same kernels as :func:`fa_bwd` with fp32 gradients (parity diagnostics)."""
    return _bwd(_lib.lib.fa_bwd_f32, torch.float32, q, k, v, o, do, lse, causal, scale, dq, dk,
                dv, workspace, stream)


def fa_validate_bwd(q_ptr, k_ptr, v_ptr, o_ptr, do_ptr, lse_ptr, dq_ptr, dk_ptr, dv_ptr, B, h, Tq,
                    Tk, d_head, causal, scale, ws_ptr, ws_bytes):
    """Host-only argument check of the backward entry points (raw integer addresses)."""
    return int(_lib.lib.fa_validate_bwd(q_ptr, k_ptr, v_ptr, o_ptr, do_ptr, lse_ptr, dq_ptr,
                                        dk_ptr, dv_ptr, B, h, Tq, Tk, d_head, int(causal),
                                        float(scale), ws_ptr, ws_bytes))


def fa_bwd_strided(q, k, v, o, do, lse, *, causal: bool, scale: float | None = None, dq=None,
                   dk=None, dv=None, workspace=None, stream=None):
    """Attention backward on strided [B, h, T, d] views (e.g. ``x.transpose(1, 2)`` of a
    [B, T, h, d] tensor) and any head dim d <= 128 that is a multiple of 8 -> (dq, dk, dv) bf16.

    Every tensor needs a contiguous last dimension; lse is contiguous [B, h, Tq] fp32.  The
    outputs default to ``torch.empty_like`` of q, k and v (same strides) and may be any such
    views.
    """
    for name, t in (("q", q), ("k", k), ("v", v), ("o", o), ("do", do)):
        if not isinstance(t, torch.Tensor) or t.dtype != torch.bfloat16 or t.dim() != 4:
            raise ValueError(f"{name} must be a 4-D bf16 tensor")
    B, h, Tq, d = q.shape
    Tk = k.shape[2]
    if (tuple(k.shape) != (B, h, Tk, d) or tuple(v.shape) != (B, h, Tk, d) or
            tuple(o.shape) != (B, h, Tq, d) or tuple(do.shape) != (B, h, Tq, d)):
        raise ValueError(f"shape mismatch: q {tuple(q.shape)}, k {tuple(k.shape)}, "
                         f"v {tuple(v.shape)}, o {tuple(o.shape)}, do {tuple(do.shape)}")
    _check_tensor("lse", lse, torch.float32, 3)
    if tuple(lse.shape) != (B, h, Tq):
        raise ValueError(f"lse must be [B, h, Tq], got {tuple(lse.shape)}")
    dq = torch.empty_like(q) if dq is None else dq
    dk = torch.empty_like(k) if dk is None else dk
    dv = torch.empty_like(v) if dv is None else dv
    for name, t, shape in (("dq", dq, (B, h, Tq, d)), ("dk", dk, (B, h, Tk, d)),
                           ("dv", dv, (B, h, Tk, d))):
        if not isinstance(t, torch.Tensor) or t.dtype != torch.bfloat16 or tuple(t.shape) != shape:
            raise ValueError(f"{name} must be a bf16 view of shape {shape}")
    if len({t.device for t in (q, k, v, o, do, lse, dq, dk, dv)}) != 1:
        raise ValueError("all tensors must be on the same device")
    need = fa_bwd_workspace_size(B, h, Tq)
    if workspace is None:
        workspace = torch.empty(max(need, 16), dtype=torch.uint8, device=q.device)
    _check_tensor("workspace", workspace, torch.uint8, 1)
    scale = _default_scale(d) if scale is None else float(scale)
    st = _lib.lib.fa_bwd_strided(
        q.data_ptr(), k.data_ptr(), v.data_ptr(), o.data_ptr(), do.data_ptr(), lse.data_ptr(),
        dq.data_ptr(), dk.data_ptr(), dv.data_ptr(), B, h, Tq, Tk, d,
        *(_strides3(n, t) for n, t in (("q", q), ("k", k), ("v", v), ("o", o), ("do", do),
                                        ("dq", dq), ("dk", dk), ("dv", dv))),
        int(bool(causal)), scale, workspace.data_ptr(), workspace.numel(),
        _stream_handle(stream, q.device))
    if st != FA_OK:
        raise FaError(st)
    return dq, dk, dv


def fa_validate_bwd_strided(q_ptr, k_ptr, v_ptr, o_ptr, do_ptr, lse_ptr, dq_ptr, dk_ptr, dv_ptr,
                            B, h, Tq, Tk, d_head, strides, causal, scale, ws_ptr, ws_bytes):
    """Host-only argument check of fa_bwd_strided (raw addresses; ``strides`` is a sequence of
    eight 3-sequences or None, for q, k, v, o, do, dq, dk, dv)."""
    import ctypes
    arr = [None if s_ is None else (ctypes.c_int64 * 3)(*s_) for s_ in strides]
    return int(_lib.lib.fa_validate_bwd_strided(q_ptr, k_ptr, v_ptr, o_ptr, do_ptr, lse_ptr,
                                                dq_ptr, dk_ptr, dv_ptr, B, h, Tq, Tk, d_head,
                                                *arr, int(causal), float(scale), ws_ptr,
                                                ws_bytes))


def fa_softmax_rows(x, *, y=None, lse=None, with_lse: bool = False, stream=None):
    """Row softmax of a contiguous [rows, cols] fp32 GPU tensor -> (y, lse or None).

    ``y`` (and, with ``with_lse`` or a given ``lse``, the [rows] fp32 log-sum-exp) are allocated
    with ``torch.empty`` unless given.
    """
    _check_tensor("x", x, torch.float32, 2)
    rows, cols = x.shape
    if y is None:
        y = torch.empty_like(x)
    _check_tensor("y", y, torch.float32, 2)
    if tuple(y.shape) != (rows, cols) or y.device != x.device:
        raise ValueError("y must match x in shape and device")
    if lse is None and with_lse:
        lse = torch.empty(rows, dtype=torch.float32, device=x.device)
    if lse is not None:
        _check_tensor("lse", lse, torch.float32, 1)
        if lse.shape[0] != rows:
            raise ValueError("lse must have one entry per row")
    st = _lib.lib.fa_softmax_rows(x.data_ptr(), y.data_ptr(),
                                  None if lse is None else lse.data_ptr(), rows, cols,
                                  _stream_handle(stream, x.device))
    if st != FA_OK:
        raise FaError(st)
    return y, lse


def fa_validate_softmax(x_ptr, y_ptr, lse_ptr, rows, cols):
    """Host-only argument check of fa_softmax_rows (raw integer addresses)."""
    return int(_lib.lib.fa_validate_softmax(x_ptr, y_ptr, lse_ptr, rows, cols))


def _gelu(entry, dtype, x, y, stream):
    if not isinstance(x, torch.Tensor) or x.device.type != "cuda" or x.dtype != dtype:
        raise ValueError(f"x must be a {dtype} GPU tensor")
    if not x.is_contiguous():
        raise ValueError("x must be contiguous")
    if y is None:
        y = torch.empty_like(x)
    if (not isinstance(y, torch.Tensor) or y.dtype != dtype or y.device != x.device or
            y.shape != x.shape or not y.is_contiguous()):
        raise ValueError("y must be a contiguous tensor like x")
    st = entry(x.data_ptr(), y.data_ptr(), x.numel(), _stream_handle(stream, x.device))
    if st != FA_OK:
        raise FaError(st)
    return y


def fa_gelu_f32(x, *, y=None, stream=None):
    """GELU (tanh form) of a contiguous fp32 GPU tensor of any shape, one pass over HBM."""
    return _gelu(_lib.lib.fa_gelu_f32, torch.float32, x, y, stream)


def fa_gelu_bf16(x, *, y=None, stream=None):
    """GELU (tanh form) of a contiguous bf16 GPU tensor, fp32 arithmetic, bf16 output."""
    return _gelu(_lib.lib.fa_gelu_bf16, torch.bfloat16, x, y, stream)


def fa_bias_gelu_dropout_bf16(x, bias, *, p: float, seed: int, offset: int = 0, y=None,
                              stream=None):
    """y = dropout(gelu(x + bias)) for a contiguous [rows, cols] bf16 tensor and a [cols] bias.

    The mask comes from Philox4x32-10 at (seed, offset) as the C header specifies.
    """
    _check_tensor("x", x, torch.bfloat16, 2)
    _check_tensor("bias", bias, torch.bfloat16, 1)
    rows, cols = x.shape
    if bias.shape[0] != cols or bias.device != x.device:
        raise ValueError("bias must have one entry per column, on x's device")
    if y is None:
        y = torch.empty_like(x)
    _check_tensor("y", y, torch.bfloat16, 2)
    if tuple(y.shape) != (rows, cols):
        raise ValueError("y must match x")
    st = _lib.lib.fa_bias_gelu_dropout_bf16(x.data_ptr(), bias.data_ptr(), y.data_ptr(), rows,
                                            cols, float(p), int(seed) & (2**64 - 1),
                                            int(offset) & (2**64 - 1),
                                            _stream_handle(stream, x.device))
    if st != FA_OK:
        raise FaError(st)
    return y


def fa_validate_gelu(x_ptr, y_ptr, n):
    """Host-only argument check of fa_gelu_f32 / fa_gelu_bf16 (raw integer addresses)."""
    return int(_lib.lib.fa_validate_gelu(x_ptr, y_ptr, n))


def fa_validate_bias_gelu_dropout(x_ptr, bias_ptr, y_ptr, rows, cols, p):
    """Host-only argument check of fa_bias_gelu_dropout_bf16 (raw integer addresses)."""
    return int(_lib.lib.fa_validate_bias_gelu_dropout(x_ptr, bias_ptr, y_ptr, rows, cols,
                                                      float(p)))


def fa_validate_fwd(q_ptr, k_ptr, v_ptr, o_ptr, lse_ptr, B, h, Tq, Tk, d_head, causal, scale):
    """Host-only argument check of the forward entry points (raw integer addresses)."""
    return int(_lib.lib.fa_validate_fwd(q_ptr, k_ptr, v_ptr, o_ptr, lse_ptr, B, h, Tq, Tk, d_head,
                                        int(causal), float(scale)))


def fa_validate_decode(q_ptr, k_ptr, v_ptr, o_ptr, lse_ptr, B, h, Tk, d_head, scale, num_splits,
                       ws_ptr, ws_bytes):
    """Host-only argument check of the decode entry point (raw integer addresses)."""
    return int(_lib.lib.fa_validate_decode(q_ptr, k_ptr, v_ptr, o_ptr, lse_ptr, B, h, Tk, d_head,
                                           float(scale), num_splits, ws_ptr, ws_bytes))
