"""``bwd``: torch front end of fa_bwd (memory, streams and argument marshalling)."""
from __future__ import annotations

import math
from typing import Optional

import torch

from . import _lib
from .fwd import _DT, _check_cu, _max_seqlen


def bwd(q: torch.Tensor, k: torch.Tensor, v: torch.Tensor, o: torch.Tensor,
        lse: torch.Tensor, dout: torch.Tensor, *, causal: bool = False,
        scale: Optional[float] = None, cu_seqlens: Optional[torch.Tensor] = None,
        max_seqlen: Optional[int] = None, grad_dtype: torch.dtype = torch.float32,
        workspace: Optional[torch.Tensor] = None,
        stream: Optional[torch.cuda.Stream] = None):
    """Gradients ``(dq, dk, dv)`` of ``sum(o * dout)`` for the forward that
    produced ``o`` and ``lse`` (``fwd`` with the same arguments).

    q, k, v, dout: float16 or bfloat16, contiguous, ``fwd``'s layouts (equal
    query and key counts).  o: the forward output (float32 or the input
    dtype).  Gradients are returned in ``grad_dtype`` (float32 or the input
    dtype).  ``workspace`` (uint8, fa_bwd_workspace_bytes) may be passed to
    avoid an allocation.
    """
    if q.dtype not in (torch.float16, torch.bfloat16):
        raise ValueError("bwd takes float16 or bfloat16 inputs")
    for name, t in (("k", k), ("v", v), ("dout", dout)):
        if t.dtype != q.dtype:
            raise ValueError(f"{name} must have q's dtype")
    if o.dtype not in (torch.float32, q.dtype) or grad_dtype not in (torch.float32, q.dtype):
        raise ValueError("o and the gradients are float32 or the input dtype")
    for name, t in (("q", q), ("k", k), ("v", v), ("o", o), ("lse", lse), ("dout", dout)):
        if not t.is_cuda or not t.is_contiguous():
            raise ValueError(f"{name} must be a contiguous device tensor")
    if k.shape != v.shape or o.shape != q.shape or dout.shape != q.shape:
        raise ValueError("shape mismatch among q, k, v, o, dout")
    if cu_seqlens is None:
        if q.dim() != 4 or k.dim() != 4 or k.shape[2] != q.shape[2]:
            raise ValueError("fixed layout needs q [B,Hq,N,d] and k/v [B,Hkv,N,d]")
        B, Hq, N, d = q.shape
        Hkv = k.shape[1]
        cu_ptr = None
    else:
        _check_cu(cu_seqlens)
        if q.dim() != 3 or k.dim() != 3 or k.shape[0] != q.shape[0]:
            raise ValueError("packed layout needs q [T,Hq,d] and k/v [T,Hkv,d]")
        _, Hq, d = q.shape
        Hkv = k.shape[1]
        B = cu_seqlens.numel() - 1
        N = _max_seqlen(cu_seqlens, max_seqlen)
        cu_ptr = cu_seqlens.data_ptr()
    if lse.dtype != torch.float32 or tuple(lse.shape) != (B, Hq, N):
        raise ValueError("lse must be float32 [B, Hq, N]")
    if scale is None:
        scale = 1.0 / math.sqrt(d)
    dt = _DT[q.dtype]
    need = _lib.bwd_workspace_bytes(B, Hq, Hkv, N, d, dt)
    stream = stream or torch.cuda.current_stream(q.device)
    # Tensors made here belong to `stream` (the caching allocator then never
    # hands their memory to other work before the kernels using it are done).
    with torch.cuda.device(q.device), torch.cuda.stream(stream):
        if workspace is None:
            workspace = torch.empty(need, dtype=torch.uint8, device=q.device)
        elif (workspace.dtype != torch.uint8 or not workspace.is_cuda
              or not workspace.is_contiguous()):
            raise ValueError("workspace must be a contiguous uint8 device tensor")
        dq = torch.empty(q.shape, dtype=grad_dtype, device=q.device)
        dk = torch.empty(k.shape, dtype=grad_dtype, device=q.device)
        dv = torch.empty(v.shape, dtype=grad_dtype, device=q.device)
        status = _lib.bwd_raw(q.data_ptr(), k.data_ptr(), v.data_ptr(), o.data_ptr(),
                              dout.data_ptr(), lse.data_ptr(), dq.data_ptr(), dk.data_ptr(),
                              dv.data_ptr(), B, Hq, Hkv, N, d, causal, float(scale), cu_ptr,
                              workspace.data_ptr(), workspace.numel(), stream.cuda_stream, dt,
                              _DT[o.dtype], _DT[grad_dtype])
    if status != _lib.FA_OK:
        raise RuntimeError(f"fa_bwd failed ({status}): {_lib.status_string(status)}")
    return dq, dk, dv
