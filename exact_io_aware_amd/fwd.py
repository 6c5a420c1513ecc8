"""``fwd``: torch front end of fa_fwd (memory, streams and argument marshalling)."""
from __future__ import annotations

import math
from typing import Optional, Sequence

import torch

from . import _lib

_DT = {torch.float32: _lib.FA_F32, torch.float16: _lib.FA_F16,
       torch.bfloat16: _lib.FA_BF16}


def fwd(q: torch.Tensor, k: torch.Tensor, v: torch.Tensor, *, causal: bool = False,
        scale: Optional[float] = None, cu_seqlens: Optional[torch.Tensor] = None,
        max_seqlen: Optional[int] = None, out_dtype: torch.dtype = torch.float32,
        out: Optional[torch.Tensor] = None, lse: Optional[torch.Tensor] = None,
        stream: Optional[torch.cuda.Stream] = None):
    """Exact attention forward on the GPU: returns ``(o, lse)``.

    Fixed length: q ``[B, Hq, N, d]``, k/v ``[B, Hkv, N, d]``.
    Packed varlen: q ``[T, Hq, d]``, k/v ``[T, Hkv, d]`` and ``cu_seqlens``
    (int32 device tensor ``[B+1]``); ``max_seqlen`` (>= the longest
    sequence) sizes the launch; if omitted it is read from ``cu_seqlens``,
    which synchronises.
    ``lse`` is float32 ``[B, Hq, N]``.  ``scale`` defaults to 1/sqrt(d).
    ``out``/``lse`` may be given to write into existing buffers.
    The kernel is enqueued on ``stream`` (default: the current stream).
    """
    if q.dtype not in _DT or k.dtype != q.dtype or v.dtype != q.dtype:
        raise ValueError("q, k, v must share one dtype among float32/float16/bfloat16")
    if out_dtype not in (torch.float32, q.dtype):
        raise ValueError("out_dtype must be float32 or the input dtype")
    for name, t in (("q", q), ("k", k), ("v", v)):
        if not t.is_cuda or not t.is_contiguous():
            raise ValueError(f"{name} must be a contiguous device tensor")
    if k.shape != v.shape:
        raise ValueError("k and v must have the same shape")
    if cu_seqlens is None:
        if q.dim() != 4 or k.dim() != 4:
            raise ValueError("fixed layout needs q [B,Hq,N,d] and k/v [B,Hkv,N,d]")
        B, Hq, N, d = q.shape
        if k.shape[0] != B or k.shape[2] != N or k.shape[3] != d:
            raise ValueError("k/v shape does not match q")
        Hkv = k.shape[1]
        cu_ptr = None
    else:
        if q.dim() != 3 or k.dim() != 3:
            raise ValueError("packed layout needs q [T,Hq,d] and k/v [T,Hkv,d]")
        if cu_seqlens.dtype != torch.int32 or not cu_seqlens.is_cuda or cu_seqlens.dim() != 1:
            raise ValueError("cu_seqlens must be an int32 device tensor [B+1]")
        if not cu_seqlens.is_contiguous():
            raise ValueError("cu_seqlens must be contiguous")
        T, Hq, d = q.shape
        if k.shape[0] != T or k.shape[2] != d:
            raise ValueError("k/v shape does not match q")
        Hkv = k.shape[1]
        B = cu_seqlens.numel() - 1
        if max_seqlen is None:
            max_seqlen = int((cu_seqlens[1:] - cu_seqlens[:-1]).max().item()) if B > 0 else 0
        N = int(max_seqlen)
        cu_ptr = cu_seqlens.data_ptr()
    if scale is None:
        scale = 1.0 / math.sqrt(d)
    if out is None:
        out = torch.empty(q.shape, dtype=out_dtype, device=q.device)
    elif out.dtype != out_dtype or out.shape != q.shape or not out.is_contiguous():
        raise ValueError("out has the wrong dtype, shape or layout")
    if lse is None:
        lse = torch.empty((B, Hq, N), dtype=torch.float32, device=q.device)
    elif lse.dtype != torch.float32 or tuple(lse.shape) != (B, Hq, N) or not lse.is_contiguous():
        raise ValueError("lse must be a contiguous float32 tensor [B, Hq, N]")
    st = (stream or torch.cuda.current_stream(q.device)).cuda_stream
    with torch.cuda.device(q.device):
        status = _lib.fwd_raw(q.data_ptr(), k.data_ptr(), v.data_ptr(), out.data_ptr(),
                              lse.data_ptr(), B, Hq, Hkv, N, d, causal, float(scale),
                              cu_ptr, st, _DT[q.dtype], _DT[out_dtype])
    if status != _lib.FA_OK:
        raise RuntimeError(f"fa_fwd failed ({status}): {_lib.status_string(status)}")
    return out, lse


def flops(Hq: int, d: int, lengths: Sequence[int], causal: bool) -> float:
    """Algorithmic FLOP of one forward: 4*d*Hq per visible (query, key) pair."""
    pairs = sum(n * (n + 1) // 2 if causal else n * n for n in lengths)
    return 4.0 * d * Hq * pairs
