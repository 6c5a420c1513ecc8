"""``attention``: the forward and backward kernels as one differentiable torch
operation (argument marshalling only: both passes run in libfa.so).

The forward keeps O and the per-row logsumexp L for the backward, which
recomputes the probabilities from L block by block instead of storing them
(the tiling-plus-recomputation idea of the Kotaemon page's method
paragraph).  O is returned in the input dtype, as torch's own attention
does.
"""
from __future__ import annotations

from typing import Optional

import torch

from .bwd import bwd
from .fwd import fwd


class _Attention(torch.autograd.Function):
    @staticmethod
    def forward(ctx, q, k, v, causal, scale, cu_seqlens, max_seqlen):
        o, lse = fwd(q, k, v, causal=causal, scale=scale, cu_seqlens=cu_seqlens,
                     max_seqlen=max_seqlen, out_dtype=q.dtype, num_splits=1)
        ctx.save_for_backward(q, k, v, o, lse)
        ctx.cu_seqlens = cu_seqlens
        ctx.causal, ctx.scale, ctx.max_seqlen = causal, scale, max_seqlen
        return o

    @staticmethod
    def backward(ctx, do):
        q, k, v, o, lse = ctx.saved_tensors
        if q.dtype not in (torch.float16, torch.bfloat16):
            raise RuntimeError("the backward pass takes float16 or bfloat16 inputs")
        dq, dk, dv = bwd(q, k, v, o, lse, do.contiguous(), causal=ctx.causal, scale=ctx.scale,
                         cu_seqlens=ctx.cu_seqlens, max_seqlen=ctx.max_seqlen,
                         grad_dtype=q.dtype)
        return dq, dk, dv, None, None, None, None


def attention(q: torch.Tensor, k: torch.Tensor, v: torch.Tensor, *, causal: bool = False,
              scale: Optional[float] = None, cu_seqlens: Optional[torch.Tensor] = None,
              max_seqlen: Optional[int] = None) -> torch.Tensor:
    """softmax(scale * q k^T) v with gradients for q, k and v.

    Layouts and arguments as for ``fwd`` (``[B, H, N, d]`` or packed
    ``[T, H, d]`` with ``cu_seqlens``); the gradients need float16 or
    bfloat16 inputs, equal query and key counts and a positive scale
    (default 1/sqrt(d)).
    """
    return _Attention.apply(q, k, v, causal, scale, cu_seqlens, max_seqlen)
