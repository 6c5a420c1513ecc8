"""``fwd`` and ``pack_v``: torch front end of libfa (memory, streams and
argument marshalling)."""
from __future__ import annotations

import math
from typing import Optional, Sequence

import torch

from . import _lib

_DT = {torch.float32: _lib.FA_F32, torch.float16: _lib.FA_F16,
       torch.bfloat16: _lib.FA_BF16}


def _max_seqlen(cu_seqlens: torch.Tensor, max_seqlen: Optional[int]) -> int:
    if max_seqlen is not None:
        return int(max_seqlen)
    B = cu_seqlens.numel() - 1
    return int((cu_seqlens[1:] - cu_seqlens[:-1]).max().item()) if B > 0 else 0


def _check_cu(cu_seqlens: torch.Tensor) -> None:
    if cu_seqlens.dtype != torch.int32 or not cu_seqlens.is_cuda or cu_seqlens.dim() != 1:
        raise ValueError("cu_seqlens must be an int32 device tensor [B+1]")
    if not cu_seqlens.is_contiguous():
        raise ValueError("cu_seqlens must be contiguous")


def pack_v(v: torch.Tensor, *, cu_seqlens: Optional[torch.Tensor] = None,
           max_seqlen: Optional[int] = None, out: Optional[torch.Tensor] = None,
           stream: Optional[torch.cuda.Stream] = None) -> torch.Tensor:
    """fa_pack_v: V (float16/bfloat16, layout as in ``fwd``) transposed into
    64-key tiles, the form ``fwd(..., vt=...)`` reads (a decode cache's
    layout).  Returns the packed uint8 tensor (``out`` if given; it must hold
    fa_workspace_bytes)."""
    if v.dtype not in (torch.float16, torch.bfloat16):
        raise ValueError("pack_v takes float16 or bfloat16 values")
    if not v.is_cuda or not v.is_contiguous():
        raise ValueError("v must be a contiguous device tensor")
    if cu_seqlens is None:
        if v.dim() != 4:
            raise ValueError("fixed layout needs v [B,Hkv,N,d]")
        B, Hkv, N, d = v.shape
        cu_ptr = None
    else:
        _check_cu(cu_seqlens)
        if v.dim() != 3:
            raise ValueError("packed layout needs v [T,Hkv,d]")
        _, Hkv, d = v.shape
        B = cu_seqlens.numel() - 1
        N = _max_seqlen(cu_seqlens, max_seqlen)
        cu_ptr = cu_seqlens.data_ptr()
    nbytes = _lib.workspace_bytes(B, Hkv, N, d, _DT[v.dtype])
    stream = stream or torch.cuda.current_stream(v.device)
    # Tensors made here belong to `stream` (the caching allocator then never
    # hands their memory to other work before the kernel reading it is done).
    with torch.cuda.device(v.device), torch.cuda.stream(stream):
        if out is None:
            out = torch.empty(max(nbytes, 16), dtype=torch.uint8, device=v.device)
        elif out.dtype != torch.uint8 or not out.is_cuda or not out.is_contiguous():
            raise ValueError("out must be a contiguous uint8 device tensor")
        status = _lib.pack_v_raw(v.data_ptr(), out.data_ptr(), out.numel(), B, Hkv, N, d,
                                 cu_ptr, stream.cuda_stream, _DT[v.dtype])
    if status != _lib.FA_OK:
        raise RuntimeError(f"fa_pack_v failed ({status}): {_lib.status_string(status)}")
    return out


def fwd(q: torch.Tensor, k: torch.Tensor, v: Optional[torch.Tensor], *, causal: bool = False,
        scale: Optional[float] = None, cu_seqlens: Optional[torch.Tensor] = None,
        max_seqlen: Optional[int] = None, out_dtype: torch.dtype = torch.float32,
        out: Optional[torch.Tensor] = None, lse: Optional[torch.Tensor] = None,
        stream: Optional[torch.cuda.Stream] = None, vt: Optional[torch.Tensor] = None,
        cu_seqlens_k: Optional[torch.Tensor] = None,
        max_seqlen_k: Optional[int] = None, num_splits: Optional[int] = None,
        split_workspace: Optional[torch.Tensor] = None,
        block_mask: Optional[torch.Tensor] = None):
    """Exact attention forward on the GPU: returns ``(o, lse)``.

    Fixed length: q ``[B, Hq, Nq, d]``, k/v ``[B, Hkv, Nk, d]``.
    Packed varlen: q ``[Tq, Hq, d]``, k/v ``[Tk, Hkv, d]`` and ``cu_seqlens``
    (int32 device tensor ``[B+1]``, query offsets); ``cu_seqlens_k`` gives
    separate key/value offsets (default: the same as the queries).
    ``max_seqlen`` / ``max_seqlen_k`` (>= the longest query / key count)
    size the launch; if omitted they are read from the offsets, which
    synchronises.
    When a sequence has fewer queries than keys, the queries are its last
    tokens (chunked prefill): with ``causal`` query row r sees keys
    ``c <= r + nk - nq``.
    ``lse`` is float32 ``[B, Hq, Nq]``.  ``scale`` defaults to 1/sqrt(d);
    any finite value is accepted.  ``out``/``lse`` may be given to write into
    existing buffers.  The kernels are enqueued on ``stream`` (default: the
    current stream), and tensors made here belong to that stream.

    The default path is fa_fwd (fa_fwd_kv): one launch, no workspace.
    ``vt`` passes V already packed by ``pack_v`` (``v`` may then be None):
    the *_packed entry points.

    Split-KV (16-bit): ``num_splits`` ranges of keys per unit, merged with
    their logsumexps (fa_fwd_kv_split, or fa_fwd_kv_split_packed with
    ``vt``); default fa_num_splits, which splits only decode-like shapes (at
    most 64 query rows per sequence) that would not fill the GPU.  The
    partials go to ``split_workspace`` (uint8, fa_split_workspace_bytes) or
    to a tensor made here.  ``num_splits=1`` never splits.

    Block-sparse (16-bit): ``block_mask`` is a contiguous uint8 device
    tensor ``[1 or B, 1 or Hq, ceil(Nq/64), ceil(Nk/64)]``; a nonzero entry
    (b, h, i, j) admits query rows [64i, 64i+64) of sequence b, head h
    against keys [64j, 64j+64) (fa_fwd_sparse, or fa_fwd_sparse_packed with
    ``vt``).  Rows that see no key get O = 0, L = -inf.
    """
    if v is None and vt is None:
        raise ValueError("v is needed unless a packed vt is given")
    if v is None:
        v = k            # shapes and dtype only; V itself comes from vt
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
        if cu_seqlens_k is not None:
            raise ValueError("cu_seqlens_k needs cu_seqlens")
        if q.dim() != 4 or k.dim() != 4:
            raise ValueError("fixed layout needs q [B,Hq,Nq,d] and k/v [B,Hkv,Nk,d]")
        B, Hq, N, d = q.shape
        if k.shape[0] != B or k.shape[3] != d:
            raise ValueError("k/v shape does not match q")
        Hkv, Nk = k.shape[1], k.shape[2]
        cu_ptr = cuk_ptr = None
    else:
        if q.dim() != 3 or k.dim() != 3:
            raise ValueError("packed layout needs q [Tq,Hq,d] and k/v [Tk,Hkv,d]")
        _check_cu(cu_seqlens)
        T, Hq, d = q.shape
        if k.shape[2] != d:
            raise ValueError("k/v shape does not match q")
        Hkv = k.shape[1]
        B = cu_seqlens.numel() - 1
        N = _max_seqlen(cu_seqlens, max_seqlen)
        cu_ptr = cu_seqlens.data_ptr()
        if cu_seqlens_k is None:
            if k.shape[0] != T:
                raise ValueError("k/v token count differs from q: pass cu_seqlens_k")
            Nk, cuk_ptr = N, cu_ptr
        else:
            _check_cu(cu_seqlens_k)
            if cu_seqlens_k.numel() != B + 1:
                raise ValueError("cu_seqlens_k must have as many entries as cu_seqlens")
            Nk = _max_seqlen(cu_seqlens_k, max_seqlen_k)
            cuk_ptr = cu_seqlens_k.data_ptr()
    same = Nk == N and cuk_ptr == cu_ptr
    if scale is None:
        scale = 1.0 / math.sqrt(d)
    packed = vt is not None
    if packed and q.dtype == torch.float32:
        raise ValueError("vt (packed V) is for float16/bfloat16 inputs")
    if packed and (vt.dtype != torch.uint8 or not vt.is_cuda or not vt.is_contiguous()):
        raise ValueError("vt must be the contiguous uint8 device tensor pack_v returns")
    dt, odt = _DT[q.dtype], _DT[out_dtype]
    stream = stream or torch.cuda.current_stream(q.device)
    st = stream.cuda_stream
    with torch.cuda.device(q.device), torch.cuda.stream(stream):
        if out is None:
            out = torch.empty(q.shape, dtype=out_dtype, device=q.device)
        elif out.dtype != out_dtype or out.shape != q.shape or not out.is_contiguous():
            raise ValueError("out has the wrong dtype, shape or layout")
        if lse is None:
            lse = torch.empty((B, Hq, N), dtype=torch.float32, device=q.device)
        elif (lse.dtype != torch.float32 or tuple(lse.shape) != (B, Hq, N)
              or not lse.is_contiguous()):
            raise ValueError("lse must be a contiguous float32 tensor [B, Hq, Nq]")
        vtp, vtn = (vt.data_ptr(), vt.numel()) if packed else (0, 0)
        if block_mask is not None:
            if q.dtype == torch.float32:
                raise ValueError("block_mask needs float16 or bfloat16 inputs")
            nqb, nkb = -(-N // 64), -(-Nk // 64)
            if (block_mask.dtype != torch.uint8 or not block_mask.is_cuda
                    or not block_mask.is_contiguous() or block_mask.dim() != 4
                    or block_mask.shape[0] not in (1, B) or block_mask.shape[1] not in (1, Hq)
                    or tuple(block_mask.shape[2:]) != (nqb, nkb)):
                raise ValueError(f"block_mask must be a contiguous uint8 device tensor "
                                 f"[1 or {B}, 1 or {Hq}, {nqb}, {nkb}]")
            if num_splits not in (None, 1):
                raise ValueError("block-sparse attention does not split over keys")
            mb, mh = int(block_mask.shape[0]), int(block_mask.shape[1])
            if packed:
                name = "fa_fwd_sparse_packed"
                status = _lib.fwd_sparse_packed_raw(
                    q.data_ptr(), k.data_ptr(), vtp, vtn, out.data_ptr(), lse.data_ptr(), B, Hq,
                    Hkv, N, Nk, d, causal, float(scale), cu_ptr, cuk_ptr,
                    block_mask.data_ptr(), mb, mh, st, dt, odt)
            else:
                name = "fa_fwd_sparse"
                status = _lib.fwd_sparse_raw(
                    q.data_ptr(), k.data_ptr(), v.data_ptr(), out.data_ptr(), lse.data_ptr(), B,
                    Hq, Hkv, N, Nk, d, causal, float(scale), cu_ptr, cuk_ptr,
                    block_mask.data_ptr(), mb, mh, st, dt, odt)
            if status != _lib.FA_OK:
                raise RuntimeError(f"{name} failed ({status}): {_lib.status_string(status)}")
            return out, lse
        n_splits = 1
        if q.dtype != torch.float32:
            n_splits = (_lib.num_splits(B, Hq, Hkv, N, Nk, d, dt) if num_splits is None
                        else int(num_splits))
        if n_splits > 1:
            need = _lib.split_workspace_bytes(B, Hq, N, d, n_splits)
            if split_workspace is None:
                split_workspace = torch.empty(need, dtype=torch.uint8, device=q.device)
            elif (split_workspace.dtype != torch.uint8 or not split_workspace.is_cuda
                  or not split_workspace.is_contiguous()):
                raise ValueError("split_workspace must be a contiguous uint8 device tensor")
            if packed:
                name = "fa_fwd_kv_split_packed"
                status = _lib.fwd_kv_split_packed_raw(
                    q.data_ptr(), k.data_ptr(), vtp, vtn, out.data_ptr(), lse.data_ptr(), B, Hq,
                    Hkv, N, Nk, d, causal, float(scale), cu_ptr, cuk_ptr, n_splits,
                    split_workspace.data_ptr(), split_workspace.numel(), st, dt, odt)
            else:
                name = "fa_fwd_kv_split"
                status = _lib.fwd_kv_split_raw(
                    q.data_ptr(), k.data_ptr(), v.data_ptr(), out.data_ptr(), lse.data_ptr(), B,
                    Hq, Hkv, N, Nk, d, causal, float(scale), cu_ptr, cuk_ptr, n_splits,
                    split_workspace.data_ptr(), split_workspace.numel(), st, dt, odt)
        elif packed and same:
            name = "fa_fwd_packed"
            status = _lib.fwd_packed_raw(q.data_ptr(), k.data_ptr(), vtp, vtn, out.data_ptr(),
                                         lse.data_ptr(), B, Hq, Hkv, N, d, causal, float(scale),
                                         cu_ptr, st, dt, odt)
        elif packed:
            name = "fa_fwd_kv_packed"
            status = _lib.fwd_kv_packed_raw(q.data_ptr(), k.data_ptr(), vtp, vtn,
                                            out.data_ptr(), lse.data_ptr(), B, Hq, Hkv, N, Nk,
                                            d, causal, float(scale), cu_ptr, cuk_ptr, st, dt,
                                            odt)
        elif same:
            name = "fa_fwd"
            status = _lib.fwd_raw(q.data_ptr(), k.data_ptr(), v.data_ptr(), out.data_ptr(),
                                  lse.data_ptr(), B, Hq, Hkv, N, d, causal, float(scale),
                                  cu_ptr, st, dt, odt)
        else:
            name = "fa_fwd_kv"
            status = _lib.fwd_kv_raw(q.data_ptr(), k.data_ptr(), v.data_ptr(), out.data_ptr(),
                                     lse.data_ptr(), B, Hq, Hkv, N, Nk, d, causal,
                                     float(scale), cu_ptr, cuk_ptr, st, dt, odt)
    if status != _lib.FA_OK:
        raise RuntimeError(f"{name} failed ({status}): {_lib.status_string(status)}")
    return out, lse


def _block_pairs(bm, nq: int, nk: int, causal: bool) -> int:
    """Visible (query, key) pairs of one head of one sequence under the
    block mask ``bm`` [row blocks, key blocks] of 64 x 64 blocks."""
    import numpy as np
    nqb, nkb = -(-nq // 64), -(-nk // 64)
    m = (np.asarray(bm)[:nqb, :nkb] != 0).astype(np.int64)
    r = np.arange(nq)
    span = np.minimum(nk, np.maximum(0, r + (nk - nq) + 1)) if causal else np.full(nq, nk)
    # keys of block j visible to row r: clip(span_r - 64 j, 0, min(64, nk - 64 j))
    j0 = 64 * np.arange(nkb)
    width = np.minimum(64, nk - j0)
    per = np.clip(span[:, None] - j0[None, :], 0, width[None, :])      # [nq, nkb]
    return int((per * m[r // 64]).sum())


def flops(Hq: int, d: int, lengths: Sequence[int], causal: bool,
          lengths_k: Optional[Sequence[int]] = None, block_mask=None) -> float:
    """Algorithmic FLOP of one forward: 4*d*Hq per visible (query, key) pair.
    ``lengths_k`` gives per-sequence key counts when they differ from the
    query counts (the queries are then the last tokens of each sequence).
    ``block_mask`` (numpy, [1 or B, 1 or Hq, row blocks, key blocks]) counts
    only the pairs its admitted 64 x 64 blocks hold."""
    if block_mask is not None:
        bm = block_mask
        ks = lengths if lengths_k is None else lengths_k
        pairs = 0
        for b, (nq, nk) in enumerate(zip(lengths, ks)):
            mb = bm[b if bm.shape[0] > 1 else 0]
            if mb.shape[0] == 1:
                pairs += Hq * _block_pairs(mb[0], int(nq), int(nk), causal)
            else:
                pairs += sum(_block_pairs(mb[h], int(nq), int(nk), causal) for h in range(Hq))
        return 4.0 * d * pairs
    if lengths_k is None:
        pairs = sum(n * (n + 1) // 2 if causal else n * n for n in lengths)
    else:
        pairs = 0
        for nq, nk in zip(lengths, lengths_k):
            nq, nk = int(nq), int(nk)
            if not causal:
                pairs += nq * nk
                continue
            # row r sees r + nk - nq + 1 keys when that is positive (never
            # more than nk, since r < nq)
            lo = max(0, nq - nk)
            pairs += sum(range(lo + nk - nq + 1, nk + 1)) if lo < nq else 0
    return 4.0 * d * Hq * pairs
