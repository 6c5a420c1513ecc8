"""Seeded synthetic attention workloads.

This module is shared by the CPU oracle and the HIP path's tests and bench.
It only draws and rounds inputs; it holds none of the attention arithmetic.

Each workload is a shape, an input precision and a seed.  Inputs are drawn
as N(0, 1) in float32 with ``numpy.random.default_rng(seed)`` (in the order
lengths (varlen only), q, k, v, each in C order) and then rounded to the
storage precision with round-to-nearest-even.  The named workloads are:

* ``tiny_fp32``   B=1, H=2, N=256, d=64, fp32, non-causal (exactness case)
* ``mha_fp16``    B=8, H=12, N=2048, d=64, fp16, causal
* ``gqa_bf16``    B=4, Hq=32, Hkv=8, N=4096, d=128, bf16, causal (headline)
* ``long_bf16``   B=1, Hq=32, Hkv=8, N=32768, d=128, bf16, causal
* ``varlen_bf16`` 16 packed sequences, lengths uniform in [1024, 8192],
                  Hq=32, Hkv=8, d=128, bf16, causal
* ``prefill_bf16`` chunked prefill: the last 1024 queries of 8192-token
                  sequences, B=4, Hq=32, Hkv=8, d=128, bf16, causal
* ``decode_bf16`` decode: one new query per sequence against an 8192-token
                  KV cache, B=32, Hq=32, Hkv=8, d=128, bf16
* ``streaming_bf16`` block-sparse: the gqa_bf16 shape (seed 1008) under a
                  streaming block mask of 64 x 64 blocks: every query block
                  sees key block 0 (the "sink") and the 16 key blocks ending
                  at its own (a 1024-key window), causal
* ``gqa_bf16_tp8`` one GPU's share of gqa_bf16 split over 8 GPUs by K/V
                  head: B=4, Hq=4, Hkv=1, N=4096, d=128, bf16, causal
* ``long_bf16_sp8`` one GPU's share of long_bf16 split over 8 GPUs by query
                  rows in zig-zag order (GPU 0: rows [0, 2048) and
                  [30720, 32768) of the 32768-token sequence): two packed
                  sequences of 2048 queries, the last queries of 2048 and
                  32768 keys, Hq=32, Hkv=8, d=128, bf16, causal

When a workload has more keys than queries (``Nk``), k and v are drawn with
the key count and the queries are the last tokens of each sequence.

Storage formats returned by :func:`make_inputs`:

* fp32 -> ``numpy.float32``
* fp16 -> ``numpy.float16``
* bf16 -> ``numpy.uint16`` holding the bfloat16 bit patterns

Fixed-length layout is ``[B, H, N, d]``; varlen layout is token-major packed
``[T, H, d]`` with ``cu_seqlens`` (int32, ``[B+1]``) giving offsets.
"""
from __future__ import annotations

import dataclasses
import math
from typing import Optional, Sequence

import numpy as np

__all__ = [
    "Workload", "WORKLOADS", "HEADLINE", "make_inputs", "make_custom", "make_custom_qk",
    "round_to_bf16_bits", "bf16_bits_to_f32", "to_f64", "varlen_lengths",
    "streaming_block_mask", "random_block_mask", "SPARSE_BLOCK",
]

SPARSE_BLOCK = 64        # query rows and keys per block of a block mask


@dataclasses.dataclass(frozen=True)
class Workload:
    name: str
    B: int               # batch size, or number of packed sequences (varlen)
    Hq: int
    Hkv: int
    N: int               # sequence length, or max sequence length (varlen)
    d: int
    dtype: str           # "fp32" | "fp16" | "bf16"
    causal: bool
    seed: int
    varlen: bool = False
    len_lo: int = 0      # varlen: inclusive range of the uniform lengths
    len_hi: int = 0
    Nk: int = 0          # keys per sequence when more than the queries (0: = N)
    sink_blocks: int = 0     # block-sparse streaming mask (0 window: dense)
    window_blocks: int = 0
    lengths_q: tuple = ()    # varlen with given query and key counts per sequence
    lengths_k: tuple = ()

    @property
    def scale(self) -> float:
        return 1.0 / math.sqrt(self.d)


WORKLOADS = {
    w.name: w for w in [
        Workload("tiny_fp32", 1, 2, 2, 256, 64, "fp32", False, 1001),
        Workload("mha_fp16", 8, 12, 12, 2048, 64, "fp16", True, 1002),
        Workload("gqa_bf16", 4, 32, 8, 4096, 128, "bf16", True, 1003),
        Workload("long_bf16", 1, 32, 8, 32768, 128, "bf16", True, 1004),
        Workload("varlen_bf16", 16, 32, 8, 8192, 128, "bf16", True, 1005,
                 varlen=True, len_lo=1024, len_hi=8192),
        Workload("prefill_bf16", 4, 32, 8, 1024, 128, "bf16", True, 1006, Nk=8192),
        Workload("decode_bf16", 32, 32, 8, 1, 128, "bf16", True, 1007, Nk=8192),
        Workload("streaming_bf16", 4, 32, 8, 4096, 128, "bf16", True, 1008,
                 sink_blocks=1, window_blocks=16),
        Workload("gqa_bf16_tp8", 4, 4, 1, 4096, 128, "bf16", True, 1009),
        Workload("long_bf16_sp8", 2, 32, 8, 2048, 128, "bf16", True, 1010, varlen=True,
                 lengths_q=(2048, 2048), lengths_k=(2048, 32768)),
    ]
}

HEADLINE = "gqa_bf16"


def round_to_bf16_bits(x: np.ndarray) -> np.ndarray:
    """float32 -> bfloat16 bit patterns (uint16), round to nearest even.

    Inputs here are finite, so no NaN special-casing is needed.
    """
    u = np.ascontiguousarray(x, dtype=np.float32).view(np.uint32)
    lsb = (u >> np.uint32(16)) & np.uint32(1)
    r = (u + np.uint32(0x7FFF) + lsb) >> np.uint32(16)
    return r.astype(np.uint16)


def bf16_bits_to_f32(bits: np.ndarray) -> np.ndarray:
    """bfloat16 bit patterns (uint16) -> float32 (exact)."""
    return (np.asarray(bits, dtype=np.uint16).astype(np.uint32)
            << np.uint32(16)).view(np.float32)


def to_f64(arr: np.ndarray, dtype: str) -> np.ndarray:
    """Exact upcast of stored inputs to float64."""
    if dtype == "bf16":
        return bf16_bits_to_f32(arr).astype(np.float64)
    return np.asarray(arr).astype(np.float64)


def _round(x32: np.ndarray, dtype: str) -> np.ndarray:
    if dtype == "fp32":
        return x32
    if dtype == "fp16":
        return x32.astype(np.float16)      # numpy rounds to nearest even
    if dtype == "bf16":
        return round_to_bf16_bits(x32)
    raise ValueError(dtype)


def varlen_lengths(rng: np.random.Generator, count: int, lo: int, hi: int) -> np.ndarray:
    """Sequence lengths uniform over the inclusive integer range [lo, hi]."""
    return rng.integers(lo, hi + 1, count)


def make_custom(B: int, Hq: int, Hkv: int, d: int, dtype: str, seed: int,
                N: Optional[int] = None,
                lengths: Optional[Sequence[int]] = None) -> dict:
    """Draw q, k, v for an arbitrary shape.

    Give ``N`` for the fixed layout or ``lengths`` for the varlen layout.
    Returns a dict with q, k, v (storage format), cu_seqlens (varlen) or
    None, N (max length), dtype and the lengths.
    """
    rng = np.random.default_rng(seed)
    return _draw(rng, B, Hq, Hkv, d, dtype, N, lengths)


def _offsets(lengths, B):
    lengths = np.asarray(lengths, dtype=np.int64)
    assert lengths.shape == (B,)
    cu = np.zeros(B + 1, dtype=np.int32)
    cu[1:] = np.cumsum(lengths)
    return lengths, cu


def _draw(rng, B, Hq, Hkv, d, dtype, N, lengths, Nk=None, lengths_k=None):
    cu_k = None
    if lengths is not None:
        lengths, cu = _offsets(lengths, B)
        qs = (int(cu[-1]), Hq, d)
        nmax = int(lengths.max()) if B > 0 else 0
        if lengths_k is not None:
            lengths_k, cu_k = _offsets(lengths_k, B)
            ks = (int(cu_k[-1]), Hkv, d)
            nkmax = int(lengths_k.max()) if B > 0 else 0
        else:
            ks, nkmax = (int(cu[-1]), Hkv, d), nmax
    else:
        cu = None
        nk = N if Nk is None else Nk
        qs, ks = (B, Hq, N, d), (B, Hkv, nk, d)
        nmax, nkmax = N, nk
    q = _round(rng.standard_normal(qs, dtype=np.float32), dtype)
    k = _round(rng.standard_normal(ks, dtype=np.float32), dtype)
    v = _round(rng.standard_normal(ks, dtype=np.float32), dtype)
    return dict(q=q, k=k, v=v, cu_seqlens=cu, N=nmax, dtype=dtype,
                lengths=None if lengths is None else lengths.tolist(),
                B=B, Hq=Hq, Hkv=Hkv, d=d, Nk=nkmax, cu_seqlens_k=cu_k,
                lengths_k=None if lengths_k is None else lengths_k.tolist())


def make_custom_qk(B: int, Hq: int, Hkv: int, d: int, dtype: str, seed: int,
                   Nq: Optional[int] = None, Nk: Optional[int] = None,
                   lengths_q: Optional[Sequence[int]] = None,
                   lengths_k: Optional[Sequence[int]] = None) -> dict:
    """Draw q, k, v with separate query and key counts.

    Fixed layout: ``Nq``, ``Nk``.  Varlen: ``lengths_q`` and ``lengths_k``
    (both), giving ``cu_seqlens`` (queries) and ``cu_seqlens_k``.
    """
    rng = np.random.default_rng(seed)
    return _draw(rng, B, Hq, Hkv, d, dtype, Nq, lengths_q, Nk, lengths_k)


def streaming_block_mask(n: int, sink_blocks: int, window_blocks: int,
                         block: int = SPARSE_BLOCK) -> np.ndarray:
    """Streaming pattern over an n x n (query, key) grid, as a uint8 block
    mask [1, 1, nb, nb]: query block i admits key blocks j < sink_blocks and
    i - window_blocks < j <= i."""
    nb = -(-n // block)
    i = np.arange(nb)[:, None]
    j = np.arange(nb)[None, :]
    m = (j < sink_blocks) | ((j <= i) & (j > i - window_blocks))
    return m.astype(np.uint8)[None, None]


def random_block_mask(rng: np.random.Generator, Bm: int, Hm: int, nq: int, nk: int,
                      density: float, block: int = SPARSE_BLOCK) -> np.ndarray:
    """A uint8 block mask [Bm, Hm, ceil(nq/block), ceil(nk/block)] whose
    entries are 1 with probability ``density``."""
    shape = (Bm, Hm, -(-nq // block), -(-nk // block))
    return (rng.random(shape) < density).astype(np.uint8)


def make_inputs(w: Workload | str) -> dict:
    """Seeded inputs of a named workload (see the module docstring)."""
    if isinstance(w, str):
        w = WORKLOADS[w]
    rng = np.random.default_rng(w.seed)
    lengths = lengths_k = None
    if w.lengths_q:
        lengths, lengths_k = list(w.lengths_q), list(w.lengths_k)
    elif w.varlen:
        lengths = varlen_lengths(rng, w.B, w.len_lo, w.len_hi)
    out = _draw(rng, w.B, w.Hq, w.Hkv, w.d, w.dtype,
                None if w.varlen else w.N, lengths, Nk=w.Nk or None, lengths_k=lengths_k)
    out["causal"] = w.causal
    out["scale"] = w.scale
    out["name"] = w.name
    out["seed"] = w.seed
    if w.window_blocks:
        out["block_mask"] = streaming_block_mask(w.N, w.sink_blocks, w.window_blocks)
    return out
