"""A numpy model of the 16-bit forward kernel's rounding, for measuring what
its lazily moved running maximum costs in accuracy (test infrastructure: it
models the HIP kernel's arithmetic, it is not the oracle and shares no code
with the kernel).

Per query row the kernel streams keys in 32-key blocks.  A wave holds 32
consecutive rows of one head; lane l (l < 32) and lane l + 32 each hold 16
of the block's keys of row l (keys 0-3, 8-11, 16-19, 24-27 and the others).
For each block:

* P = exp2(scale * log2(e) * s - m) in fp32 against the row's reference
  maximum m (log2 units);
* each lane sums its 16 P in fp32; if any lane of the wave has a sum above
  the limit (or not finite), every row of the wave moves m to its true
  running maximum, rescales its accumulators by exp2(m_old - m_new) and
  forms P again (the "settle");
* the row's normaliser adds the fp32 sums; P is rounded to bf16 (round to
  nearest even) for the P.V product, which accumulates in fp32.

O = acc / l and L = (m + log2 l) ln 2 at the end.  ``limit=None`` models
the conventional form instead: the maximum moves at every block where a
score exceeds it (the dominant P is then exactly 1).
"""
from __future__ import annotations

import numpy as np

LOG2E = 1.4426950408889634
NO_MAX = -3.402823466e38


def _bf16(x: np.ndarray) -> np.ndarray:
    """Round float32 values to bfloat16 (RNE), returned as float32."""
    u = np.ascontiguousarray(x, dtype=np.float32).view(np.uint32)
    lsb = (u >> np.uint32(16)) & np.uint32(1)
    r = ((u + np.uint32(0x7FFF) + lsb) >> np.uint32(16)) << np.uint32(16)
    return r.astype(np.uint32).view(np.float32)


def _half_of_key(j: np.ndarray) -> np.ndarray:
    """Which lane half holds key j of a 32-key block (0 or 1)."""
    return (j // 4) % 2


def wave_forward(q: np.ndarray, k: np.ndarray, v: np.ndarray, rows: np.ndarray, scale: float,
                 causal: bool, limit, p_round=_bf16):
    """Model one wave: query rows ``rows`` (<= 32 of one head) against keys
    k, v [n, d] (float64 holding the stored 16-bit values).  Returns (O, L)
    in float64 for those rows."""
    n = k.shape[0]
    R = len(rows)
    sl2 = np.float32(scale * LOG2E)
    s_all = (q[rows] @ k.T).astype(np.float32)           # fp32 scores, [R, n]
    m = np.full(R, NO_MAX, np.float32)
    ell = np.zeros((R, 2), np.float32)
    acc = np.zeros((R, v.shape[1]), np.float64)
    last = n if not causal else int(rows.max()) + 1
    nblk = (last + 31) // 32
    for b in range(nblk):
        j = np.arange(32 * b, 32 * b + 32)
        valid = j[None, :] < n
        if causal:
            valid = valid & (j[None, :] <= rows[:, None])
        jj = np.minimum(j, n - 1)
        s = np.where(valid, s_all[:, jj], -np.inf).astype(np.float32)
        half = _half_of_key(j - 32 * b)

        def form(mref):
            x = (s.astype(np.float64) * np.float64(sl2) - mref[:, None].astype(np.float64))
            x = x.astype(np.float32)                     # one rounding (the FMA)
            with np.errstate(over="ignore"):
                p = np.exp2(x.astype(np.float64)).astype(np.float32)
            sums = np.stack([p[:, half == h].astype(np.float32).sum(axis=1, dtype=np.float32)
                             for h in (0, 1)], axis=1)
            return p, sums

        p, sums = form(m)
        if limit is None:
            # Conventional: move to the running maximum whenever it grows.
            bm = np.where(valid, s * sl2, -np.inf).max(axis=1).astype(np.float32)
            m_new = np.maximum(m, bm)
            need = m_new != m
            settle = bool(need.any())
        else:
            settle = bool((~(sums <= np.float32(limit))).any())
        if settle:
            bm = np.where(valid, s, -np.inf).max(axis=1).astype(np.float32) * sl2
            m_new = np.maximum(m, np.where(np.isfinite(bm), bm, m)).astype(np.float32)
            moved = m_new != m
            alpha = np.where(moved, np.exp2((m.astype(np.float64) - m_new)), 1.0)
            alpha = np.where(np.isfinite(alpha), alpha, 0.0)
            ell = (ell * alpha[:, None].astype(np.float32)).astype(np.float32)
            acc = acc * alpha[:, None]
            m = m_new
            p, sums = form(m)
        ell = (ell + sums).astype(np.float32)
        pr = p_round(np.where(valid, p, 0.0).astype(np.float32)).astype(np.float64)
        acc += pr @ v[jj]
    lt = ell.sum(axis=1, dtype=np.float32).astype(np.float64)
    O = acc / lt[:, None]
    L = (m.astype(np.float64) + np.log2(lt)) * np.log(2.0)
    return O, L


def head_forward(q, k, v, scale, causal, limit, p_round=_bf16):
    """All rows of one head, in waves of 32 consecutive rows."""
    n = q.shape[0]
    O = np.empty((n, v.shape[1]))
    L = np.empty(n)
    for r0 in range(0, n, 32):
        rows = np.arange(r0, min(n, r0 + 32))
        O[rows], L[rows] = wave_forward(q, k, v, rows, scale, causal, limit, p_round)
    return O, L
