"""Plain float64 attention on the CPU: the oracle (test infrastructure only).

Nothing in the product imports this module.  It states, as plainly as numpy
allows, what the exact IO-aware attention forward pass returns:

* the output ``O = softmax(scale * Q K^T) V``, the standard attention
  formula given on the Kotaemon page ("Kotaemon FlashAttention应用：加快注意力
  计算", the formula paragraph), with ``scale = 1/sqrt(d_k)`` in the
  configurations used here;
* the per-row normaliser that the tiling sketch on the HolySheep article
  ("Flash Attention", French edition, section "Principe fondamental : tiling
  et streaming") returns next to O.  It is read here as the natural-log
  logsumexp of the scaled, masked scores of the row,
  ``L_r = ln sum_c exp(scale * q_r . k_c)``.

The pages state that the tiled method with an online running maximum and
normaliser gives exactly this result (Kotaemon page, method list and the
paragraph after it; HolySheep article, Chinese edition, section
"IO 感知的算法设计").  So the oracle is the definition written out: it
materialises the whole score matrix (in row chunks, each row complete),
which is exactly what the GPU path must avoid.

Readings of points the pages leave open:

* Causal masking is top-left aligned: query row r of a sequence sees keys
  c <= r (indices within the sequence).  The manual chunking recipe in the
  French HolySheep article ("Erreurs courantes", item 1) gives query chunk
  [i, i+c) the key prefix [0, i+c), which is this alignment.
* Grouped-query attention: query head h reads key/value head
  ``h // (Hq // Hkv)``, contiguous groups; the page on transformer memory
  footprint ("Empreinte mémoire et calcul des couches Transformer dans les
  LLM en production", section "Les deux géants consommateurs") uses H_KV = 8
  for Llama-style models.
* Varlen packing: sequences are packed token-major ``[T, H, d]`` with
  int32 offsets ``cu_seqlens`` ``[B+1]``; L is returned as ``[B, Hq, Nmax]``
  with NaN in rows past a sequence's length.

Every array argument is float64 (the exact upcast of the stored inputs).
"""
from __future__ import annotations

import math
import os
from concurrent.futures import ProcessPoolExecutor
from typing import Iterable, Optional, Sequence, Tuple

import numpy as np

# Row chunk budget for the materialised score matrix (bytes of float64).
_CHUNK_BYTES = 256 << 20


def visible_keys(r: int, n: int, causal: bool) -> int:
    """Number of keys query row ``r`` of an ``n``-long sequence sees."""
    return r + 1 if causal else n


def softmax_rows(S: np.ndarray) -> Tuple[np.ndarray, np.ndarray, np.ndarray]:
    """Row softmax of a score block whose masked entries are -inf.

    Returns ``(P, m, ell)``: the probabilities, the row maxima and the row
    sums of ``exp(S - m)``; the logsumexp of row r is ``m_r + ln ell_r``.
    Every row must hold at least one finite entry.
    """
    m = S.max(axis=1, keepdims=True)
    E = np.exp(S - m)
    ell = E.sum(axis=1, keepdims=True)
    return E / ell, m[:, 0], ell[:, 0]


def _group(h: int, Hq: int, Hkv: int) -> int:
    if Hq % Hkv:
        raise ValueError("Hq must be a multiple of Hkv")
    return h // (Hq // Hkv)


def _head_rows(q: np.ndarray, k: np.ndarray, v: np.ndarray, causal: bool,
               scale: float, rows: Optional[np.ndarray] = None):
    """Attention of one head of one sequence, by the definition.

    q: [n, d], k/v: [n, d].  Returns O [R, d] and L [R] for the requested
    rows (all rows if ``rows`` is None).  The score rows are formed in
    chunks so that a very long sequence never holds more than
    ``_CHUNK_BYTES`` of scores; every row is complete within its chunk.
    """
    n = q.shape[0]
    if rows is None:
        rows = np.arange(n)
    rows = np.asarray(rows, dtype=np.int64)
    O = np.empty((rows.size, v.shape[1]), dtype=np.float64)
    L = np.empty(rows.size, dtype=np.float64)
    chunk = max(1, _CHUNK_BYTES // (8 * max(n, 1)))
    cols = np.arange(n)
    for s in range(0, rows.size, chunk):
        r = rows[s:s + chunk]
        S = scores(q[r], k, scale)                        # [R, n]
        if causal:
            S = causal_mask(S, r, cols)
        P, m, ell = softmax_rows(S)
        O[s:s + chunk] = combine(P, v)
        L[s:s + chunk] = logsumexp_of(m, ell)
    return O, L


def scores(q: np.ndarray, k: np.ndarray, scale: float) -> np.ndarray:
    """``scale * q k^T`` (the scaled dot products of the formula)."""
    return scale * (q @ k.T)


def causal_mask(S: np.ndarray, rows: np.ndarray, cols: np.ndarray) -> np.ndarray:
    """Set the scores of keys after the query (col > row) to -inf."""
    return np.where(cols[None, :] > rows[:, None], -np.inf, S)


def combine(P: np.ndarray, v: np.ndarray) -> np.ndarray:
    """The probability-weighted sum of value rows, ``P v``."""
    return P @ v


def logsumexp_of(m: np.ndarray, ell: np.ndarray) -> np.ndarray:
    """Natural-log logsumexp from the row maximum and the row sum of
    ``exp(S - m)``."""
    return m + np.log(ell)


def attention(q: np.ndarray, k: np.ndarray, v: np.ndarray, *, causal: bool,
              scale: float, cu_seqlens: Optional[np.ndarray] = None,
              workers: int = 1):
    """Exact attention forward: returns ``(O, L)`` in float64.

    Fixed layout: q ``[B, Hq, N, d]``, k/v ``[B, Hkv, N, d]``; O has q's
    shape and L is ``[B, Hq, N]``.
    Varlen layout (``cu_seqlens`` given): q ``[T, Hq, d]``, k/v
    ``[T, Hkv, d]``; O is ``[T, Hq, d]`` and L is ``[B, Hq, Nmax]`` with NaN
    past each sequence's length.
    ``workers`` > 1 spreads the (sequence, head) units over processes.
    """
    units = list(_units(q, k, cu_seqlens))
    results = _map(units, q, k, v, causal, scale, cu_seqlens, workers)
    return _assemble(q, cu_seqlens, units, results)


def _units(q, k, cu_seqlens):
    if cu_seqlens is None:
        B, Hq = q.shape[0], q.shape[1]
    else:
        B, Hq = len(cu_seqlens) - 1, q.shape[1]
    for b in range(B):
        for h in range(Hq):
            yield (b, h)


def _slices(q, k, v, b, h, cu_seqlens):
    Hq, Hkv = q.shape[1], k.shape[1]
    g = _group(h, Hq, Hkv)
    if cu_seqlens is None:
        return q[b, h], k[b, g], v[b, g]
    s, e = int(cu_seqlens[b]), int(cu_seqlens[b + 1])
    return q[s:e, h], k[s:e, g], v[s:e, g]


def _run_unit(args):
    qs, ks, vs, causal, scale = args
    return _head_rows(qs, ks, vs, causal, scale)


def _map(units, q, k, v, causal, scale, cu_seqlens, workers):
    jobs = [(*_slices(q, k, v, b, h, cu_seqlens), causal, scale) for b, h in units]
    if workers <= 1:
        return [_run_unit(j) for j in jobs]
    with ProcessPoolExecutor(max_workers=workers, initializer=_one_blas_thread) as ex:
        return list(ex.map(_run_unit, jobs, chunksize=1))


def _one_blas_thread():
    for var in ("OMP_NUM_THREADS", "OPENBLAS_NUM_THREADS", "MKL_NUM_THREADS"):
        os.environ[var] = "1"
    try:  # the environment variables only help before BLAS starts
        from threadpoolctl import threadpool_limits
        threadpool_limits(1)
    except Exception:
        pass


def _assemble(q, cu_seqlens, units, results):
    O = np.empty(q.shape, dtype=np.float64)
    if cu_seqlens is None:
        B, Hq, N = q.shape[0], q.shape[1], q.shape[2]
        L = np.empty((B, Hq, N), dtype=np.float64)
        for (b, h), (o, l) in zip(units, results):
            O[b, h] = o
            L[b, h] = l
        return O, L
    B, Hq = len(cu_seqlens) - 1, q.shape[1]
    lens = np.diff(np.asarray(cu_seqlens, dtype=np.int64))
    L = np.full((B, Hq, int(lens.max()) if B else 0), np.nan)
    for (b, h), (o, l) in zip(units, results):
        s = int(cu_seqlens[b])
        O[s:s + o.shape[0], h] = o
        L[b, h, :o.shape[0]] = l
    return O, L


def attention_rows(q: np.ndarray, k: np.ndarray, v: np.ndarray, *, causal: bool,
                   scale: float, picks: Iterable[Tuple[int, int, int]],
                   cu_seqlens: Optional[np.ndarray] = None):
    """The same definition, for a few ``(b, h, row)`` picks only.

    Used to check very large workloads row by row.  Returns O rows
    ``[P, d]`` and L ``[P]`` in the order of ``picks``.
    """
    picks = list(picks)
    O = np.empty((len(picks), v.shape[-1]), dtype=np.float64)
    L = np.empty(len(picks), dtype=np.float64)
    by_unit = {}
    for i, (b, h, r) in enumerate(picks):
        by_unit.setdefault((b, h), []).append((i, r))
    for (b, h), items in by_unit.items():
        qs, ks, vs = _slices(q, k, v, b, h, cu_seqlens)
        idx = [i for i, _ in items]
        rows = np.array([r for _, r in items], dtype=np.int64)
        if rows.size and (rows.min() < 0 or rows.max() >= qs.shape[0]):
            raise IndexError("row out of range")
        o, l = _head_rows(qs, ks, vs, causal, scale, rows)
        O[idx] = o
        L[idx] = l
    return O, L


def attention_bruteforce(q, k, v, *, causal: bool, scale: float):
    """Element-by-element attention with pure Python loops (tiny inputs).

    No maximum is subtracted: every weight is ``exp(scale * q_r . k_c)``
    summed with ``math.fsum``, so it checks the stabilised oracle through a
    different route.  Fixed layout only: q ``[B, Hq, Nq, d]``,
    k/v ``[B, Hkv, Nk, d]``; with Nq < Nk the queries are the last Nq
    tokens (query r sees keys up to r + Nk - Nq when causal), and a row that
    sees no key gets O = 0, L = -inf.  Returns nested lists O[b][h][r][j],
    L[b][h][r].
    """
    B, Hq, N, d = (len(q), len(q[0]), len(q[0][0]), len(q[0][0][0]))
    Hkv, Nk = len(k[0]), len(k[0][0])
    per_group = Hq // Hkv
    O, L = [], []
    for b in range(B):
        Ob, Lb = [], []
        for h in range(Hq):
            g = 0
            while not (g * per_group <= h < (g + 1) * per_group):
                g += 1
            Oh, Lh = [], []
            for r in range(N):
                last = min(r + Nk - N, Nk - 1) if causal else Nk - 1
                if last < 0:
                    Oh.append([0.0] * d)
                    Lh.append(-math.inf)
                    continue
                w = []
                for c in range(last + 1):
                    dot = math.fsum(float(q[b][h][r][i]) * float(k[b][g][c][i])
                                    for i in range(d))
                    w.append(math.exp(scale * dot))
                den = math.fsum(w)
                Oh.append([math.fsum(w[c] * float(v[b][g][c][j])
                                     for c in range(last + 1)) / den
                           for j in range(d)])
                Lh.append(math.log(den))
            Ob.append(Oh)
            Lb.append(Lh)
        O.append(Ob)
        L.append(Lb)
    return O, L


def attention_tiled_online(q, k, v, *, causal: bool, scale: float,
                           Br: int, Bc: int,
                           cu_seqlens: Optional[np.ndarray] = None):
    """The tiled method with an online softmax, in float64.

    Follows the method as the Kotaemon page lists it (method list, and the
    online maximum/normaliser update that follows): Q is cut into row blocks
    of ``Br``; for each row block, key/value blocks of ``Bc`` rows are taken
    in order; each block's scores update a running row maximum ``m`` and
    normaliser ``ell``, the accumulated output is rescaled by
    ``exp(m_old - m_new)``, and the block's ``P V`` is added.  At the end
    ``O = acc / ell`` and ``L = m + ln ell``.  exp(-inf) is taken as 0.
    Same layouts and return values as :func:`attention`.
    """
    O = np.empty(q.shape, dtype=np.float64)
    units = list(_units(q, k, cu_seqlens))
    if cu_seqlens is None:
        L = np.empty(q.shape[:3], dtype=np.float64)
    else:
        lens = np.diff(np.asarray(cu_seqlens, dtype=np.int64))
        L = np.full((len(lens), q.shape[1], int(lens.max())), np.nan)
    for b, h in units:
        qs, ks, vs = _slices(q, k, v, b, h, cu_seqlens)
        n = qs.shape[0]
        o = np.empty_like(qs)
        lse = np.empty(n)
        for i0 in range(0, n, Br):
            rows = np.arange(i0, min(i0 + Br, n))
            m = np.full(rows.size, -np.inf)
            ell = np.zeros(rows.size)
            acc = np.zeros((rows.size, vs.shape[1]))
            for j0 in range(0, n, Bc):
                cols = np.arange(j0, min(j0 + Bc, n))
                S = scale * (qs[rows] @ ks[cols].T)
                if causal:
                    S = np.where(cols[None, :] > rows[:, None], -np.inf, S)
                m_new = np.maximum(m, S.max(axis=1))
                safe = np.where(np.isneginf(m_new), 0.0, m_new)
                P = np.exp(S - safe[:, None])
                alpha = np.where(np.isneginf(m), 0.0, np.exp(m - safe))
                ell = alpha * ell + P.sum(axis=1)
                acc = alpha[:, None] * acc + P @ vs[cols]
                m = m_new
            o[rows] = acc / ell[:, None]
            lse[rows] = m + np.log(ell)
        if cu_seqlens is None:
            O[b, h] = o
            L[b, h] = lse
        else:
            s = int(cu_seqlens[b])
            O[s:s + n, h] = o
            L[b, h, :n] = lse
    return O, L


# ---------------------------------------------------------------------------
# Queries against a longer key/value sequence (chunked prefill).

def offset_mask(S: np.ndarray, rows: np.ndarray, cols: np.ndarray, offset: int) -> np.ndarray:
    """Causal mask when the ``nq`` queries are the last tokens of an
    ``nk``-token sequence: query row r is token ``r + offset`` of the
    sequence (``offset = nk - nq``) and sees keys ``c <= r + offset``."""
    return np.where(cols[None, :] > rows[:, None] + offset, -np.inf, S)


def _head_rows_qk(q: np.ndarray, k: np.ndarray, v: np.ndarray, causal: bool,
                  scale: float, rows: Optional[np.ndarray] = None):
    """One head of one sequence, nq queries against nk keys, by the
    definition.  Rows that see no key get O = 0 and L = -inf."""
    nq, nk = q.shape[0], k.shape[0]
    if rows is None:
        rows = np.arange(nq)
    rows = np.asarray(rows, dtype=np.int64)
    O = np.zeros((rows.size, v.shape[1]), dtype=np.float64)
    L = np.full(rows.size, -np.inf, dtype=np.float64)
    offset = nk - nq
    chunk = max(1, _CHUNK_BYTES // (8 * max(nk, 1)))
    cols = np.arange(nk)
    for s in range(0, rows.size, chunk):
        r = rows[s:s + chunk]
        seen = (np.minimum(r + offset, nk - 1) >= 0) if causal else np.full(r.size, nk > 0)
        if not seen.any():
            continue
        r_seen = r[seen]
        S = scores(q[r_seen], k, scale)                   # [R, nk]
        if causal:
            S = offset_mask(S, r_seen, cols, offset)
        P, m, ell = softmax_rows(S)
        idx = np.arange(s, s + r.size)[seen]
        O[idx] = combine(P, v)
        L[idx] = logsumexp_of(m, ell)
    return O, L


def _run_unit_qk(args):
    qs, ks, vs, causal, scale = args
    return _head_rows_qk(qs, ks, vs, causal, scale)


def attention_qk(q: np.ndarray, k: np.ndarray, v: np.ndarray, *, causal: bool,
                 scale: float, cu_seqlens_q: Optional[np.ndarray] = None,
                 cu_seqlens_k: Optional[np.ndarray] = None, workers: int = 1):
    """Attention of nq queries against nk keys per sequence (chunked
    prefill): returns ``(O, L)`` in float64.

    The queries are the last nq tokens of an nk-token sequence, so with
    ``causal`` query row r sees keys ``c <= r + nk - nq`` (bottom-right
    alignment).  This is the manual chunking recipe of the French HolySheep
    article ("Erreurs courantes", item 1): the query chunk ``[i, i+c)``
    attends to the key prefix ``[0, i+c)``.  When nq = nk it is
    :func:`attention`.  Rows that see no key (causal with nq > nk, or
    nk = 0) get O = 0 and L = -inf.

    Fixed layout: q ``[B, Hq, Nq, d]``, k/v ``[B, Hkv, Nk, d]``; L is
    ``[B, Hq, Nq]``.  Varlen (both offset arrays given): q ``[Tq, Hq, d]``,
    k/v ``[Tk, Hkv, d]``; L is ``[B, Hq, max nq]`` with NaN past each
    sequence's query count.
    """
    if (cu_seqlens_q is None) != (cu_seqlens_k is None):
        raise ValueError("give both cu_seqlens_q and cu_seqlens_k, or neither")
    Hq, Hkv = q.shape[1], k.shape[1]
    if cu_seqlens_q is None:
        B = q.shape[0]
        units = [(b, h) for b in range(B) for h in range(Hq)]
        jobs = [(q[b, h], k[b, _group(h, Hq, Hkv)], v[b, _group(h, Hq, Hkv)], causal, scale)
                for b, h in units]
    else:
        B = len(cu_seqlens_q) - 1
        if len(cu_seqlens_k) != B + 1:
            raise ValueError("cu_seqlens_q and cu_seqlens_k differ in length")
        units = [(b, h) for b in range(B) for h in range(Hq)]
        jobs = []
        for b, h in units:
            sq, eq = int(cu_seqlens_q[b]), int(cu_seqlens_q[b + 1])
            sk, ek = int(cu_seqlens_k[b]), int(cu_seqlens_k[b + 1])
            g = _group(h, Hq, Hkv)
            jobs.append((q[sq:eq, h], k[sk:ek, g], v[sk:ek, g], causal, scale))
    if workers <= 1:
        results = [_run_unit_qk(j) for j in jobs]
    else:
        with ProcessPoolExecutor(max_workers=workers, initializer=_one_blas_thread) as ex:
            results = list(ex.map(_run_unit_qk, jobs, chunksize=1))
    O = np.empty(q.shape, dtype=np.float64)
    if cu_seqlens_q is None:
        L = np.empty(q.shape[:3], dtype=np.float64)
        for (b, h), (o, l) in zip(units, results):
            O[b, h] = o
            L[b, h] = l
        return O, L
    lens = np.diff(np.asarray(cu_seqlens_q, dtype=np.int64))
    L = np.full((B, Hq, int(lens.max()) if B else 0), np.nan)
    for (b, h), (o, l) in zip(units, results):
        s = int(cu_seqlens_q[b])
        O[s:s + o.shape[0], h] = o
        L[b, h, :o.shape[0]] = l
    return O, L


def pair_count(nq: int, nk: int, causal: bool) -> int:
    """Visible (query, key) pairs of one head of one sequence with nq
    queries at the end of an nk-token sequence."""
    if not causal:
        return nq * nk
    off = nk - nq
    return sum(max(0, min(r + off + 1, nk)) for r in range(nq))


# ---------------------------------------------------------------------------
# Block-sparse attention.
#
# The Kotaemon page names block-sparse attention only as a direction of the
# method, with no layout.  Reading taken here: a 0/1 mask over blocks of
# ``block`` query rows x ``block`` keys of the (query row, key) grid of each
# sequence and head admits or removes whole blocks of scores; removed scores
# are -inf, exactly as the causal mask removes single scores.  Everything
# else is the definition above.

def sparse_allowed(bm: np.ndarray, rows: np.ndarray, nk: int, block: int, causal: bool,
                   offset: int) -> np.ndarray:
    """Visibility of keys 0..nk-1 for the given query rows: the block of
    (row, key) is admitted by ``bm`` [row blocks, key blocks], and with
    ``causal`` the key is at most the row's position ``row + offset``."""
    cols = np.arange(nk)
    allowed = bm[rows // block][:, cols // block] != 0
    if causal:
        allowed &= cols[None, :] <= rows[:, None] + offset
    return allowed


def _head_rows_sparse(q: np.ndarray, k: np.ndarray, v: np.ndarray, bm: np.ndarray,
                      causal: bool, scale: float, block: int):
    """One head of one sequence under the block mask ``bm``, by the
    definition.  Rows that see no key get O = 0 and L = -inf."""
    nq, nk = q.shape[0], k.shape[0]
    O = np.zeros((nq, v.shape[1]), dtype=np.float64)
    L = np.full(nq, -np.inf, dtype=np.float64)
    chunk = max(1, _CHUNK_BYTES // (8 * max(nk, 1)))
    for s in range(0, nq, chunk):
        r = np.arange(s, min(nq, s + chunk))
        allowed = sparse_allowed(bm, r, nk, block, causal, nk - nq)
        seen = allowed.any(axis=1)
        if not seen.any():
            continue
        rs = r[seen]
        S = np.where(allowed[seen], scores(q[rs], k, scale), -np.inf)
        P, m, ell = softmax_rows(S)
        O[rs] = combine(P, v)
        L[rs] = logsumexp_of(m, ell)
    return O, L


def _run_unit_sparse(args):
    return _head_rows_sparse(*args)


def attention_block_sparse(q: np.ndarray, k: np.ndarray, v: np.ndarray,
                           block_mask: np.ndarray, *, causal: bool, scale: float,
                           block: int = 64, cu_seqlens_q: Optional[np.ndarray] = None,
                           cu_seqlens_k: Optional[np.ndarray] = None, workers: int = 1):
    """Block-sparse attention: returns ``(O, L)`` in float64.

    ``block_mask`` has shape ``[Bm, Hm, ceil(Nq/block), ceil(Nk/block)]``
    with Bm in {1, B} and Hm in {1, Hq} (1 = the same mask for every
    sequence / query head); entry [b, h, i, j] != 0 admits the scores of
    query rows [i*block, (i+1)*block) against keys [j*block, (j+1)*block)
    of sequence b, head h (row and key indices within the sequence; the
    queries are the last nq tokens, as in :func:`attention_qk`).  With
    ``causal`` the causal mask applies as well.  Rows that see no key get
    O = 0 and L = -inf.  Layouts as :func:`attention_qk`.
    """
    if (cu_seqlens_q is None) != (cu_seqlens_k is None):
        raise ValueError("give both cu_seqlens_q and cu_seqlens_k, or neither")
    Hq, Hkv = q.shape[1], k.shape[1]
    B = q.shape[0] if cu_seqlens_q is None else len(cu_seqlens_q) - 1
    bm_all = np.asarray(block_mask)
    if bm_all.ndim != 4 or bm_all.shape[0] not in (1, B) or bm_all.shape[1] not in (1, Hq):
        raise ValueError("block_mask must be [1 or B, 1 or Hq, row blocks, key blocks]")

    def mask_of(b, h, nq, nk):
        m = bm_all[b if bm_all.shape[0] > 1 else 0, h if bm_all.shape[1] > 1 else 0]
        need = (-(-nq // block), -(-nk // block))
        if m.shape[0] < need[0] or m.shape[1] < need[1]:
            raise ValueError("block_mask too small for the sequence")
        return m[:need[0], :need[1]]

    units = [(b, h) for b in range(B) for h in range(Hq)]
    jobs = []
    for b, h in units:
        g = _group(h, Hq, Hkv)
        if cu_seqlens_q is None:
            qs, ks, vs = q[b, h], k[b, g], v[b, g]
        else:
            sq, eq = int(cu_seqlens_q[b]), int(cu_seqlens_q[b + 1])
            sk, ek = int(cu_seqlens_k[b]), int(cu_seqlens_k[b + 1])
            qs, ks, vs = q[sq:eq, h], k[sk:ek, g], v[sk:ek, g]
        jobs.append((qs, ks, vs, mask_of(b, h, qs.shape[0], ks.shape[0]), causal, scale, block))
    if workers <= 1:
        results = [_run_unit_sparse(j) for j in jobs]
    else:
        with ProcessPoolExecutor(max_workers=workers, initializer=_one_blas_thread) as ex:
            results = list(ex.map(_run_unit_sparse, jobs, chunksize=1))
    O = np.empty(q.shape, dtype=np.float64)
    if cu_seqlens_q is None:
        L = np.empty(q.shape[:3], dtype=np.float64)
        for (b, h), (o, l) in zip(units, results):
            O[b, h] = o
            L[b, h] = l
        return O, L
    lens = np.diff(np.asarray(cu_seqlens_q, dtype=np.int64))
    L = np.full((B, Hq, int(lens.max()) if B else 0), np.nan)
    for (b, h), (o, l) in zip(units, results):
        s = int(cu_seqlens_q[b])
        O[s:s + o.shape[0], h] = o
        L[b, h, :o.shape[0]] = l
    return O, L


def sparse_pair_count(bm: np.ndarray, nq: int, nk: int, causal: bool, block: int = 64) -> int:
    """Visible (query, key) pairs of one head of one sequence under the
    block mask ``bm`` [ceil(nq/block), ceil(nk/block)]."""
    total = 0
    for s in range(0, nq, block):
        r = np.arange(s, min(nq, s + block))
        total += int(sparse_allowed(bm, r, nk, block, causal, nk - nq).sum())
    return total


# ---------------------------------------------------------------------------
# Backward pass: gradients of the forward map.

def _head_backward(q, k, v, do, causal, scale):
    """Gradients of one head of one sequence, by the chain rule written out.

    With S = scale * q k^T (masked), P = softmax(S) row-wise and O = P v:
      dV = P^T dO,   dP = dO v^T,
      dS = P * (dP - D) with D_r = sum_c P_rc dP_rc = sum_j dO_rj O_rj,
      dQ = scale * dS k,   dK = scale * dS^T q.
    Rows are taken in chunks (each complete); dK and dV sum over them.
    """
    n, d = q.shape
    dq = np.empty_like(q)
    dk = np.zeros_like(k)
    dv = np.zeros_like(v)
    chunk = max(1, _CHUNK_BYTES // (8 * max(n, 1)))
    cols = np.arange(n)
    for s in range(0, n, chunk):
        r = np.arange(s, min(s + chunk, n))
        S = scores(q[r], k, scale)
        if causal:
            S = causal_mask(S, r, cols)
        P, _, _ = softmax_rows(S)
        O = combine(P, v)
        dv += P.T @ do[r]
        dP = do[r] @ v.T
        D = np.sum(do[r] * O, axis=1, keepdims=True)
        dS = P * (dP - D)
        dq[r] = scale * (dS @ k)
        dk += scale * (dS.T @ q[r])
    return dq, dk, dv


def _run_unit_bwd(args):
    return _head_backward(*args)


def attention_backward(q, k, v, do, *, causal: bool, scale: float,
                       cu_seqlens: Optional[np.ndarray] = None, workers: int = 1):
    """Gradients (dQ, dK, dV) of sum(O * dO) for the attention forward of
    :func:`attention`, in float64 (same layouts as q, k, v).

    The Kotaemon page describes the method as tiling plus recomputation (the
    paragraph after the formula): a backward pass recomputes the score
    blocks from the saved per-row statistics instead of keeping the n x n
    matrix.  What it must produce is fixed by calculus: the derivative of
    the forward map.  For grouped-query attention a K/V head's gradient is
    the sum over the query heads that read it.
    """
    units = list(_units(q, k, cu_seqlens))
    Hq, Hkv = q.shape[1], k.shape[1]
    jobs = []
    for b, h in units:
        qs, ks, vs = _slices(q, k, v, b, h, cu_seqlens)
        if cu_seqlens is None:
            dos = do[b, h]
        else:
            dos = do[int(cu_seqlens[b]):int(cu_seqlens[b + 1]), h]
        jobs.append((qs, ks, vs, dos, causal, scale))
    if workers <= 1:
        results = [_run_unit_bwd(j) for j in jobs]
    else:
        with ProcessPoolExecutor(max_workers=workers, initializer=_one_blas_thread) as ex:
            results = list(ex.map(_run_unit_bwd, jobs, chunksize=1))
    dQ = np.empty(q.shape, dtype=np.float64)
    dK = np.zeros(k.shape, dtype=np.float64)
    dV = np.zeros(v.shape, dtype=np.float64)
    for (b, h), (dq, dk, dv) in zip(units, results):
        g = _group(h, Hq, Hkv)
        if cu_seqlens is None:
            dQ[b, h] = dq
            dK[b, g] += dk
            dV[b, g] += dv
        else:
            s, e = int(cu_seqlens[b]), int(cu_seqlens[b + 1])
            dQ[s:e, h] = dq
            dK[s:e, g] += dk
            dV[s:e, g] += dv
    return dQ, dK, dV


def unit_flops(n: int, d: int, causal: bool) -> float:
    """Algorithmic FLOP of one head of one sequence: the two contractions
    over the visible (query, key) pairs, 2*d each."""
    pairs = n * (n + 1) // 2 if causal else n * n
    return 4.0 * d * pairs


def default_workers() -> int:
    try:
        return len(os.sched_getaffinity(0))
    except AttributeError:  # pragma: no cover
        return os.cpu_count() or 1


__all__ = [
    "attention", "attention_rows", "attention_bruteforce",
    "attention_tiled_online", "attention_qk", "attention_backward", "pair_count",
    "softmax_rows",
    "visible_keys", "unit_flops", "default_workers",
]
