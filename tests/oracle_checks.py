"""Pins of the CPU oracle: facts fixed by the pages and by mathematics.

Each ``check_*`` function takes an attention callable with the oracle's
signature ``attn(q, k, v, *, causal, scale, cu_seqlens=None) -> (O, L)``
and returns the largest deviation it finds from a fact that does not come
from the oracle itself.  The real oracle must score at or below ``TOL`` on
every check; each planted mistake (see ``test_oracle_pins.py``) must exceed
it on at least one.
"""
from __future__ import annotations

import math
import os

import numpy as np

TOL = 1e-10
GOLDEN = os.path.join(os.path.dirname(__file__), "golden", "hand_2x2.txt")


def _rng(seed):
    return np.random.default_rng(seed)


def _rand(seed, B=2, Hq=4, Hkv=2, N=7, d=5):
    r = _rng(seed)
    return (r.standard_normal((B, Hq, N, d)), r.standard_normal((B, Hkv, N, d)),
            r.standard_normal((B, Hkv, N, d)))


def _err(a, b):
    a = np.asarray(a, dtype=np.float64)
    b = np.asarray(b, dtype=np.float64)
    if a.shape != b.shape:
        return math.inf
    if not (np.isfinite(a).all() and np.isfinite(b).all()):
        return math.inf
    return float(np.max(np.abs(a - b))) if a.size else 0.0


def check_golden(attn):
    """The hand-worked 2x2 example (tests/golden/hand_2x2.txt)."""
    q = np.array([[[[math.log(3), 0.0], [0.0, math.log(7)]]]])
    k = np.array([[[[1.0, 0.0], [0.0, 1.0]]]])
    v = np.array([[[[4.0, 0.0], [0.0, 8.0]]]])
    worst = 0.0
    with open(GOLDEN) as f:
        rows = [ln.split() for ln in f if ln.strip() and not ln.startswith("#")]
    for causal in (False, True):
        O, L = attn(q, k, v, causal=causal, scale=1.0)
        for c, r, o0, o1, lexpr in rows:
            if int(c) != int(causal):
                continue
            r = int(r)
            Lexp = math.log(float(lexpr[2:]))
            worst = max(worst, abs(O[0, 0, r, 0] - float(o0)),
                        abs(O[0, 0, r, 1] - float(o1)), abs(L[0, 0, r] - Lexp))
    return worst


def check_bruteforce(attn):
    """Pure-Python, no-max-subtraction sums with math.fsum (tiny inputs)."""
    from oracle import attention_bruteforce
    worst = 0.0
    for causal in (False, True):
        q, k, v = _rand(11 + causal)
        O, L = attn(q, k, v, causal=causal, scale=0.41)
        Ob, Lb = attention_bruteforce(q.tolist(), k.tolist(), v.tolist(),
                                      causal=causal, scale=0.41)
        worst = max(worst, _err(O, Ob), _err(L, Lb))
    return worst


def check_library(attn):
    """torch's scaled_dot_product_attention (the routine the French
    HolySheep article calls) and torch.logsumexp, in float64 on the CPU."""
    import torch
    import torch.nn.functional as F
    worst = 0.0
    for causal in (False, True):
        q, k, v = _rand(21 + causal, B=2, Hq=6, Hkv=2, N=37, d=16)
        scale = 0.23
        O, L = attn(q, k, v, causal=causal, scale=scale)
        tq, tk, tv = (torch.from_numpy(x) for x in (q, k, v))
        To = F.scaled_dot_product_attention(tq, tk, tv, is_causal=causal,
                                            scale=scale, enable_gqa=True)
        kr = tk.repeat_interleave(q.shape[1] // k.shape[1], dim=1)
        S = scale * torch.matmul(tq, kr.transpose(-1, -2))
        if causal:
            n = q.shape[2]
            S = S.masked_fill(torch.ones(n, n, dtype=torch.bool).triu(1), -math.inf)
        TL = torch.logsumexp(S, dim=-1)
        worst = max(worst, _err(O, To.numpy()), _err(L, TL.numpy()))
    return worst


def check_identical_keys(attn):
    """All keys equal: every visible key gets the same weight, so O is the
    mean of the visible values and L = scale*q.k + ln(#visible).  With
    q = 0 as well, L = ln(#visible)."""
    worst = 0.0
    r = _rng(31)
    B, Hq, Hkv, N, d = 1, 4, 2, 9, 6
    for causal in (False, True):
        for zero_q in (False, True):
            q = np.zeros((B, Hq, N, d)) if zero_q else r.standard_normal((B, Hq, N, d))
            k = np.broadcast_to(r.standard_normal((B, Hkv, 1, d)), (B, Hkv, N, d)).copy()
            v = r.standard_normal((B, Hkv, N, d))
            scale = 0.7
            O, L = attn(q, k, v, causal=causal, scale=scale)
            for h in range(Hq):
                g = h // (Hq // Hkv)
                n_vis = np.arange(1, N + 1) if causal else np.full(N, N)
                mean = (np.cumsum(v[0, g], axis=0) / np.arange(1, N + 1)[:, None]
                        if causal else np.broadcast_to(v[0, g].mean(axis=0), (N, d)))
                Lx = scale * (q[0, h] @ k[0, g, 0]) + np.log(n_vis)
                worst = max(worst, _err(O[0, h], mean), _err(L[0, h], Lx))
    return worst


def check_causal_row0(attn):
    """Causal row 0 sees only key 0: O_0 = V_0 and L_0 = scale*q_0.k_0."""
    q, k, v = _rand(41)
    scale = 0.9
    O, L = attn(q, k, v, causal=True, scale=scale)
    worst = 0.0
    for b in range(q.shape[0]):
        for h in range(q.shape[1]):
            g = h // (q.shape[1] // k.shape[1])
            worst = max(worst, _err(O[b, h, 0], v[b, g, 0]),
                        abs(L[b, h, 0] - scale * math.fsum(q[b, h, 0] * k[b, g, 0])))
    return worst


def check_tiled_online(attn):
    """The tiled method with the online maximum/normaliser update gives the
    materialised result (block sizes that do and do not divide N)."""
    from oracle import attention_tiled_online
    worst = 0.0
    q, k, v = _rand(51, B=1, Hq=4, Hkv=2, N=101, d=8)
    for causal in (False, True):
        O, L = attn(q, k, v, causal=causal, scale=0.3)
        for Br, Bc in ((48, 40), (16, 16), (7, 13), (128, 64), (1, 1)):
            Ot, Lt = attention_tiled_online(q, k, v, causal=causal, scale=0.3, Br=Br, Bc=Bc)
            worst = max(worst, _err(O, Ot), _err(L, Lt))
    return worst


def check_prefix(attn):
    """Causal row r equals the last row of non-causal attention over the
    prefix [0, r]."""
    q, k, v = _rand(61, B=1, Hq=2, Hkv=1, N=12, d=4)
    O, L = attn(q, k, v, causal=True, scale=0.5)
    worst = 0.0
    for r in range(q.shape[2]):
        Op, Lp = attn(q[:, :, :r + 1], k[:, :, :r + 1], v[:, :, :r + 1],
                      causal=False, scale=0.5)
        worst = max(worst, _err(O[:, :, r], Op[:, :, r]), _err(L[:, :, r], Lp[:, :, r]))
    return worst


def check_permutation(attn):
    """Non-causal: permuting key/value rows together changes nothing."""
    q, k, v = _rand(71, N=10)
    perm = _rng(72).permutation(10)
    O, L = attn(q, k, v, causal=False, scale=0.6)
    Op, Lp = attn(q, k[:, :, perm], v[:, :, perm], causal=False, scale=0.6)
    return max(_err(O, Op), _err(L, Lp))


def check_shift(attn):
    """Adding w to every key adds scale*q.w to a row's scores: O unchanged,
    L shifted by scale*q.w."""
    q, k, v = _rand(81, N=8, d=5)
    w = _rng(82).standard_normal(5)
    worst = 0.0
    for causal in (False, True):
        O, L = attn(q, k, v, causal=causal, scale=0.8)
        Os, Ls = attn(q, k + w, v, causal=causal, scale=0.8)
        worst = max(worst, _err(O, Os), _err(Ls - L, 0.8 * (q @ w)))
    return worst


def check_gqa_equals_repeated(attn):
    """GQA equals multi-head attention with each K/V head repeated for the
    query heads of its group (contiguous groups)."""
    q, k, v = _rand(91, B=2, Hq=6, Hkv=3, N=9, d=4)
    worst = 0.0
    for causal in (False, True):
        O, L = attn(q, k, v, causal=causal, scale=0.4)
        Om, Lm = attn(q, np.repeat(k, 2, axis=1), np.repeat(v, 2, axis=1),
                      causal=causal, scale=0.4)
        worst = max(worst, _err(O, Om), _err(L, Lm))
    return worst


def check_varlen_equals_fixed(attn):
    """Packed sequences give the same result as each sequence run alone."""
    r = _rng(101)
    lens = [5, 1, 9, 3]
    Hq, Hkv, d = 4, 2, 3
    T = sum(lens)
    q, k, v = (r.standard_normal((T, H, d)) for H in (Hq, Hkv, Hkv))
    cu = np.concatenate([[0], np.cumsum(lens)]).astype(np.int32)
    worst = 0.0
    for causal in (False, True):
        O, L = attn(q, k, v, causal=causal, scale=0.5, cu_seqlens=cu)
        for b, n in enumerate(lens):
            s = cu[b]
            sl = slice(s, s + n)
            Of, Lf = attn(q[sl].transpose(1, 0, 2)[None], k[sl].transpose(1, 0, 2)[None],
                          v[sl].transpose(1, 0, 2)[None], causal=causal, scale=0.5)
            worst = max(worst, _err(O[sl], Of[0].transpose(1, 0, 2)),
                        _err(L[b, :, :n], Lf[0]))
            if not np.isnan(L[b, :, n:]).all():
                worst = math.inf
    return worst


def check_large_scale(attn):
    """A huge scale must not overflow: the softmax becomes the argmax."""
    q, k, v = _rand(111, B=1, Hq=2, Hkv=2, N=6, d=4)
    O, L = attn(q, k, v, causal=False, scale=1e3)
    worst = 0.0
    for h in range(2):
        s = q[0, h] @ k[0, h].T
        top = np.argmax(s, axis=1)
        worst = max(worst, _err(O[0, h], v[0, h][top]),
                    _err(L[0, h] / 1e3, s.max(axis=1)))
    return worst if np.isfinite(O).all() else math.inf


def check_convex(attn):
    """Each output is a convex combination of the visible value rows."""
    q, k, v = _rand(121, N=11)
    worst = 0.0
    for causal in (False, True):
        O, _ = attn(q, k, v, causal=causal, scale=1.3)
        for b in range(2):
            for h in range(4):
                g = h // 2
                for r in range(11):
                    vis = v[b, g, :r + 1] if causal else v[b, g]
                    lo, hi = vis.min(axis=0), vis.max(axis=0)
                    worst = max(worst, float(np.max(lo - O[b, h, r])),
                                float(np.max(O[b, h, r] - hi)), 0.0)
    return worst


CHECKS = [
    check_golden, check_bruteforce, check_library, check_identical_keys,
    check_causal_row0, check_tiled_online, check_prefix, check_permutation,
    check_shift, check_gqa_equals_repeated, check_varlen_equals_fixed,
    check_large_scale, check_convex,
]


# ---------------------------------------------------------------------------
# Queries against a longer key/value sequence (chunked prefill).  Each check
# takes ``attn_qk(q, k, v, *, causal, scale, cu_seqlens_q=None,
# cu_seqlens_k=None) -> (O, L)``.

def _rand_qk(seed, B=2, Hq=4, Hkv=2, Nq=5, Nk=11, d=6):
    r = _rng(seed)
    return (r.standard_normal((B, Hq, Nq, d)), r.standard_normal((B, Hkv, Nk, d)),
            r.standard_normal((B, Hkv, Nk, d)))


def check_qk_chunk_recipe(attn_qk):
    """The manual chunking recipe (French HolySheep article, "Erreurs
    courantes", item 1): the query chunk [i, i+c) of a sequence, attending to
    the key prefix [0, i+c), gives rows i .. i+c-1 of attention over the
    whole sequence (computed by the pinned full-sequence oracle)."""
    from oracle import attention
    q, k, v = _rand(61, B=2, Hq=4, Hkv=2, N=13, d=5)
    worst = 0.0
    for causal in (True, False):
        Of, Lf = attention(q, k, v, causal=causal, scale=0.37)
        for i, c in ((0, 13), (0, 4), (4, 5), (9, 4), (12, 1)):
            end = i + c if causal else 13
            O, L = attn_qk(q[:, :, i:i + c], k[:, :, :end], v[:, :, :end],
                           causal=causal, scale=0.37)
            worst = max(worst, _err(O, Of[:, :, i:i + c]), _err(L, Lf[:, :, i:i + c]))
    return worst


def check_qk_bruteforce(attn_qk):
    """Pure-Python sums (no max subtraction) with the queries at the end of
    a longer key sequence."""
    from oracle import attention_bruteforce
    worst = 0.0
    for causal in (False, True):
        q, k, v = _rand_qk(63 + causal)
        O, L = attn_qk(q, k, v, causal=causal, scale=0.52)
        Ob, Lb = attention_bruteforce(q.tolist(), k.tolist(), v.tolist(),
                                      causal=causal, scale=0.52)
        worst = max(worst, _err(O, Ob), _err(L, Lb))
    return worst


def check_qk_library(attn_qk):
    """torch's scaled_dot_product_attention with an explicit boolean mask
    (key c visible to query r iff c <= r + Nk - Nq), float64 on the CPU."""
    import torch
    import torch.nn.functional as F
    worst = 0.0
    for causal in (False, True):
        q, k, v = _rand_qk(65 + causal, B=2, Hq=6, Hkv=3, Nq=19, Nk=45, d=16)
        O, L = attn_qk(q, k, v, causal=causal, scale=0.19)
        tq, tk, tv = (torch.from_numpy(x) for x in (q, k, v))
        Nq, Nk = q.shape[2], k.shape[2]
        vis = torch.arange(Nk)[None, :] <= torch.arange(Nq)[:, None] + (Nk - Nq)
        mask = vis if causal else None
        kr = tk.repeat_interleave(2, dim=1)
        vr = tv.repeat_interleave(2, dim=1)
        To = F.scaled_dot_product_attention(tq, kr, vr, attn_mask=mask, scale=0.19)
        S = 0.19 * torch.matmul(tq, kr.transpose(-1, -2))
        if causal:
            S = S.masked_fill(~vis, -math.inf)
        worst = max(worst, _err(O, To.numpy()), _err(L, torch.logsumexp(S, -1).numpy()))
    return worst


def check_qk_no_visible_key(attn_qk):
    """Causal with more queries than keys: query r sees keys up to
    r + Nk - Nq, so the first Nq - Nk rows see none (O = 0, L = -inf) and
    the rest are the Nk-token causal attention (pinned full oracle)."""
    from oracle import attention
    q, k, v = _rand_qk(67, Nq=9, Nk=4)
    O, L = attn_qk(q, k, v, causal=True, scale=0.8)
    worst = 0.0
    if not (np.isneginf(L[:, :, :5]).all()):
        return math.inf
    worst = max(worst, float(np.abs(O[:, :, :5]).max()))
    Of, Lf = attention(q[:, :, 5:], k, v, causal=True, scale=0.8)
    return max(worst, _err(O[:, :, 5:], Of), _err(L[:, :, 5:], Lf))


def check_qk_varlen(attn_qk):
    """Packed sequences with their own query and key counts = each sequence
    alone; L rows past a sequence's query count stay NaN."""
    r = _rng(69)
    Hq, Hkv, d = 4, 2, 5
    nq, nk = [3, 1, 6], [7, 1, 6]
    cq = np.concatenate([[0], np.cumsum(nq)]).astype(np.int32)
    ck = np.concatenate([[0], np.cumsum(nk)]).astype(np.int32)
    q = r.standard_normal((cq[-1], Hq, d))
    k = r.standard_normal((ck[-1], Hkv, d))
    v = r.standard_normal((ck[-1], Hkv, d))
    worst = 0.0
    for causal in (False, True):
        O, L = attn_qk(q, k, v, causal=causal, scale=0.6, cu_seqlens_q=cq, cu_seqlens_k=ck)
        for b in range(3):
            qs = q[cq[b]:cq[b + 1]].transpose(1, 0, 2)[None]
            ks = k[ck[b]:ck[b + 1]].transpose(1, 0, 2)[None]
            vs = v[ck[b]:ck[b + 1]].transpose(1, 0, 2)[None]
            Ob, Lb = attn_qk(qs, ks, vs, causal=causal, scale=0.6)
            worst = max(worst, _err(O[cq[b]:cq[b + 1]], Ob[0].transpose(1, 0, 2)),
                        _err(L[b, :, :nq[b]], Lb[0]))
            if not np.isnan(L[b, :, nq[b]:]).all():
                return math.inf
    return worst


QK_CHECKS = [check_qk_chunk_recipe, check_qk_bruteforce, check_qk_library,
             check_qk_no_visible_key, check_qk_varlen]


# ---------------------------------------------------------------------------
# Block-sparse attention.  Each check takes ``attn_sp(q, k, v, block_mask, *,
# causal, scale, block=64, cu_seqlens_q=None, cu_seqlens_k=None) -> (O, L)``.

def _elementwise(bm2, nq, nk, block):
    """The element mask of a block mask, by repeating every entry into a
    block x block square (numpy kron) and cutting to nq x nk."""
    return np.kron(bm2 != 0, np.ones((block, block), dtype=bool))[:nq, :nk]


def _same_inf(a, b):
    """-inf in the same places of two L arrays; 0 or inf as an error."""
    return 0.0 if np.array_equal(np.isneginf(a), np.isneginf(b)) else math.inf


def _finite_err(a, b):
    fa, fb = np.where(np.isneginf(a), 0.0, a), np.where(np.isneginf(b), 0.0, b)
    return max(_same_inf(a, b), _err(fa, fb))


def check_sparse_all_ones(attn_sp):
    """A mask that admits every block is plain attention (the pinned
    query/key oracle), fixed and packed, with and without causal, with
    more keys than queries, at block sizes 4 and 64."""
    from oracle import attention_qk
    worst = 0.0
    for causal in (False, True):
        for (nq, nk, blk) in ((13, 13, 4), (5, 11, 4), (70, 70, 64), (33, 90, 64)):
            q, k, v = _rand_qk(81 + nq, B=2, Hq=4, Hkv=2, Nq=nq, Nk=nk, d=5)
            bm = np.ones((1, 1, -(-nq // blk), -(-nk // blk)), np.uint8)
            O, L = attn_sp(q, k, v, bm, causal=causal, scale=0.41, block=blk)
            Oq, Lq = attention_qk(q, k, v, causal=causal, scale=0.41)
            worst = max(worst, _err(O, Oq), _err(L, Lq))
    r = _rng(82)
    nq, nk = [3, 1, 6], [7, 1, 6]
    cq = np.concatenate([[0], np.cumsum(nq)]).astype(np.int32)
    ck = np.concatenate([[0], np.cumsum(nk)]).astype(np.int32)
    q = r.standard_normal((cq[-1], 4, 5))
    k, v = r.standard_normal((ck[-1], 2, 5)), r.standard_normal((ck[-1], 2, 5))
    for causal in (False, True):
        O, L = attn_sp(q, k, v, np.ones((3, 4, 2, 2), np.uint8), causal=causal, scale=0.6,
                       block=4, cu_seqlens_q=cq, cu_seqlens_k=ck)
        Oq, Lq = attention_qk(q, k, v, causal=causal, scale=0.6, cu_seqlens_q=cq,
                              cu_seqlens_k=ck)
        worst = max(worst, _err(O, Oq), _err(np.nan_to_num(L, nan=7.0),
                                              np.nan_to_num(Lq, nan=7.0)))
    return worst


def check_sparse_library(attn_sp):
    """torch's scaled_dot_product_attention, float64 on the CPU, with the
    block mask expanded to an explicit boolean mask (numpy kron) and
    combined with the bottom-right causal mask; a different random mask per
    sequence and query head; every row keeps key block 0 so that no row is
    empty (the library returns NaN there)."""
    import torch
    import torch.nn.functional as F
    worst = 0.0
    r = _rng(83)
    B, Hq, Hkv, Nq, Nk, d, blk = 2, 6, 3, 11, 17, 16, 3
    for causal in (False, True):
        q, k, v = _rand_qk(84 + causal, B=B, Hq=Hq, Hkv=Hkv, Nq=Nq, Nk=Nk, d=d)
        bm = (r.random((B, Hq, -(-Nq // blk), -(-Nk // blk))) < 0.5).astype(np.uint8)
        bm[..., 0] = 1
        O, L = attn_sp(q, k, v, bm, causal=causal, scale=0.23, block=blk)
        vis = np.stack([np.stack([_elementwise(bm[b, h], Nq, Nk, blk) for h in range(Hq)])
                        for b in range(B)])
        if causal:
            vis &= np.arange(Nk)[None, :] <= np.arange(Nq)[:, None] + (Nk - Nq)
        tq, tk, tv = (torch.from_numpy(x) for x in (q, k, v))
        kr = tk.repeat_interleave(Hq // Hkv, dim=1)
        vr = tv.repeat_interleave(Hq // Hkv, dim=1)
        tm = torch.from_numpy(vis)
        To = F.scaled_dot_product_attention(tq, kr, vr, attn_mask=tm, scale=0.23)
        S = (0.23 * torch.matmul(tq, kr.transpose(-1, -2))).masked_fill(~tm, -math.inf)
        worst = max(worst, _err(O, To.numpy()), _err(L, torch.logsumexp(S, -1).numpy()))
    return worst


def check_sparse_bruteforce(attn_sp):
    """Pure-Python sums over the admitted (row, key) pairs, no maximum
    subtracted, on tiny inputs whose masks leave some rows with no key
    (O = 0, L = -inf there)."""
    r = _rng(85)
    B, Hq, Hkv, Nq, Nk, d, blk = 1, 2, 1, 5, 7, 3, 2
    worst = 0.0
    for causal in (False, True):
        q, k, v = _rand_qk(86 + causal, B=B, Hq=Hq, Hkv=Hkv, Nq=Nq, Nk=Nk, d=d)
        bm = (r.random((B, Hq, 3, 4)) < 0.5).astype(np.uint8)
        bm[0, 0, 1, :] = 0                       # rows 2, 3 of head 0 see nothing
        bm[0, 1, 0, :] = 1
        O, L = attn_sp(q, k, v, bm, causal=causal, scale=0.7, block=blk)
        for h in range(Hq):
            for i in range(Nq):
                keys = [c for c in range(Nk) if bm[0, h, i // blk, c // blk]
                        and (not causal or c <= i + Nk - Nq)]
                if not keys:
                    if not (L[0, h, i] == -math.inf and not np.any(O[0, h, i])):
                        return math.inf
                    continue
                w = [math.exp(0.7 * sum(q[0, h, i, t] * k[0, 0, c, t] for t in range(d)))
                     for c in keys]
                tot = math.fsum(w)
                for t in range(d):
                    o = math.fsum(wc * v[0, 0, c, t] for wc, c in zip(w, keys)) / tot
                    worst = max(worst, abs(O[0, h, i, t] - o))
                worst = max(worst, abs(L[0, h, i] - math.log(tot)))
    return worst


def check_sparse_removed_key_blocks(attn_sp):
    """Without causal, a mask that admits the same key blocks for every row
    block is attention over those keys alone (the pinned query/key oracle
    on the gathered K and V)."""
    from oracle import attention_qk
    q, k, v = _rand_qk(87, B=2, Hq=4, Hkv=2, Nq=9, Nk=22, d=4)
    keep_blocks = np.array([1, 0, 1, 1, 0, 1], np.uint8)      # blocks of 4 keys
    bm = np.broadcast_to(keep_blocks, (1, 1, 3, 6)).copy()
    O, L = attn_sp(q, k, v, bm, causal=False, scale=0.5, block=4)
    keep = np.repeat(keep_blocks != 0, 4)[:22]
    Oq, Lq = attention_qk(q, k[:, :, keep], v[:, :, keep], causal=False, scale=0.5)
    return max(_err(O, Oq), _err(L, Lq))


def check_sparse_block_diagonal(attn_sp):
    """A block-diagonal mask makes every block of rows its own sequence:
    equal to the pinned packed-sequence oracle with one sequence per block
    (causal and not)."""
    from oracle import attention
    r = _rng(88)
    N, blk = 10, 4
    q, k, v = (r.standard_normal((1, h, N, 3)) for h in (4, 2, 2))
    bm = np.eye(3, dtype=np.uint8)[None, None]
    cu = np.array([0, 4, 8, 10], np.int32)
    worst = 0.0
    for causal in (False, True):
        O, L = attn_sp(q, k, v, bm, causal=causal, scale=0.9, block=blk)
        Op, Lp = attention(*(x[0].transpose(1, 0, 2) for x in (q, k, v)), causal=causal,
                           scale=0.9, cu_seqlens=cu)
        worst = max(worst, _err(O[0], Op.transpose(1, 0, 2)))
        for b in range(3):
            worst = max(worst, _err(L[0, :, cu[b]:cu[b + 1]], Lp[b, :, :cu[b + 1] - cu[b]]))
    return worst


def check_sparse_broadcast(attn_sp):
    """A mask given once (1 x 1) equals the same mask repeated for every
    sequence and head; a per-head mask gives each head its own pattern
    (head h alone, run as a one-head problem, matches)."""
    r = _rng(89)
    q, k, v = _rand_qk(90, B=2, Hq=4, Hkv=2, Nq=8, Nk=8, d=3)
    one = (r.random((1, 1, 4, 4)) < 0.6).astype(np.uint8)
    one[..., 0] = 1
    worst = 0.0
    for causal in (False, True):
        O1, L1 = attn_sp(q, k, v, one, causal=causal, scale=0.5, block=2)
        Or, Lr = attn_sp(q, k, v, np.broadcast_to(one, (2, 4, 4, 4)).copy(), causal=causal,
                         scale=0.5, block=2)
        worst = max(worst, _finite_err(L1, Lr), _err(O1, Or))
        per = (r.random((2, 4, 4, 4)) < 0.6).astype(np.uint8)
        Oh, Lh = attn_sp(q, k, v, per, causal=causal, scale=0.5, block=2)
        for b in range(2):
            for h in range(4):
                g = h // 2
                Os, Ls = attn_sp(q[b:b + 1, h:h + 1], k[b:b + 1, g:g + 1], v[b:b + 1, g:g + 1],
                                 per[b:b + 1, h:h + 1], causal=causal, scale=0.5, block=2)
                worst = max(worst, _err(Oh[b, h], Os[0, 0]), _finite_err(Lh[b, h], Ls[0, 0]))
    return worst


SPARSE_CHECKS = [check_sparse_all_ones, check_sparse_library, check_sparse_bruteforce,
                 check_sparse_removed_key_blocks, check_sparse_block_diagonal,
                 check_sparse_broadcast]


# ---------------------------------------------------------------------------
# Backward pass.  Each check takes ``attn_bwd(q, k, v, do, *, causal, scale,
# cu_seqlens=None) -> (dQ, dK, dV)``.

def _rand_bwd(seed, B=2, Hq=4, Hkv=2, N=7, d=5):
    r = _rng(seed)
    return (r.standard_normal((B, Hq, N, d)), r.standard_normal((B, Hkv, N, d)),
            r.standard_normal((B, Hkv, N, d)), r.standard_normal((B, Hq, N, d)))


def check_bwd_finite_differences(attn_bwd):
    """Central differences (Richardson-extrapolated, step 1e-3) of
    F = sum(O * dO), with O from the pinned forward oracle, against the
    gradient, on every input element of a tiny case."""
    from oracle import attention
    worst = 0.0
    for causal in (False, True):
        q, k, v, do = _rand_bwd(71 + causal, B=1, Hq=2, Hkv=1, N=4, d=3)
        scale = 0.61
        grads = attn_bwd(q, k, v, do, causal=causal, scale=scale)

        def F(qq, kk, vv):
            return float(np.sum(attention(qq, kk, vv, causal=causal, scale=scale)[0] * do))

        for which, (x, g) in enumerate(zip((q, k, v), grads)):
            for idx in np.ndindex(x.shape):
                def at(hh):
                    xs = [q.copy(), k.copy(), v.copy()]
                    xs[which][idx] += hh
                    return F(*xs)

                def D(hh):
                    return (at(hh) - at(-hh)) / (2 * hh)
                fd = (4 * D(5e-4) - D(1e-3)) / 3
                worst = max(worst, abs(fd - g[idx]))
    # Richardson error is ~h^4 plus rounding ~1e-13: scale to the common TOL.
    return worst * (TOL / 1e-8)


def check_bwd_library(attn_bwd):
    """torch autograd through scaled_dot_product_attention (float64, CPU,
    GQA), the routine the French HolySheep article calls."""
    import torch
    import torch.nn.functional as F
    worst = 0.0
    for causal in (False, True):
        q, k, v, do = _rand_bwd(73 + causal, B=2, Hq=6, Hkv=2, N=29, d=16)
        scale = 0.27
        dQ, dK, dV = attn_bwd(q, k, v, do, causal=causal, scale=scale)
        tq, tk, tv = (torch.from_numpy(x).requires_grad_() for x in (q, k, v))
        o = F.scaled_dot_product_attention(tq, tk, tv, is_causal=causal, scale=scale,
                                           enable_gqa=True)
        (o * torch.from_numpy(do)).sum().backward()
        worst = max(worst, _err(dQ, tq.grad.numpy()), _err(dK, tk.grad.numpy()),
                    _err(dV, tv.grad.numpy()))
    return worst


def check_bwd_closed_forms(attn_bwd):
    """Facts of the softmax derivative: each row of dS sums to zero, so with
    all keys equal dQ = 0; shifting every key by w leaves O unchanged, so the
    dK of a K/V head sums to zero over its keys; P's rows sum to one, so
    dV summed over keys is dO summed over rows and over the group's query
    heads; causal row 0 sees one key, so its dQ is 0."""
    worst = 0.0
    r = _rng(75)
    for causal in (False, True):
        q, k, v, do = _rand_bwd(76 + causal)
        dQ, dK, dV = attn_bwd(q, k, v, do, causal=causal, scale=0.45)
        worst = max(worst, float(np.abs(dK.sum(axis=2)).max()))
        G = q.shape[1] // k.shape[1]
        dos = do.reshape(do.shape[0], k.shape[1], G, *do.shape[2:]).sum(axis=(2, 3))
        worst = max(worst, _err(dV.sum(axis=2), dos))
        if causal:
            worst = max(worst, float(np.abs(dQ[:, :, 0]).max()))
        keq = np.broadcast_to(r.standard_normal((2, 2, 1, 5)), k.shape).copy()
        dQ2, _, _ = attn_bwd(q, keq, v, do, causal=causal, scale=0.45)
        worst = max(worst, float(np.abs(dQ2).max()))
    return worst


def check_bwd_gqa_equals_repeated(attn_bwd):
    """GQA gradients = MHA gradients with K/V heads repeated per contiguous
    group, the K/V ones summed back over the group."""
    q, k, v, do = _rand_bwd(77, Hq=6, Hkv=2)
    worst = 0.0
    for causal in (False, True):
        dQ, dK, dV = attn_bwd(q, k, v, do, causal=causal, scale=0.5)
        kr, vr = np.repeat(k, 3, axis=1), np.repeat(v, 3, axis=1)
        dQr, dKr, dVr = attn_bwd(q, kr, vr, do, causal=causal, scale=0.5)
        sh = (dKr.shape[0], 2, 3) + dKr.shape[2:]
        worst = max(worst, _err(dQ, dQr), _err(dK, dKr.reshape(sh).sum(axis=2)),
                    _err(dV, dVr.reshape(sh).sum(axis=2)))
    return worst


def check_bwd_varlen_equals_fixed(attn_bwd):
    """Packed sequences = each sequence alone."""
    r = _rng(79)
    lens = [5, 1, 9]
    cu = np.concatenate([[0], np.cumsum(lens)]).astype(np.int32)
    T, Hq, Hkv, d = cu[-1], 4, 2, 3
    q, k, v, do = (r.standard_normal((T, h, d)) for h in (Hq, Hkv, Hkv, Hq))
    worst = 0.0
    for causal in (False, True):
        dQ, dK, dV = attn_bwd(q, k, v, do, causal=causal, scale=0.7, cu_seqlens=cu)
        for b in range(3):
            sl = slice(cu[b], cu[b + 1])
            one = [x[sl].transpose(1, 0, 2)[None] for x in (q, k, v, do)]
            g = attn_bwd(*one, causal=causal, scale=0.7)
            for full, part in zip((dQ, dK, dV), g):
                worst = max(worst, _err(full[sl], part[0].transpose(1, 0, 2)))
    return worst


BWD_CHECKS = [check_bwd_finite_differences, check_bwd_library, check_bwd_closed_forms,
              check_bwd_gqa_equals_repeated, check_bwd_varlen_equals_fixed]
