"""The oracle against facts that do not come from the oracle (CPU only)."""
from __future__ import annotations

import importlib

import numpy as np
import pytest

import oracle
import workloads
from tests import oracle_checks as C

exact = importlib.import_module("oracle.exact")


@pytest.mark.parametrize("check", C.CHECKS, ids=lambda f: f.__name__)
def test_oracle_pin(check):
    assert check(oracle.attention) <= C.TOL


def test_softmax_rows_sum_to_one():
    r = np.random.default_rng(5)
    S = r.standard_normal((17, 23)) * 30
    S[np.triu_indices(17, 1, 23)] = -np.inf
    P, m, ell = oracle.softmax_rows(S)
    assert np.allclose(P.sum(axis=1), 1.0, atol=1e-14, rtol=0)
    assert (P >= 0).all()
    assert np.array_equal(m, S.max(axis=1))
    assert np.allclose(m + np.log(ell), np.log(np.exp(S).sum(axis=1)), atol=1e-12)


def test_attention_rows_matches_full():
    w = workloads.make_custom(2, 4, 2, 16, "bf16", seed=7, N=300)
    q, k, v = (workloads.to_f64(w[x], "bf16") for x in "qkv")
    O, L = oracle.attention(q, k, v, causal=True, scale=0.25)
    picks = [(0, 0, 0), (1, 3, 299), (0, 2, 150), (1, 1, 63)]
    Or, Lr = oracle.attention_rows(q, k, v, causal=True, scale=0.25, picks=picks)
    for i, (b, h, r) in enumerate(picks):
        # BLAS blocking differs with the row count: equal up to rounding
        assert np.max(np.abs(Or[i] - O[b, h, r])) < 1e-13
        assert abs(Lr[i] - L[b, h, r]) < 1e-13


def test_pool_matches_serial():
    w = workloads.make_custom(1, 4, 4, 32, "fp16", seed=8, N=200)
    q, k, v = (workloads.to_f64(w[x], "fp16") for x in "qkv")
    O1, L1 = oracle.attention(q, k, v, causal=True, scale=0.2, workers=1)
    O2, L2 = oracle.attention(q, k, v, causal=True, scale=0.2, workers=2)
    assert np.array_equal(O1, O2) and np.array_equal(L1, L2)


# ---------------------------------------------------------------------------
# Planted mistakes: each plausible error in a piece of the oracle must be
# caught by at least one pin above.

def _mutants():
    ln2 = np.log(2.0)
    return {
        "drop_scale": ("scores", lambda q, k, scale: q @ k.T),
        "square_scale": ("scores", lambda q, k, scale: scale * scale * (q @ k.T)),
        "transposed_scores": ("scores", lambda q, k, scale: scale * (q @ k.T).T),
        "causal_off_by_one": ("causal_mask", lambda S, r, c: np.where(
            c[None, :] > r[:, None] + 1, -np.inf, S)),
        "causal_strict": ("causal_mask", lambda S, r, c: np.where(
            c[None, :] >= np.maximum(r[:, None], 1), -np.inf, S)),
        "causal_reversed": ("causal_mask", lambda S, r, c: np.where(
            c[None, :] < r[:, None], -np.inf, S)),
        "gqa_modulo": ("_group", lambda h, Hq, Hkv: h % Hkv),
        "lse_log2": ("logsumexp_of", lambda m, ell: m / ln2 + np.log2(ell)),
        "lse_no_max": ("logsumexp_of", lambda m, ell: np.log(ell)),
        "unnormalised": ("softmax_rows", lambda S: (
            np.exp(S - S.max(1, keepdims=True)), S.max(1),
            np.exp(S - S.max(1, keepdims=True)).sum(1))),
        "values_reversed": ("combine", lambda P, v: P @ v[::-1]),
        "keys_as_values": ("combine", None),
    }


@pytest.mark.parametrize("name", sorted(_mutants()))
def test_pins_catch_planted_mistake(name, monkeypatch):
    attr, fn = _mutants()[name]
    if name == "keys_as_values":
        orig_head = exact._head_rows
        monkeypatch.setattr(exact, "_head_rows",
                            lambda q, k, v, causal, scale, rows=None:
                            orig_head(q, k, k, causal, scale, rows))
    else:
        monkeypatch.setattr(exact, attr, fn)
    worst = 0.0
    for check in C.CHECKS:
        try:
            worst = max(worst, check(oracle.attention))
        except Exception:
            worst = np.inf
        if worst > C.TOL:
            break
    assert worst > C.TOL, f"no pin caught the planted mistake {name}"


# ---------------------------------------------------------------------------
# Input generation (shared with the GPU side): rounding and lengths.

def test_bf16_rounding_matches_torch():
    import torch
    x = np.random.default_rng(3).standard_normal(100000).astype(np.float32) * 7
    x[:4] = [1.00390625, 1.01171875, -1.00390625, 3.0]   # ties to even
    ours = workloads.round_to_bf16_bits(x)
    ref = torch.from_numpy(x).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    assert np.array_equal(ours, ref)
    back = workloads.bf16_bits_to_f32(ours)
    assert np.array_equal(back, torch.from_numpy(x).to(torch.bfloat16).float().numpy())


def test_varlen_lengths():
    w = workloads.make_inputs("varlen_bf16")
    lens = np.diff(w["cu_seqlens"])
    assert lens.min() >= 1024 and lens.max() <= 8192 and len(lens) == 16
    assert w["cu_seqlens"][0] == 0 and w["cu_seqlens"].dtype == np.int32
    assert w["q"].shape == (int(w["cu_seqlens"][-1]), 32, 128)
    assert w["N"] == lens.max()


def test_shard_workloads():
    """One GPU's shares: gqa_bf16 by K/V head (1 of 8) and long_bf16 by
    zig-zag query rows (GPU 0 of 8: the first and the last 2048 rows)."""
    t = workloads.make_inputs("gqa_bf16_tp8")
    assert t["q"].shape == (4, 4, 4096, 128) and t["k"].shape == (4, 1, 4096, 128)
    s = workloads.make_inputs("long_bf16_sp8")
    assert list(s["cu_seqlens"]) == [0, 2048, 4096]
    assert list(s["cu_seqlens_k"]) == [0, 2048, 2048 + 32768]
    assert s["q"].shape == (4096, 32, 128) and s["k"].shape == (34816, 8, 128)
    assert (s["N"], s["Nk"]) == (2048, 32768)
    # Zig-zag balance: this share's visible pairs are 1/8 of long_bf16's.
    share = sum(oracle.pair_count(2048, nk, True) for nk in (2048, 32768))
    assert share * 8 == oracle.pair_count(32768, 32768, True)


def test_workload_shapes():
    for name, wl in workloads.WORKLOADS.items():
        if wl.varlen or wl.N > 4096:
            continue
        x = workloads.make_inputs(name)
        assert x["q"].shape == (wl.B, wl.Hq, wl.N, wl.d)
        assert x["k"].shape == (wl.B, wl.Hkv, wl.Nk or wl.N, wl.d)
        assert x["v"].shape == x["k"].shape


# ---------------------------------------------------------------------------
# Queries against a longer key/value sequence (chunked prefill).

@pytest.mark.parametrize("check", C.QK_CHECKS, ids=lambda f: f.__name__)
def test_oracle_qk_pin(check):
    assert check(oracle.attention_qk) <= C.TOL


def _qk_mutants():
    return {
        "top_left": ("offset_mask", lambda S, r, c, off: np.where(
            c[None, :] > r[:, None], -np.inf, S)),
        "offset_plus_one": ("offset_mask", lambda S, r, c, off: np.where(
            c[None, :] > r[:, None] + off + 1, -np.inf, S)),
        "offset_reversed": ("offset_mask", lambda S, r, c, off: np.where(
            c[None, :] > r[:, None] - off, -np.inf, S)),
        "unseen_rows_zero_lse": ("_head_rows_qk", None),
        "scores_of_prefix_only": ("scores", None),
    }


@pytest.mark.parametrize("name", sorted(_qk_mutants()))
def test_qk_pins_catch_planted_mistake(name, monkeypatch):
    attr, fn = _qk_mutants()[name]
    if name == "unseen_rows_zero_lse":
        orig = exact._head_rows_qk

        def fn(q, k, v, causal, scale, rows=None):
            O, L = orig(q, k, v, causal, scale, rows)
            return O, np.where(np.isneginf(L), 0.0, L)
    elif name == "scores_of_prefix_only":
        orig_s = exact.scores

        def fn(q, k, scale):          # keys past the query count ignored
            S = orig_s(q, k, scale)
            S[:, q.shape[0]:] = -np.inf if q.shape[0] < k.shape[0] else S[:, q.shape[0]:]
            return S
    monkeypatch.setattr(exact, attr, fn)
    worst = 0.0
    for check in C.QK_CHECKS:
        try:
            worst = max(worst, check(oracle.attention_qk))
        except Exception:
            worst = np.inf
        if worst > C.TOL:
            break
    assert worst > C.TOL, f"no pin caught the planted mistake {name}"


def test_pair_count():
    for nq, nk in ((5, 5), (3, 9), (9, 4), (1, 7), (7, 0)):
        brute = sum(1 for r in range(nq) for c in range(nk) if c <= r + nk - nq)
        assert oracle.pair_count(nq, nk, True) == brute
        assert oracle.pair_count(nq, nk, False) == nq * nk


# ---------------------------------------------------------------------------
# Block-sparse attention.

@pytest.mark.parametrize("check", C.SPARSE_CHECKS, ids=lambda f: f.__name__)
def test_oracle_sparse_pin(check):
    assert check(oracle.attention_block_sparse) <= C.TOL


def _sparse_allowed_mutant(name):
    def allowed(bm, rows, nk, block, causal, offset):
        cols = np.arange(nk)
        rb = (rows + 1) // block if name == "row_block_off_by_one" else rows // block
        cb = (cols + 1) // block if name == "key_block_off_by_one" else cols // block
        rb = np.minimum(rb, bm.shape[0] - 1)
        cb = np.minimum(cb, bm.shape[1] - 1)
        if name == "block_transposed":        # key block used as the row-block index
            a = bm[np.minimum(cb, bm.shape[0] - 1)][:, np.minimum(rb, bm.shape[1] - 1)].T != 0
        elif name == "mask_ignored":
            a = np.ones((rows.size, nk), bool)
        else:
            a = bm[rb][:, cb] != 0
        if causal and name != "causal_dropped":
            a &= cols[None, :] <= rows[:, None] + (0 if name == "causal_top_left" else offset)
        return a
    return allowed


@pytest.mark.parametrize("name", ["row_block_off_by_one", "key_block_off_by_one",
                                  "block_transposed", "mask_ignored", "causal_dropped",
                                  "causal_top_left", "mask_of_kv_head", "empty_rows_zero"])
def test_sparse_pins_catch_planted_mistake(name, monkeypatch):
    orig = exact.attention_block_sparse
    if name == "mask_of_kv_head":
        def attn_sp(q, k, v, bm, *, causal, scale, block=64, cu_seqlens_q=None,
                    cu_seqlens_k=None):
            G = q.shape[1] // k.shape[1]
            if bm.shape[1] > 1:             # head h reads the mask of head h // G
                bm = bm[:, np.arange(bm.shape[1]) // G]
            return orig(q, k, v, bm, causal=causal, scale=scale, block=block,
                        cu_seqlens_q=cu_seqlens_q, cu_seqlens_k=cu_seqlens_k)
    elif name == "empty_rows_zero":
        def attn_sp(*a, **kw):
            O, L = orig(*a, **kw)
            return O, np.where(np.isneginf(L), 0.0, L)
    else:
        monkeypatch.setattr(exact, "sparse_allowed", _sparse_allowed_mutant(name))
        attn_sp = orig
    worst = 0.0
    for check in C.SPARSE_CHECKS:
        try:
            worst = max(worst, check(attn_sp))
        except Exception:
            worst = np.inf
        if worst > C.TOL:
            break
    assert worst > C.TOL, f"no pin caught the planted mistake {name}"


def test_sparse_pair_count():
    r = np.random.default_rng(91)
    for nq, nk, blk in ((9, 9, 2), (5, 13, 4), (13, 5, 3)):
        bm = (r.random((-(-nq // blk), -(-nk // blk))) < 0.5).astype(np.uint8)
        for causal in (False, True):
            brute = sum(1 for i in range(nq) for c in range(nk)
                        if bm[i // blk, c // blk] and (not causal or c <= i + nk - nq))
            assert oracle.sparse_pair_count(bm, nq, nk, causal, blk) == brute


# ---------------------------------------------------------------------------
# Backward pass.

@pytest.mark.parametrize("check", C.BWD_CHECKS, ids=lambda f: f.__name__)
def test_oracle_bwd_pin(check):
    assert check(oracle.attention_backward) <= C.TOL


def _bwd_mutant(name):
    """A copy of the per-head backward with one plausible mistake."""
    def head(q, k, v, do, causal, scale):
        n = q.shape[0]
        S = scale * (q @ k.T)
        if causal:
            S = np.where(np.arange(n)[None, :] > np.arange(n)[:, None], -np.inf, S)
        P = np.exp(S - S.max(1, keepdims=True))
        P /= P.sum(1, keepdims=True)
        O = P @ v
        dv = (P if name == "dv_untransposed" else P.T) @ do
        dP = do @ v.T
        D = dP.sum(1, keepdims=True) if name == "delta_without_p" else \
            np.sum(do * O, 1, keepdims=True)
        dS = P * dP if name == "no_delta" else P * (dP - D)
        dq = (1.0 if name == "dq_no_scale" else scale) * (dS @ k)
        dk = scale * ((dS if name == "dk_untransposed" else dS.T) @ q)
        return dq, dk, dv
    return head


@pytest.mark.parametrize("name", ["no_delta", "delta_without_p", "dq_no_scale",
                                  "dk_untransposed", "dv_untransposed", "gqa_first_head_only"])
def test_bwd_pins_catch_planted_mistake(name, monkeypatch):
    if name == "gqa_first_head_only":
        orig = exact.attention_backward

        def attn_bwd(q, k, v, do, *, causal, scale, cu_seqlens=None, workers=1):
            G = q.shape[1] // k.shape[1]
            dQ, dK, dV = orig(q, k, v, do, causal=causal, scale=scale, cu_seqlens=cu_seqlens)
            if G == 1:
                return dQ, dK, dV
            keep = np.zeros(q.shape[1], bool)
            keep[::G] = True
            do2 = do.copy()
            do2[:, ~keep] = 0            # head axis is 1 in both layouts
            _, dK1, dV1 = orig(q, k, v, do2, causal=causal, scale=scale, cu_seqlens=cu_seqlens)
            return dQ, dK1, dV1
    else:
        monkeypatch.setattr(exact, "_head_backward", _bwd_mutant(name))
        attn_bwd = exact.attention_backward
    worst = 0.0
    for check in C.BWD_CHECKS:
        try:
            worst = max(worst, check(attn_bwd))
        except Exception:
            worst = np.inf
        if worst > C.TOL:
            break
    assert worst > C.TOL, f"no pin caught the planted mistake {name}"


def test_flop_and_visibility_counts():
    """unit_flops and visible_keys against counting the visible (query,
    key) pairs one by one."""
    for n in (1, 2, 7, 33):
        for causal in (False, True):
            vis = [[c <= r or not causal for c in range(n)] for r in range(n)]
            for r in range(n):
                assert oracle.visible_keys(r, n, causal) == sum(vis[r])
            assert oracle.unit_flops(n, 64, causal) == 4.0 * 64 * sum(map(sum, vis))
