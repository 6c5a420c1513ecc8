"""Tensors past 2^31 elements (needs an MI355X, ~40 GB of its memory).

Q, O and dQ of B = 520 sequences × 32 query heads × 1024 rows × d = 128 hold
2.18e9 elements (O and dQ in fp32: 8.7 GB each), so every sequence from
b = 512 on lies past element 2^31 and past byte 2^32 of O: any 32-bit
element or byte offset in the loads, the epilogue stores or the backward's
accumulators would land on the wrong rows.  Inputs are drawn on the device
with torch's seeded generator (plumbing, not the path under test); the
oracle then runs on whole (sequence, head group) slices copied back: the
first sequence, the last one below 2^31 and two past it.
"""
from __future__ import annotations

import numpy as np
import pytest

import oracle
from tests import gpu_util as G

pytestmark = pytest.mark.gpu

DEV = "cuda:0"
B, HQ, HKV, N, D = 520, 32, 8, 1024, 128
GRP = HQ // HKV
PICKS = [(0, 0), (511, 7), (512, 3), (519, 6)]      # (sequence, K/V head)


@pytest.fixture(scope="module")
def inputs():
    import torch
    assert torch.cuda.is_available(), "GPU tests need a GPU"
    import exact_io_aware_amd as fa
    fa.load()
    assert B * HQ * N * D > 2 ** 31
    g = torch.Generator(device=DEV).manual_seed(31)
    mk = lambda *s: torch.randn(*s, generator=g, device=DEV, dtype=torch.bfloat16)  # noqa: E731
    q, k, v = mk(B, HQ, N, D), mk(B, HKV, N, D), mk(B, HKV, N, D)
    do = mk(B, HQ, N, D)
    yield q, k, v, do
    del q, k, v, do
    torch.cuda.empty_cache()


def _f64(t):
    import torch
    return t.to(torch.float64).cpu().numpy()


def _slices(t4, b, kvh, heads):
    return _f64(t4[b:b + 1, heads])


def test_forward_past_2_31_elements(inputs):
    import torch

    import exact_io_aware_amd as fa
    q, k, v, _ = inputs
    scale = 1.0 / np.sqrt(D)
    G.say(f"large forward: q {tuple(q.shape)} ({q.numel()} elements)")
    o, lse = fa.fwd(q, k, v, causal=True)
    torch.cuda.synchronize()
    for b, kvh in PICKS:
        hs = slice(kvh * GRP, (kvh + 1) * GRP)
        Oref, Lref = oracle.attention(_slices(q, b, kvh, hs), _slices(k, b, kvh, slice(kvh, kvh + 1)),
                                      _slices(v, b, kvh, slice(kvh, kvh + 1)), causal=True,
                                      scale=scale)
        O, L = _f64(o[b:b + 1, hs]), _f64(lse[b:b + 1, hs])
        eo, el = np.abs(O - Oref).max(), np.abs(L - Lref).max()
        G.say(f"  sequence {b}, K/V head {kvh}: O {eo:.3e}, L {el:.3e}")
        assert np.isfinite(O).all()
        assert eo <= G.O_TOL["bf16"] and el <= G.L_TOL, (b, kvh)


def test_backward_past_2_31_elements(inputs):
    import torch

    import exact_io_aware_amd as fa
    q, k, v, do = inputs
    scale = 1.0 / np.sqrt(D)
    G.say("large backward")
    o, lse = fa.fwd(q, k, v, causal=True)
    dq, dk, dv = fa.bwd(q, k, v, o, lse, do, causal=True)
    torch.cuda.synchronize()
    del o, lse
    for b, kvh in PICKS:
        hs, ks = slice(kvh * GRP, (kvh + 1) * GRP), slice(kvh, kvh + 1)
        ref = oracle.attention_backward(_slices(q, b, kvh, hs), _slices(k, b, kvh, ks),
                                        _slices(v, b, kvh, ks), _slices(do, b, kvh, hs),
                                        causal=True, scale=scale)
        got = (_f64(dq[b:b + 1, hs]), _f64(dk[b:b + 1, ks]), _f64(dv[b:b + 1, ks]))
        for name, a, r in zip(("dq", "dk", "dv"), got, ref):
            err = np.abs(a - r).max()
            G.say(f"  sequence {b}, K/V head {kvh}: {name} {err:.3e} (max |ref| {np.abs(r).max():.3e})")
            assert np.isfinite(a).all(), name
            assert err <= G.grad_bar("bf16") * np.abs(r).max(), (b, kvh, name)
