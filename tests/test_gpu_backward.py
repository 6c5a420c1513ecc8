"""Backward pass on the GPU vs the oracle's gradients (needs an MI355X)."""
from __future__ import annotations

import numpy as np
import pytest

import oracle
import workloads
from tests import gpu_util as G

pytestmark = pytest.mark.gpu

# (dtype, d, B, Hq, Hkv, N or lengths, causal)
CASES = [
    ("bf16", 128, 2, 8, 2, 200, True),
    ("bf16", 128, 2, 8, 2, 200, False),
    ("bf16", 64, 1, 4, 4, 333, True),
    ("fp16", 128, 1, 4, 1, 130, True),
    ("fp16", 64, 2, 6, 3, 97, False),
    ("bf16", 128, 3, 8, 2, [70, 1, 190], True),
    ("fp16", 64, 2, 4, 2, [129, 64], False),
    ("bf16", 128, 3, 8, 2, [70, 0, 33], True),        # an empty sequence
    ("fp16", 64, 2, 8, 2, 300, True),                 # d = 64 causal, 4 heads per workgroup
    ("bf16", 64, 2, 4, 2, [100, 257], True),          # d = 64 causal varlen, 2 heads per workgroup
]


def _make(case, seed):
    dtype, d, B, Hq, Hkv, n, causal = case
    if isinstance(n, list):
        w = workloads.make_custom(B, Hq, Hkv, d, dtype, seed=seed, lengths=n)
        g = workloads.make_custom(B, Hq, Hq, d, dtype, seed=seed + 5000, lengths=n)
    else:
        w = workloads.make_custom(B, Hq, Hkv, d, dtype, seed=seed, N=n)
        g = workloads.make_custom(B, Hq, Hq, d, dtype, seed=seed + 5000, N=n)
    w["dout"] = g["q"]                     # dO: seeded N(0,1), rounded like the inputs
    w["causal"] = causal
    w["scale"] = 1.0 / np.sqrt(d)
    return w


def _gpu(w, grad_dtype=None, out_dtype=None):
    import torch

    import exact_io_aware_amd as fa
    dev = "cuda:0"
    q, k, v, do = (G.to_device(w[x], w["dtype"], dev) for x in ("q", "k", "v", "dout"))
    cu = None if w["cu_seqlens"] is None else torch.from_numpy(w["cu_seqlens"]).to(dev)
    ms = w["N"] if cu is not None else None
    o, lse = fa.fwd(q, k, v, causal=w["causal"], scale=w["scale"], cu_seqlens=cu, max_seqlen=ms,
                    out_dtype=out_dtype or torch.float32)
    dq, dk, dv = fa.bwd(q, k, v, o, lse, do, causal=w["causal"], scale=w["scale"],
                        cu_seqlens=cu, max_seqlen=ms,
                        grad_dtype=grad_dtype or torch.float32)
    torch.cuda.synchronize()
    return tuple(x.double().cpu().numpy() for x in (dq, dk, dv))


def _oracle(w):
    q, k, v = G.f64_inputs(w)
    do = workloads.to_f64(w["dout"], w["dtype"])
    return oracle.attention_backward(q, k, v, do, causal=w["causal"], scale=w["scale"],
                                     cu_seqlens=w["cu_seqlens"])


@pytest.mark.parametrize("i", range(len(CASES)), ids=lambda i: "-".join(map(str, CASES[i][:5])))
def test_backward_parity(i):
    case = CASES[i]
    w = _make(case, seed=900 + i)
    ref = _oracle(w)
    G.say(f"backward case {case}")
    got = _gpu(w)
    terms = G.grad_term_sums(w)
    u = {"bf16": 2.0 ** -8, "fp16": 2.0 ** -11}[w["dtype"]]
    for name, a, r, t, c in zip(("dq", "dk", "dv"), got, ref, terms, (3.0, 3.0, 1.0)):
        err = np.abs(a - r)
        ratio = float((err / (c * u * t + 1e-6)).max())
        G.say(f"  {name}: max err {err.max():.3e}, max |ref| {np.abs(r).max():.3e}, "
              f"rel {err.max() / np.abs(r).max():.3e}, of the element-wise bound {ratio:.2f}")
        assert np.isfinite(a).all()
        assert err.max() <= G.grad_bar(w["dtype"]) * np.abs(r).max(), name
        # element by element: within the first-order bound of the roundings
        # (grad_term_sums: P and dS rounded, u each, and D's error from the
        # forward's P rounding, u * A_r: 3u in all for dQ and dK, u for dV),
        # with 25 % of slack for the fp32 sums and second-order terms
        assert ratio <= 1.25, (name, ratio)


@pytest.mark.parametrize("case", [("bf16", 128, 2, 8, 2, 200, True),
                                  ("fp16", 64, 2, 4, 2, [129, 64], False)],
                         ids=["bf16-d128", "fp16-d64-varlen"])
def test_backward_from_16bit_o(case):
    """O stored in the input type (the forward's 16-bit output) feeds the D
    rows: the same bar, with O's rounding (half an ulp) inside it."""
    w = _make(case, seed=960)
    ref = _oracle(w)
    G.say(f"backward from 16-bit O, case {case}")
    got = _gpu(w, out_dtype=G.torch_dtype(w["dtype"]))
    for name, a, r in zip(("dq", "dk", "dv"), got, ref):
        err = np.abs(a - r)
        G.say(f"  {name}: max err {err.max():.3e}, max |ref| {np.abs(r).max():.3e}")
        assert np.isfinite(a).all()
        assert err.max() <= G.grad_bar(w["dtype"]) * np.abs(r).max(), name


def test_backward_gradients_in_input_dtype_and_deterministic():
    import torch
    w = _make(("bf16", 128, 1, 8, 1, 257, True), seed=950)   # 8 query heads per K/V head
    ref = _oracle(w)
    G.say("backward, bf16 gradients, twice")
    a = _gpu(w, grad_dtype=torch.bfloat16)
    b = _gpu(w, grad_dtype=torch.bfloat16)
    for name, x, y, r in zip(("dq", "dk", "dv"), a, b, ref):
        assert np.array_equal(x, y), f"{name} differs between runs"
        # the stored bf16 adds half an ulp of the value on top of the bar
        bar = G.grad_bar("bf16") * np.abs(r).max() + np.abs(r) * 2.0 ** -8
        assert (np.abs(x - r) <= bar).all(), name


@pytest.mark.parametrize("name", ["gqa_bf16", "mha_fp16"])
def test_backward_workload_full(name):
    """The backward at the full size of the workloads bench.py times for it
    (gqa_bf16: B=4, Hq=32, Hkv=8, N=4096, d=128; mha_fp16: B=8, H=12,
    N=2048, d=64; causal; dO drawn as bench.py draws it), checked against
    the oracle on every sequence and head."""
    w = workloads.make_inputs(name)
    w["dout"] = workloads.make_custom(w["B"], w["Hq"], w["Hq"], w["d"], w["dtype"],
                                      seed=w["seed"] + 100, N=w["N"])["q"]
    G.say(f"backward {name}")
    got = _gpu(w)
    q, k, v = G.f64_inputs(w)
    do = workloads.to_f64(w["dout"], w["dtype"])
    ref = oracle.attention_backward(q, k, v, do, causal=True, scale=w["scale"],
                                    workers=min(16, oracle.default_workers()))
    for name_, a, r in zip(("dq", "dk", "dv"), got, ref):
        err = np.abs(a - r)
        G.say(f"  {name_}: max err {err.max():.3e}, max |ref| {np.abs(r).max():.3e}")
        assert np.isfinite(a).all()
        assert err.max() <= G.grad_bar(w["dtype"]) * np.abs(r).max(), name_
