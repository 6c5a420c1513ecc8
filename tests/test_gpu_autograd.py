"""``attention``: the forward and backward kernels as one differentiable torch
operation (needs an MI355X).  Its output and gradients must be exactly what
the two entry points give when called directly, and within the backward's
bar of the oracle's gradients."""
from __future__ import annotations

import numpy as np
import pytest

import oracle
import workloads
from tests import gpu_util as G

pytestmark = pytest.mark.gpu

CASES = [
    ("bf16", 128, 2, 8, 2, 200, True),
    ("fp16", 64, 2, 4, 2, [129, 64], False),
]


def _make(case, seed):
    dtype, d, B, Hq, Hkv, n, causal = case
    kw = {"lengths": n} if isinstance(n, list) else {"N": n}
    w = workloads.make_custom(B, Hq, Hkv, d, dtype, seed=seed, **kw)
    w["dout"] = workloads.make_custom(B, Hq, Hq, d, dtype, seed=seed + 5000, **kw)["q"]
    w["causal"] = causal
    w["scale"] = 1.0 / np.sqrt(d)
    return w


@pytest.mark.parametrize("case", CASES, ids=["bf16-d128-gqa-causal", "fp16-d64-varlen"])
def test_attention_autograd_matches_entry_points_and_oracle(case):
    import torch

    import exact_io_aware_amd as fa
    w = _make(case, seed=1300)
    dev = "cuda:0"
    q, k, v, do = (G.to_device(w[x], w["dtype"], dev) for x in ("q", "k", "v", "dout"))
    cu = None if w["cu_seqlens"] is None else torch.from_numpy(w["cu_seqlens"]).to(dev)
    ms = w["N"] if cu is not None else None
    G.say(f"autograd attention {case}")
    qg, kg, vg = (t.clone().requires_grad_(True) for t in (q, k, v))
    o = fa.attention(qg, kg, vg, causal=w["causal"], scale=w["scale"], cu_seqlens=cu,
                     max_seqlen=ms)
    o.backward(do)
    torch.cuda.synchronize()
    # the same two calls made directly
    o_ref, lse = fa.fwd(q, k, v, causal=w["causal"], scale=w["scale"], cu_seqlens=cu,
                        max_seqlen=ms, out_dtype=q.dtype, num_splits=1)
    dq, dk, dv = fa.bwd(q, k, v, o_ref, lse, do, causal=w["causal"], scale=w["scale"],
                        cu_seqlens=cu, max_seqlen=ms, grad_dtype=q.dtype)
    torch.cuda.synchronize()
    assert o.dtype == q.dtype and torch.equal(o.detach(), o_ref)
    for name, a, b in (("dq", qg.grad, dq), ("dk", kg.grad, dk), ("dv", vg.grad, dv)):
        assert a.dtype == q.dtype and torch.equal(a, b), name
    # and the oracle's gradients, within the bar (plus half an ulp of the
    # 16-bit gradients and of the 16-bit O that feeds the D rows)
    qf, kf, vf = G.f64_inputs(w)
    dof = workloads.to_f64(w["dout"], w["dtype"])
    ref = oracle.attention_backward(qf, kf, vf, dof, causal=w["causal"], scale=w["scale"],
                                    cu_seqlens=w["cu_seqlens"])
    ulp = {"bf16": 2.0 ** -8, "fp16": 2.0 ** -11}[w["dtype"]]
    for name, a, r in zip(("dq", "dk", "dv"), (qg.grad, kg.grad, vg.grad), ref):
        got = a.double().cpu().numpy()
        err = np.abs(got - r)
        G.say(f"  {name}: max err {err.max():.3e}, max |ref| {np.abs(r).max():.3e}")
        assert np.isfinite(got).all()
        assert (err <= G.grad_bar(w["dtype"]) * np.abs(r).max() + np.abs(r) * ulp).all(), name


def test_attention_fp32_forward_only():
    """fp32 inputs: the forward runs (the exactness path); asking for their
    gradients raises rather than falling back to anything."""
    import torch

    import exact_io_aware_amd as fa
    w = workloads.make_custom(1, 2, 2, 64, "fp32", seed=1310, N=100)
    q, k, v = (torch.from_numpy(w[x]).to("cuda:0").requires_grad_(True) for x in "qkv")
    G.say("autograd attention, fp32")
    o = fa.attention(q, k, v, causal=True)
    o_ref, _ = fa.fwd(q.detach(), k.detach(), v.detach(), causal=True, out_dtype=torch.float32)
    torch.cuda.synchronize()
    assert torch.equal(o.detach(), o_ref)
    with pytest.raises(RuntimeError):
        o.sum().backward()
