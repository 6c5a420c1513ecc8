"""Seeded random shapes against the oracle (needs an MI355X).

Each case draws its own shape from a fixed seed: input type, head size,
head counts and grouping (1 to 8 query heads per K/V head), batch,
fixed-length or packed sequences (empty and one-token ones included), more
or fewer queries than keys, causal or not, any finite scale, output type,
packed V and split-KV.  Sizes stay small enough for the oracle to finish in
well under a second per case while still spanning several tiles and ragged
ends.  The forward is compared element by element with the oracle's
``attention_qk`` (which is ``attention`` when the query and key counts are
equal) under the first-order bound of the P rounding (these shapes and
scales are not the workloads' distribution), the backward with
``attention_backward`` under the element-wise rounding bound.
"""
from __future__ import annotations

import numpy as np
import pytest

import oracle
import workloads
from tests import gpu_util as G

pytestmark = pytest.mark.gpu

DEV = "cuda:0"
N_FWD, N_BWD = 32, 12


def _fwd_case(i):
    rng = np.random.default_rng(7000 + i)
    dtype = str(rng.choice(["fp32", "fp16", "bf16"], p=[0.2, 0.4, 0.4]))
    d = int(rng.choice([64, 128]))
    Hkv = int(rng.integers(1, 5))
    Hq = Hkv * int(rng.choice([1, 2, 3, 4, 8]))
    B = int(rng.integers(1, 4))
    causal = bool(rng.random() < 0.7)
    form = str(rng.choice(["fixed", "varlen", "qk_fixed", "qk_varlen"]))
    scale = float(rng.choice([1.0 / np.sqrt(d), 0.05, 0.3, -0.2]))
    if form == "fixed":
        lay = dict(Nq=int(rng.integers(1, 401)))
        lay["Nk"] = lay["Nq"]
    elif form == "qk_fixed":
        lay = dict(Nq=int(rng.integers(1, 201)), Nk=int(rng.integers(1, 401)))
    else:
        lq = rng.integers(0, 301, B)
        lq[rng.integers(0, B)] = max(1, int(lq.max()))
        lk = lq.copy() if form == "varlen" else rng.integers(0, 401, B)
        lay = dict(lengths_q=[int(x) for x in lq], lengths_k=[int(x) for x in lk])
    opts = {}
    if dtype != "fp32":
        opts["packed"] = bool(rng.random() < 0.3)
        opts["num_splits"] = [None, 1, 2, 3][int(rng.integers(0, 4))]
        opts["out_in_dtype"] = bool(rng.random() < 0.3)
    return dict(dtype=dtype, d=d, B=B, Hq=Hq, Hkv=Hkv, causal=causal, scale=scale,
                form=form, seed=7000 + i, **lay, **opts)


def _bwd_case(i):
    rng = np.random.default_rng(8000 + i)
    dtype = str(rng.choice(["fp16", "bf16"]))
    d = int(rng.choice([64, 128]))
    Hkv = int(rng.integers(1, 4))
    Hq = Hkv * int(rng.choice([1, 2, 4, 8]))
    B = int(rng.integers(1, 4))
    causal = bool(rng.random() < 0.7)
    scale = float(rng.choice([1.0 / np.sqrt(d), 0.05, 0.3]))
    if rng.random() < 0.5:
        lay = dict(N=int(rng.integers(1, 321)))
    else:
        ls = rng.integers(0, 257, B)
        ls[rng.integers(0, B)] = max(1, int(ls.max()))
        lay = dict(lengths=[int(x) for x in ls])
    return dict(dtype=dtype, d=d, B=B, Hq=Hq, Hkv=Hkv, causal=causal, scale=scale,
                seed=8000 + i, **lay)


FWD = [_fwd_case(i) for i in range(N_FWD)]
BWD = [_bwd_case(i) for i in range(N_BWD)]


@pytest.fixture(scope="module", autouse=True)
def gpu_ready():
    import torch
    assert torch.cuda.is_available(), "GPU tests need a GPU"
    import exact_io_aware_amd as fa
    fa.load()


@pytest.mark.parametrize("c", FWD, ids=[f"fwd{i}" for i in range(N_FWD)])
def test_random_forward(c):
    import torch

    import exact_io_aware_amd as fa
    if "lengths_q" in c:
        w = workloads.make_custom_qk(c["B"], c["Hq"], c["Hkv"], c["d"], c["dtype"], c["seed"],
                                     lengths_q=c["lengths_q"], lengths_k=c["lengths_k"])
    else:
        w = workloads.make_custom_qk(c["B"], c["Hq"], c["Hkv"], c["d"], c["dtype"], c["seed"],
                                     Nq=c["Nq"], Nk=c["Nk"])
    w["causal"], w["scale"] = c["causal"], c["scale"]
    G.say(f"random forward {c}")
    q, k, v = (G.to_device(w[x], w["dtype"], DEV) for x in "qkv")
    cu = cuk = None
    kw = {}
    if w["cu_seqlens"] is not None:
        cu = torch.from_numpy(w["cu_seqlens"]).to(DEV)
        cuk = torch.from_numpy(w["cu_seqlens_k"]).to(DEV)
        kw = dict(cu_seqlens=cu, cu_seqlens_k=cuk, max_seqlen=w["N"], max_seqlen_k=max(1, w["Nk"]))
    odt = G.torch_dtype(w["dtype"]) if c.get("out_in_dtype") else torch.float32
    lse = torch.full((w["B"], w["Hq"], w["N"]), float("nan"), device=DEV)
    vt = None
    if c.get("packed"):
        vt = fa.pack_v(v, cu_seqlens=cuk, max_seqlen=kw.get("max_seqlen_k"))
    o, lse = fa.fwd(q, k, None if vt is not None else v, causal=w["causal"], scale=w["scale"],
                    out_dtype=odt, lse=lse, vt=vt, num_splits=c.get("num_splits"), **kw)
    torch.cuda.synchronize()
    O, L = o.double().cpu().numpy(), lse.double().cpu().numpy()
    qf, kf, vf = G.f64_inputs(w)
    Oref, Lref = oracle.attention_qk(qf, kf, vf, causal=w["causal"], scale=w["scale"],
                                     cu_seqlens_q=w["cu_seqlens"], cu_seqlens_k=w["cu_seqlens_k"])
    # Scales other than 1/sqrt(d) leave the workloads' score distribution, so
    # the bar is the first-order bound of the P rounding (the derived bar of
    # the stress tests; never below the stated one), plus half an ulp of O
    # when O is stored in 16 bits.
    A, _ = oracle.attention_qk(qf, kf, np.abs(vf), causal=w["causal"], scale=w["scale"],
                               cu_seqlens_q=w["cu_seqlens"], cu_seqlens_k=w["cu_seqlens_k"])
    bar = G.o_bar_derived(w["dtype"], A)
    if c.get("out_in_dtype"):
        bar = bar + np.abs(Oref) * {"bf16": 2.0 ** -8, "fp16": 2.0 ** -11}[w["dtype"]]
    out_name = w["dtype"] if c.get("out_in_dtype") else "fp32"
    G.say(f"  errors {G.compare_qk(w, O, L, Oref, Lref, out_dtype=out_name, bar=bar)}")


@pytest.mark.parametrize("c", BWD, ids=[f"bwd{i}" for i in range(N_BWD)])
def test_random_backward(c):
    import torch

    import exact_io_aware_amd as fa
    lay = dict(lengths=c["lengths"]) if "lengths" in c else dict(N=c["N"])
    w = workloads.make_custom(c["B"], c["Hq"], c["Hkv"], c["d"], c["dtype"], seed=c["seed"], **lay)
    w["dout"] = workloads.make_custom(c["B"], c["Hq"], c["Hq"], c["d"], c["dtype"],
                                      seed=c["seed"] + 5000, **lay)["q"]
    w["causal"], w["scale"] = c["causal"], c["scale"]
    G.say(f"random backward {c}")
    q, k, v, do = (G.to_device(w[x], w["dtype"], DEV) for x in ("q", "k", "v", "dout"))
    cu = None if w["cu_seqlens"] is None else torch.from_numpy(w["cu_seqlens"]).to(DEV)
    ms = w["N"] if cu is not None else None
    o, lse = fa.fwd(q, k, v, causal=w["causal"], scale=w["scale"], cu_seqlens=cu, max_seqlen=ms)
    dq, dk, dv = fa.bwd(q, k, v, o, lse, do, causal=w["causal"], scale=w["scale"],
                        cu_seqlens=cu, max_seqlen=ms)
    torch.cuda.synchronize()
    got = tuple(x.double().cpu().numpy() for x in (dq, dk, dv))
    qf, kf, vf = G.f64_inputs(w)
    ref = oracle.attention_backward(qf, kf, vf, workloads.to_f64(w["dout"], w["dtype"]),
                                    causal=w["causal"], scale=w["scale"],
                                    cu_seqlens=w["cu_seqlens"])
    terms = G.grad_term_sums(w)
    u = {"bf16": 2.0 ** -8, "fp16": 2.0 ** -11}[w["dtype"]]
    for name, a, r, t, k_ in zip(("dq", "dk", "dv"), got, ref, terms, (3.0, 3.0, 1.0)):
        assert np.isfinite(a).all(), name
        err = np.abs(a - r)
        ratio = float((err / (k_ * u * t + 1e-6)).max()) if err.size else 0.0
        G.say(f"  {name}: max err {err.max() if err.size else 0.0:.3e}, "
              f"of the element-wise bound {ratio:.2f}")
        # the first-order rounding bound of each element (see grad_term_sums),
        # with 25 % of slack for the fp32 sums and second-order terms
        assert ratio <= 1.25, (name, ratio)
