"""No kernel reads LDS it did not write (needs an MI355X).

libfa_poison.so is the same library built with FA_POISON_LDS=1: every
kernel fills its LDS buffers with NaN before use.  A kernel that read a
location none of its loads or stores wrote (a tile row past the sequence
end that was not zero-filled, a staging slot read before its write) would
then give NaN, or at least other bits, where the normal build silently
reuses stale data.  Each case runs every kernel it reaches under both
builds and compares the raw bits of all outputs.
"""
from __future__ import annotations

import numpy as np
import pytest

import workloads
from tests import gpu_util as G

pytestmark = pytest.mark.gpu

DEV = "cuda:0"


@pytest.fixture(scope="module", autouse=True)
def gpu_ready():
    import torch
    assert torch.cuda.is_available(), "GPU tests need a GPU"
    import exact_io_aware_amd as fa
    from exact_io_aware_amd import _lib
    assert fa.load().fa_build_flags() == 0
    with _lib.poisoned_lds() as lib:
        assert lib.fa_build_flags() == 1, "libfa_poison.so is not the poisoning build"


def _bits(t):
    import torch
    t = t.contiguous()
    return t.view(torch.int32) if t.element_size() == 4 else t.view(torch.int16)


def _both_builds(run):
    import torch

    from exact_io_aware_amd import _lib
    ref = [t.clone() for t in run()]
    torch.cuda.synchronize()
    with _lib.poisoned_lds():
        got = run()
        torch.cuda.synchronize()
    for i, (a, b) in enumerate(zip(ref, got)):
        assert torch.equal(_bits(a), _bits(b)), f"output {i} differs under poisoned LDS"


def _dev(w):
    return [G.to_device(w[x], w["dtype"], DEV) for x in "qkv"]


def _fwd_run(w, **kw):
    """fa.fwd on w's inputs with NaN-filled O and L made fresh per call."""
    import torch

    import exact_io_aware_amd as fa
    q, k, v = _dev(w)
    cu = cuk = None
    if w["cu_seqlens"] is not None:
        cu = torch.from_numpy(w["cu_seqlens"]).to(DEV)
        ck = w.get("cu_seqlens_k")
        cuk = cu if ck is None else torch.from_numpy(ck).to(DEV)
        kw.update(cu_seqlens=cu, cu_seqlens_k=cuk, max_seqlen=w["N"],
                  max_seqlen_k=w.get("Nk", w["N"]))
    odt = kw.pop("out_dtype", torch.float32)
    packed = kw.pop("packed", False)

    def run():
        out = torch.full(q.shape, float("nan"), device=DEV, dtype=odt)
        lse = torch.full((w["B"], w["Hq"], w["N"]), float("nan"), device=DEV)
        if packed:
            vt = fa.pack_v(v, cu_seqlens=cuk, max_seqlen=kw.get("max_seqlen_k"))
            o, l = fa.fwd(q, k, None, causal=w["causal"], vt=vt, out=out, lse=lse,
                          out_dtype=odt, **kw)
            return o, l, vt
        return fa.fwd(q, k, v, causal=w["causal"], out=out, lse=lse, out_dtype=odt, **kw)

    return run


# (name, inputs, fwd keyword arguments): every forward kernel and path.
def _fwd_cases():
    def fixed(dtype, d, B, Hq, Hkv, n, causal, seed):
        w = workloads.make_custom(B, Hq, Hkv, d, dtype, seed=seed, N=n)
        w["causal"] = causal
        return w

    def qk(dtype, d, B, Hq, Hkv, causal, seed, **kw):
        w = workloads.make_custom_qk(B, Hq, Hkv, d, dtype, seed=seed, **kw)
        w["causal"] = causal
        return w

    def varlen(dtype, d, Hq, Hkv, lens, causal, seed):
        w = workloads.make_custom(len(lens), Hq, Hkv, d, dtype, seed=seed, lengths=lens)
        w["causal"] = causal
        return w

    lens = [300, 1, 777, 64, 0, 129, 512, 33]
    return [
        ("mfma bf16 d128 causal", lambda: fixed("bf16", 128, 2, 8, 2, 333, True, 61), {}),
        ("mfma fp16 d64 causal", lambda: fixed("fp16", 64, 3, 4, 4, 500, True, 62), {}),
        ("mfma bf16 d64", lambda: fixed("bf16", 64, 2, 2, 2, 257, False, 63), {}),
        ("mfma fp16 d128, fp16 O", lambda: fixed("fp16", 128, 2, 6, 3, 190, False, 64),
         {"out_dtype": "in"}),
        ("mfma varlen", lambda: varlen("bf16", 128, 4, 1, lens, True, 65), {}),
        ("chunked prefill", lambda: qk("bf16", 128, 2, 8, 2, True, 66, Nq=100, Nk=700), {}),
        ("decode", lambda: qk("bf16", 128, 3, 8, 2, True, 67, Nq=1, Nk=1500), {}),
        ("decode varlen packed",
         lambda: qk("bf16", 128, 4, 8, 2, True, 68, lengths_q=[1, 2, 1, 1],
                    lengths_k=[100, 2000, 1, 64]), {"packed": True}),
        ("split-KV + merge", lambda: fixed("bf16", 128, 2, 8, 2, 1000, True, 69),
         {"num_splits": 3}),
        ("packed V", lambda: fixed("fp16", 64, 2, 4, 2, 450, True, 70), {"packed": True}),
        ("fp32", lambda: fixed("fp32", 64, 1, 2, 2, 256, False, 71), {}),
        ("fp32 d128 causal", lambda: fixed("fp32", 128, 2, 2, 1, 200, True, 72), {}),
    ]


FWD = _fwd_cases()


@pytest.mark.parametrize("i", range(len(FWD)), ids=[c[0] for c in FWD])
def test_forward_reads_only_lds_it_wrote(i):
    import torch
    name, make, kw = FWD[i]
    w = make()
    kw = dict(kw)
    if kw.get("out_dtype") == "in":
        kw["out_dtype"] = torch.float16 if w["dtype"] == "fp16" else torch.bfloat16
    G.say(f"poisoned LDS: {name}")
    _both_builds(_fwd_run(w, **kw))


def test_block_sparse_reads_only_lds_it_wrote():
    import torch

    import exact_io_aware_amd as fa
    B, Hq, N = 2, 8, 700
    w = workloads.make_custom(B, Hq, 2, 128, "bf16", seed=73, N=N)
    q, k, v = _dev(w)
    nb = (N + 63) // 64
    mask = workloads.random_block_mask(np.random.default_rng(73), B, Hq, N, N, 0.4)
    mask[..., np.arange(nb), np.arange(nb)] = 1
    mb = torch.from_numpy(mask).to(DEV)

    def run():
        out = torch.full(q.shape, float("nan"), device=DEV)
        lse = torch.full((B, Hq, N), float("nan"), device=DEV)
        return fa.fwd(q, k, v, causal=True, block_mask=mb, out=out, lse=lse)

    G.say("poisoned LDS: block-sparse")
    _both_builds(run)


@pytest.mark.parametrize("case", [("bf16", 128, 2, 8, 2, 384), ("fp16", 64, 3, 4, 4, 300),
                                  ("bf16", 128, 4, 4, 1, [200, 1, 450, 0])],
                         ids=["bf16-d128", "fp16-d64", "bf16-d128-varlen"])
def test_backward_reads_only_lds_it_wrote(case):
    import torch

    import exact_io_aware_amd as fa
    dtype, d, B, Hq, Hkv, n = case
    if isinstance(n, list):
        w = workloads.make_custom(B, Hq, Hkv, d, dtype, seed=74, lengths=n)
        kw = dict(cu_seqlens=torch.from_numpy(w["cu_seqlens"]).to(DEV), max_seqlen=max(n))
    else:
        w = workloads.make_custom(B, Hq, Hkv, d, dtype, seed=74, N=n)
        kw = {}
    q, k, v = _dev(w)
    gen = torch.Generator().manual_seed(74)
    do = torch.randn(q.shape, generator=gen).to(q.dtype).to(DEV)
    o, lse = fa.fwd(q, k, v, causal=True, **kw)
    G.say(f"poisoned LDS: backward {case}")
    _both_builds(lambda: fa.bwd(q, k, v, o, lse, do, causal=True, **kw))
