"""Order independence (needs an MI355X).

Every workgroup of the attention kernels writes only its own rows of O and
L (or of dQ) and reads only the inputs, so the order in which workgroups are
handed out must not change one bit of the result.  Each case runs under the
library's own order and under each forced order (unit-major or
row-block-major, with and without the XCD remap) and compares the raw bits;
a difference would mean a race or a dependence between workgroups.
"""
from __future__ import annotations

import numpy as np
import pytest

import workloads
from tests import gpu_util as G

pytestmark = pytest.mark.gpu

ORDERS = (0, 1, 2, 3)


@pytest.fixture(scope="module", autouse=True)
def gpu_ready():
    import torch
    assert torch.cuda.is_available(), "GPU tests need a GPU"
    import exact_io_aware_amd as fa
    fa.load()
    yield
    fa.debug_force_order(-1)


def _bits(t):
    import torch
    t = t.contiguous()
    return t.view(torch.int32) if t.element_size() == 4 else t.view(torch.int16)


def _same(a, b):
    import torch
    return all(torch.equal(_bits(x), _bits(y)) for x, y in zip(a, b))


def _under_each_order(run):
    """run() under the library's order, then under each forced one."""
    import torch

    import exact_io_aware_amd as fa
    fa.debug_force_order(-1)
    ref = [t.clone() for t in run()]
    torch.cuda.synchronize()
    try:
        for order in ORDERS:
            fa.debug_force_order(order)
            got = run()
            torch.cuda.synchronize()
            assert _same(ref, got), f"order {order} changed the result"
    finally:
        fa.debug_force_order(-1)


def _inputs(dtype, d, B, Hq, Hkv, n, seed):
    if isinstance(n, list):
        w = workloads.make_custom(B, Hq, Hkv, d, dtype, seed=seed, lengths=n)
    else:
        w = workloads.make_custom(B, Hq, Hkv, d, dtype, seed=seed, N=n)
    return w, [G.to_device(w[x], dtype, "cuda:0") for x in "qkv"]


# (dtype, d, B, Hq, Hkv, N or lengths, causal): unit counts that allow the
# XCD remap and ones that do not, GQA packing 4 and 1, ragged tails, varlen
# with an empty and a one-token sequence.
FWD_CASES = [
    ("bf16", 128, 4, 8, 2, 600, True),
    ("bf16", 128, 2, 8, 2, 333, True),
    ("fp16", 64, 8, 4, 4, 500, True),
    ("bf16", 64, 8, 2, 2, 257, False),
    ("fp16", 128, 3, 6, 3, 190, False),
    ("bf16", 128, 8, 4, 1, [300, 1, 777, 64, 0, 129, 512, 33], True),
]


@pytest.mark.parametrize("case", FWD_CASES, ids=lambda c: f"{c[0]}-d{c[1]}-B{c[2]}-c{int(c[6])}")
def test_forward_is_independent_of_workgroup_order(case):
    import torch

    import exact_io_aware_amd as fa
    dtype, d, B, Hq, Hkv, n, causal = case
    w, (q, k, v) = _inputs(dtype, d, B, Hq, Hkv, n, seed=41)
    kw, nmax = {}, n
    if isinstance(n, list):
        nmax = max(n)
        kw = dict(cu_seqlens=torch.from_numpy(w["cu_seqlens"]).to("cuda:0"), max_seqlen=nmax)

    def run():
        # NaN-filled outputs: rows past a packed sequence's end (L of the
        # padding) are never written and must stay as they were.
        out = torch.full(q.shape, float("nan"), device="cuda:0")
        lse = torch.full((B, Hq, nmax), float("nan"), device="cuda:0")
        return fa.fwd(q, k, v, causal=causal, out=out, lse=lse, **kw)

    G.say(f"order independence {case}")
    _under_each_order(run)


def test_split_kv_is_independent_of_workgroup_order():
    import exact_io_aware_amd as fa
    _, (q, k, v) = _inputs("bf16", 128, 2, 8, 2, 1000, seed=42)
    G.say("order independence, split-KV")
    _under_each_order(lambda: fa.fwd(q, k, v, causal=True, num_splits=3))


def test_block_sparse_is_independent_of_workgroup_order():
    import torch

    import exact_io_aware_amd as fa
    B, Hq, N = 4, 8, 700
    _, (q, k, v) = _inputs("bf16", 128, B, Hq, 2, N, seed=43)
    nb = (N + 63) // 64
    rng = np.random.default_rng(43)
    mask = (rng.random((B, Hq, nb, nb)) < 0.5).astype(np.uint8)
    mask[..., np.arange(nb), np.arange(nb)] = 1
    mb = torch.from_numpy(mask).to("cuda:0")
    G.say("order independence, block-sparse")
    _under_each_order(lambda: fa.fwd(q, k, v, causal=True, block_mask=mb))


@pytest.mark.parametrize("case", [("bf16", 128, 4, 8, 2, 384, True),
                                  ("fp16", 64, 8, 4, 4, 300, True),
                                  ("bf16", 128, 8, 4, 1, [200, 1, 450, 64, 0, 97, 256, 31], True)],
                         ids=lambda c: f"{c[0]}-d{c[1]}-B{c[2]}")
def test_backward_is_independent_of_workgroup_order(case):
    import torch

    import exact_io_aware_amd as fa
    dtype, d, B, Hq, Hkv, n, causal = case
    w, (q, k, v) = _inputs(dtype, d, B, Hq, Hkv, n, seed=44)
    kw = {}
    if isinstance(n, list):
        kw = dict(cu_seqlens=torch.from_numpy(w["cu_seqlens"]).to("cuda:0"), max_seqlen=max(n))
    gen = torch.Generator().manual_seed(44)
    do = torch.randn(q.shape, generator=gen).to(q.dtype).to("cuda:0")
    fa.debug_force_order(-1)
    o, lse = fa.fwd(q, k, v, causal=causal, **kw)
    G.say(f"order independence, backward {case}")
    _under_each_order(lambda: fa.bwd(q, k, v, o, lse, do, causal=causal, **kw))
