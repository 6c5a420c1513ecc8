"""fa_fwd_kv_split_noalloc (split-KV partials in the library's fixed device
scratch, for callers that cannot allocate) against fa_fwd_kv_split with a
caller workspace: the same kernels, so bitwise the same O and L, on two
calls in a row (the second smaller, so stale partials of the first would
show).  Called through the C ABI.  Needs an MI355X."""
from __future__ import annotations

import numpy as np
import pytest

import workloads
from tests import gpu_util as G

pytestmark = pytest.mark.gpu


def _inputs(B, Hq, Hkv, Nq, Nk, d, dtype, seed, lens_q=None, lens_k=None):
    if lens_q is not None:
        return workloads.make_custom_qk(B, Hq, Hkv, d, dtype, seed, lengths_q=lens_q,
                                        lengths_k=lens_k)
    return workloads.make_custom_qk(B, Hq, Hkv, d, dtype, seed, Nq=Nq, Nk=Nk)


def _call(w, splits, noalloc):
    import torch

    import exact_io_aware_amd as fa
    from exact_io_aware_amd import _lib
    dev = "cuda:0"
    q, k, v = (G.to_device(w[x], w["dtype"], dev) for x in "qkv")
    cu = cuk = None
    if w["cu_seqlens"] is not None:
        cu = torch.from_numpy(w["cu_seqlens"]).to(dev)
        cuk = torch.from_numpy(w["cu_seqlens_k"]).to(dev)
    o = torch.full(q.shape, float("nan"), device=dev)
    lse = torch.full((w["B"], w["Hq"], w["N"]), float("nan"), device=dev)
    dt = fa.FA_BF16 if w["dtype"] == "bf16" else fa.FA_F16
    st = torch.cuda.current_stream().cuda_stream
    a = (q.data_ptr(), k.data_ptr(), v.data_ptr(), o.data_ptr(), lse.data_ptr(), w["B"],
         w["Hq"], w["Hkv"], w["N"], w["Nk"], w["d"], w["causal"], w["scale"],
         None if cu is None else cu.data_ptr(), None if cuk is None else cuk.data_ptr(), splits)
    if noalloc:
        status = _lib.fwd_kv_split_noalloc_raw(*a, st, dt, fa.FA_F32)
    else:
        part = torch.empty(max(16, fa.split_workspace_bytes(w["B"], w["Hq"], w["N"], w["d"],
                                                             splits)),
                           dtype=torch.uint8, device=dev)
        status = _lib.fwd_kv_split_raw(*a, part.data_ptr(), part.numel(), st, dt, fa.FA_F32)
    torch.cuda.synchronize()
    assert status == 0, _lib.status_string(status)
    return o.cpu().numpy(), lse.cpu().numpy()


def test_split_noalloc_matches_workspace_entry_point():
    cases = [  # (B, Hq, Hkv, Nq, Nk, d, dtype, splits, lens_q, lens_k); the second is smaller
        (4, 32, 8, 1, 3000, 128, "bf16", 12, None, None),
        (2, 8, 2, 2, 700, 64, "fp16", 3, None, None),
        (3, 8, 2, 1, 1000, 128, "bf16", 5, [1, 1, 1], [1000, 37, 512]),
    ]
    for i, (B, Hq, Hkv, Nq, Nk, d, dtype, splits, lq, lk) in enumerate(cases):
        w = _inputs(B, Hq, Hkv, Nq, Nk, d, dtype, seed=900 + i, lens_q=lq, lens_k=lk)
        w["causal"], w["scale"] = True, d ** -0.5
        G.say(f"no-alloc split-KV case {i}: B={B} Hq={Hq} Hkv={Hkv} Nq={Nq} Nk={Nk} d={d} "
              f"{dtype} splits={splits}")
        O1, L1 = _call(w, splits, noalloc=False)
        O2, L2 = _call(w, splits, noalloc=True)
        assert np.array_equal(np.isnan(O1), np.isnan(O2))
        assert np.array_equal(np.nan_to_num(O1, nan=7.0), np.nan_to_num(O2, nan=7.0))
        assert np.array_equal(np.nan_to_num(L1, nan=7.0), np.nan_to_num(L2, nan=7.0))
        if lq is None:
            assert np.isfinite(O2).all() and np.isfinite(L2).all()


def test_split_noalloc_rejects_partials_above_the_scratch():
    import torch

    import exact_io_aware_amd as fa
    from exact_io_aware_amd import _lib
    cap = _lib.noalloc_scratch_bytes()
    B, Hq, Hkv, Nq, Nk, d, splits = 64, 32, 8, 8, 256, 128, 8
    assert fa.split_workspace_bytes(B, Hq, Nq, d, splits) > cap
    dev = "cuda:0"
    q = torch.zeros((B, Hq, Nq, d), dtype=torch.bfloat16, device=dev)
    k = torch.zeros((B, Hkv, Nk, d), dtype=torch.bfloat16, device=dev)
    o = torch.full((B, Hq, Nq, d), float("nan"), device=dev)
    lse = torch.empty((B, Hq, Nq), device=dev)
    G.say("no-alloc split-KV above the scratch size")
    st = _lib.fwd_kv_split_noalloc_raw(q.data_ptr(), k.data_ptr(), k.data_ptr(), o.data_ptr(),
                                       lse.data_ptr(), B, Hq, Hkv, Nq, Nk, d, 1, 0.1, None, None,
                                       splits, torch.cuda.current_stream().cuda_stream,
                                       fa.FA_BF16, fa.FA_F32)
    torch.cuda.synchronize()
    assert st == _lib.STATUS["FA_ERR_SCRATCH"]
    assert torch.isnan(o).all()              # nothing was launched
