"""Chunked prefill on the GPU vs the oracle: each sequence's queries are its
last tokens and attend to a longer key/value prefix (fa_fwd_kv,
fa_fwd_kv_packed).  Needs an MI355X."""
from __future__ import annotations

import numpy as np
import pytest

import oracle
import workloads
from tests import gpu_util as G

pytestmark = pytest.mark.gpu

# (dtype, d, B, Hq, Hkv, query counts, key counts, causal); lists = varlen
CASES = [
    ("bf16", 128, 2, 8, 2, 100, 333, True),
    ("bf16", 128, 2, 8, 2, 100, 333, False),
    ("bf16", 128, 1, 8, 1, 1, 517, True),          # one query: a decode step
    ("fp16", 64, 2, 4, 4, 65, 200, True),
    ("fp16", 64, 1, 4, 2, 200, 130, True),         # more queries than keys
    ("fp32", 64, 1, 2, 2, 50, 160, True),
    ("fp32", 128, 1, 4, 2, 33, 97, False),
    ("bf16", 128, 3, 8, 2, [5, 64, 100], [300, 64, 101], True),
    ("fp16", 64, 3, 4, 2, [10, 1, 70], [40, 0, 30], True),   # a sequence with no keys
    ("fp32", 64, 2, 2, 1, [17, 40], [90, 41], True),
]


def _make(case, seed):
    dtype, d, B, Hq, Hkv, nq, nk, causal = case
    if isinstance(nq, list):
        w = workloads.make_custom_qk(B, Hq, Hkv, d, dtype, seed, lengths_q=nq, lengths_k=nk)
    else:
        w = workloads.make_custom_qk(B, Hq, Hkv, d, dtype, seed, Nq=nq, Nk=nk)
    w["causal"] = causal
    w["scale"] = 1.0 / np.sqrt(d)
    return w


def _run(w, out_dtype=None, packed=False):
    import torch

    import exact_io_aware_amd as fa
    dev = "cuda:0"
    q, k, v = (G.to_device(w[x], w["dtype"], dev) for x in "qkv")
    cu = cuk = None
    if w["cu_seqlens"] is not None:
        cu = torch.from_numpy(w["cu_seqlens"]).to(dev)
        cuk = torch.from_numpy(w["cu_seqlens_k"]).to(dev)
    lse = torch.full((w["B"], w["Hq"], w["N"]), float("nan"), device=dev)
    # packed: V packed by fa_pack_v first (the *_packed entry points).
    vt = fa.pack_v(v, cu_seqlens=cuk, max_seqlen=w["Nk"] if cuk is not None else None) \
        if packed else None
    o, lse = fa.fwd(q, k, None if packed else v, causal=w["causal"], scale=w["scale"], cu_seqlens=cu,
                    cu_seqlens_k=cuk, max_seqlen=w["N"] if cu is not None else None,
                    max_seqlen_k=w["Nk"] if cu is not None else None,
                    out_dtype=out_dtype or torch.float32, lse=lse, vt=vt)
    torch.cuda.synchronize()
    return o.double().cpu().numpy(), lse.double().cpu().numpy()


def _oracle(w):
    q, k, v = G.f64_inputs(w)
    return oracle.attention_qk(q, k, v, causal=w["causal"], scale=w["scale"],
                               cu_seqlens_q=w["cu_seqlens"], cu_seqlens_k=w["cu_seqlens_k"])


@pytest.mark.parametrize("i", range(len(CASES)),
                         ids=lambda i: "-".join(map(str, CASES[i][:7])).replace(" ", ""))
def test_prefill_parity(i):
    case = CASES[i]
    w = _make(case, seed=700 + i)
    Oref, Lref = _oracle(w)
    outs = ["fp32"] if w["dtype"] == "fp32" else ["fp32", w["dtype"]]
    for od in outs:
        G.say(f"prefill case {case} out={od}")
        O, L = _run(w, out_dtype=G.torch_dtype(od))
        G.say(f"  errors {G.compare_qk(w, O, L, Oref, Lref, od)}")


def test_prefill_row_major_matches_packed():
    """fa_fwd_kv (V read transposed on chip) and fa_fwd_kv_packed (V packed by
    fa_pack_v) feed the same operands to the same products: bitwise equal."""
    w = _make(("bf16", 128, 3, 8, 2, [5, 64, 100], [300, 64, 101], True), seed=760)
    G.say("fa_fwd_kv vs fa_fwd_kv_packed")
    O1, L1 = _run(w)
    O2, L2 = _run(w, packed=True)
    assert np.array_equal(O1, O2)
    assert np.array_equal(np.nan_to_num(L1, nan=7.0), np.nan_to_num(L2, nan=7.0))


def test_chunks_reassemble_full_sequence():
    """The manual chunking recipe on the GPU: four query chunks of a
    1000-token causal sequence, each against its key prefix, agree with the
    rows of one full-sequence call."""
    import torch

    import exact_io_aware_amd as fa
    w = workloads.make_custom(1, 8, 2, 128, "bf16", seed=761, N=1000)
    q, k, v = (G.to_device(w[x], "bf16", "cuda:0") for x in "qkv")
    G.say("chunks vs full sequence")
    of, lf = fa.fwd(q, k, v, causal=True)
    for i0, c in ((0, 250), (250, 250), (500, 333), (833, 167)):
        qc = q[:, :, i0:i0 + c].contiguous()
        kc = k[:, :, :i0 + c].contiguous()
        vc = v[:, :, :i0 + c].contiguous()
        oc, lc = fa.fwd(qc, kc, vc, causal=True)
        torch.cuda.synchronize()
        assert (oc - of[:, :, i0:i0 + c]).abs().max().item() <= 8e-3
        assert (lc - lf[:, :, i0:i0 + c]).abs().max().item() <= 1e-4


def test_zigzag_share_workload_full():
    """long_bf16_sp8 (one GPU's zig-zag share of long_bf16: 2048 queries
    against 2048 keys and 2048 queries against 32768 keys, packed) at full
    size, every row of every head against the oracle."""
    w = workloads.make_inputs("long_bf16_sp8")
    G.say("workload long_bf16_sp8")
    O, L = _run(w)
    q, k, v = G.f64_inputs(w)
    Oref, Lref = oracle.attention_qk(q, k, v, causal=True, scale=w["scale"],
                                     cu_seqlens_q=w["cu_seqlens"],
                                     cu_seqlens_k=w["cu_seqlens_k"],
                                     workers=min(16, oracle.default_workers()))
    G.say(f"  errors {G.compare_qk(w, O, L, Oref, Lref)}")


def test_prefill_workload_full():
    """The prefill_bf16 workload at full size (B=4, 32 query heads, the last
    1024 queries of 8192-token sequences), checked against the oracle on
    every sequence and head."""
    w = workloads.make_inputs("prefill_bf16")
    G.say("workload prefill_bf16")
    O, L = _run(w)
    q, k, v = G.f64_inputs(w)
    Oref, Lref = oracle.attention_qk(q, k, v, causal=True, scale=w["scale"],
                                     workers=min(16, oracle.default_workers()))
    w1 = dict(w, cu_seqlens=None)
    G.say(f"  errors {G.compare_qk(w1, O, L, Oref, Lref)}")
