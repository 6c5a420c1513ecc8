"""Decode on the GPU vs the oracle: a few new queries per sequence against a
long key/value cache, with the keys split across workgroups and the partial
results merged through their logsumexps (split-KV).  Needs an MI355X."""
from __future__ import annotations

import pytest

import oracle
import workloads
from tests import gpu_util as G
from tests.test_gpu_prefill import _make, _oracle

pytestmark = pytest.mark.gpu


def _run(w, num_splits=None, out_dtype=None, packed=False):
    import torch

    import exact_io_aware_amd as fa
    dev = "cuda:0"
    q, k, v = (G.to_device(w[x], w["dtype"], dev) for x in "qkv")
    cu = cuk = None
    if w["cu_seqlens"] is not None:
        cu = torch.from_numpy(w["cu_seqlens"]).to(dev)
        cuk = torch.from_numpy(w["cu_seqlens_k"]).to(dev)
    lse = torch.full((w["B"], w["Hq"], w["N"]), float("nan"), device=dev)
    # packed: the K/V cache's V kept packed (fa_pack_v; the *_packed entry
    # points); otherwise V itself is read and transposed on chip.
    vt = fa.pack_v(v, cu_seqlens=cuk, max_seqlen=w["Nk"] if cuk is not None else None) \
        if packed else None
    o, lse = fa.fwd(q, k, None if packed else v, causal=w["causal"], scale=w["scale"],
                    cu_seqlens=cu, vt=vt,
                    cu_seqlens_k=cuk, max_seqlen=w["N"] if cu is not None else None,
                    max_seqlen_k=w["Nk"] if cu is not None else None,
                    out_dtype=out_dtype or torch.float32, lse=lse, num_splits=num_splits)
    torch.cuda.synchronize()
    return o.double().cpu().numpy(), lse.double().cpu().numpy()


DECODE = [
    ("bf16", 128, 4, 32, 8, 1, 2000, True),
    ("bf16", 128, 2, 8, 2, 4, 1500, True),        # four new tokens (speculative step)
    ("fp16", 64, 3, 8, 8, 1, 777, True),
    ("bf16", 128, 5, 8, 2, [1, 1, 1, 1, 1], [100, 3000, 1, 64, 777], True),
    ("fp16", 128, 3, 4, 1, [2, 1, 3], [513, 2, 1000], False),
    # Shapes of the decode kernel's edges (G * nq <= 32 rows in one block):
    ("bf16", 128, 2, 32, 4, 4, 700, True),        # G * nq = 32, a full block
    ("fp16", 128, 3, 16, 2, [1, 3, 2], [1, 60, 130], True),   # one key; one partial tile
    ("bf16", 64, 3, 8, 4, [2, 2, 1], [0, 5, 64], True),       # a sequence with no keys
    ("fp16", 64, 2, 8, 8, 3, 2, True),            # fewer keys than queries: row 0 sees none
    ("bf16", 128, 2, 8, 2, 5, 1000, False),
    ("bf16", 128, 2, 32, 1, 1, 3000, True),       # one K/V head for 32 query heads
    ("fp16", 64, 2, 16, 1, 2, 900, True),         # G = 16, two queries: 32 rows
]


@pytest.mark.parametrize("i", range(len(DECODE)),
                         ids=lambda i: "-".join(map(str, DECODE[i][:7])).replace(" ", ""))
def test_decode_parity_auto_splits(i):
    case = DECODE[i]
    w = _make(case, seed=800 + i)
    Oref, Lref = _oracle(w)
    for od in ("fp32", w["dtype"]):
        for packed in (False, True):
            G.say(f"decode case {case} out={od} packed={packed}")
            O, L = _run(w, out_dtype=G.torch_dtype(od), packed=packed)
            G.say(f"  errors {G.compare_qk(w, O, L, Oref.copy(), Lref.copy(), od)}")


@pytest.mark.parametrize("splits", [1, 2, 3, 7, 16, 40])
def test_decode_explicit_splits(splits):
    """Every split count gives the exact result, including counts with
    empty splits (more splits than the shortest sequence has tiles)."""
    w = _make(("bf16", 128, 3, 8, 2, [1, 2, 1], [2500, 70, 640], True), seed=850)
    Oref, Lref = _oracle(w)
    for packed in (False, True):
        G.say(f"decode with {splits} splits packed={packed}")
        O, L = _run(w, num_splits=splits, packed=packed)
        G.say(f"  errors {G.compare_qk(w, O, L, Oref.copy(), Lref.copy())}")


def test_splits_on_prefill_shape():
    """Split-KV applied to a many-query shape agrees with the unsplit call."""
    w = _make(("bf16", 128, 2, 8, 2, 200, 900, True), seed=851)
    Oref, Lref = _oracle(w)
    for splits in (1, 4):
        G.say(f"prefill shape with {splits} splits")
        O, L = _run(w, num_splits=splits)
        G.say(f"  errors {G.compare_qk(w, O, L, Oref, Lref)}")


def test_num_splits_heuristic():
    import exact_io_aware_amd as fa
    assert fa.num_splits(4, 32, 8, 1, 8192, 128, fa.FA_BF16) > 1       # small decode: split
    assert fa.num_splits(32, 32, 8, 1, 8192, 128, fa.FA_BF16) == 1     # one workgroup per CU
    assert fa.num_splits(4, 32, 8, 4096, 4096, 128, fa.FA_BF16) == 1   # prefill: no split
    assert fa.num_splits(4, 32, 8, 1, 8192, 128, fa.FA_F32) == 1        # fp32: never


def test_decode_workload_full():
    """decode_bf16 at full size (32 sequences, 8192-token cache): the oracle on
    every sequence and head."""
    w = workloads.make_inputs("decode_bf16")
    G.say("workload decode_bf16")
    O, L = _run(w)
    q, k, v = G.f64_inputs(w)
    Oref, Lref = oracle.attention_qk(q, k, v, causal=True, scale=w["scale"],
                                     workers=min(16, oracle.default_workers()))
    w1 = dict(w, cu_seqlens=None)
    G.say(f"  errors {G.compare_qk(w1, O, L, Oref, Lref)}")
