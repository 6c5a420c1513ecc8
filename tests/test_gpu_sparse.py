"""Block-sparse attention on the GPU vs the oracle (fa_fwd_sparse,
fa_fwd_sparse_packed).  Needs an MI355X."""
from __future__ import annotations

import numpy as np
import pytest

import oracle
import workloads
from tests import gpu_util as G

pytestmark = pytest.mark.gpu

# (dtype, d, B, Hq, Hkv, query counts, key counts, causal, mask kind, density);
# lists = packed varlen.  Mask kinds: "one" (one mask for all), "head" (per
# query head), "batch" (per sequence), "both", "stream" (sink + window).
CASES = [
    ("bf16", 128, 2, 8, 2, 300, 300, True, "one", 0.5),
    ("bf16", 128, 2, 8, 2, 257, 257, False, "both", 0.4),
    ("bf16", 64, 1, 4, 4, 333, 333, True, "head", 0.6),
    ("fp16", 128, 1, 4, 1, 130, 130, True, "batch", 0.5),
    ("fp16", 64, 2, 6, 3, 97, 97, False, "head", 0.3),
    ("bf16", 128, 2, 8, 2, 100, 333, True, "head", 0.5),       # queries at the end
    ("bf16", 128, 1, 8, 2, 1024, 1024, True, "stream", 0.0),
    ("bf16", 128, 4, 8, 2, [70, 1, 190, 130], [70, 1, 190, 130], True, "both", 0.5),
    ("fp16", 64, 3, 4, 2, [10, 64, 100], [40, 64, 300], True, "head", 0.6),
    ("bf16", 128, 1, 32, 8, 600, 600, True, "head", 0.15),     # many empty rows
    ("bf16", 128, 3, 8, 2, [50, 0, 80], [50, 0, 80], True, "both", 0.5),  # an empty sequence
]


def _make(case, seed):
    dtype, d, B, Hq, Hkv, nq, nk, causal, kind, dens = case
    if isinstance(nq, list):
        w = workloads.make_custom_qk(B, Hq, Hkv, d, dtype, seed, lengths_q=nq, lengths_k=nk)
    else:
        w = workloads.make_custom_qk(B, Hq, Hkv, d, dtype, seed, Nq=nq, Nk=nk)
    w["causal"] = causal
    w["scale"] = 1.0 / np.sqrt(d)
    rng = np.random.default_rng(seed + 1)
    Bm = B if kind in ("batch", "both") else 1
    Hm = Hq if kind in ("head", "both") else 1
    if kind == "stream":
        w["block_mask"] = workloads.streaming_block_mask(w["N"], 1, 4)
    else:
        w["block_mask"] = workloads.random_block_mask(rng, Bm, Hm, w["N"], w["Nk"], dens)
    return w


def _run(w, out_dtype=None, packed=False, mask=None):
    import torch

    import exact_io_aware_amd as fa
    dev = "cuda:0"
    q, k, v = (G.to_device(w[x], w["dtype"], dev) for x in "qkv")
    cu = cuk = None
    if w["cu_seqlens"] is not None:
        cu = torch.from_numpy(w["cu_seqlens"]).to(dev)
        cuk = torch.from_numpy(w["cu_seqlens_k"]).to(dev)
    bm = torch.from_numpy(np.ascontiguousarray(w["block_mask"] if mask is None else mask)).to(dev)
    lse = torch.full((w["B"], w["Hq"], w["N"]), float("nan"), device=dev)
    # packed: V packed by fa_pack_v first (the *_packed entry points).
    vt = fa.pack_v(v, cu_seqlens=cuk, max_seqlen=w["Nk"] if cuk is not None else None) \
        if packed else None
    o, lse = fa.fwd(q, k, None if packed else v, causal=w["causal"], scale=w["scale"], cu_seqlens=cu,
                    cu_seqlens_k=cuk, max_seqlen=w["N"] if cu is not None else None,
                    max_seqlen_k=w["Nk"] if cu is not None else None,
                    out_dtype=out_dtype or torch.float32, lse=lse, block_mask=bm, vt=vt)
    torch.cuda.synchronize()
    return o.double().cpu().numpy(), lse.double().cpu().numpy()


def _oracle(w, mask=None):
    q, k, v = G.f64_inputs(w)
    return oracle.attention_block_sparse(
        q, k, v, w["block_mask"] if mask is None else mask, causal=w["causal"],
        scale=w["scale"], cu_seqlens_q=w["cu_seqlens"], cu_seqlens_k=w["cu_seqlens_k"])


@pytest.mark.parametrize("i", range(len(CASES)),
                         ids=lambda i: "-".join(map(str, CASES[i][:9])).replace(" ", ""))
def test_sparse_parity(i):
    case = CASES[i]
    w = _make(case, seed=900 + i)
    Oref, Lref = _oracle(w)
    for od in ("fp32", w["dtype"]):
        G.say(f"sparse case {case} out={od}")
        O, L = _run(w, out_dtype=G.torch_dtype(od))
        G.say(f"  errors {G.compare_qk(w, O, L, Oref.copy(), Lref.copy(), od)}")


def test_sparse_all_ones_equals_dense_bitwise():
    """Admitting every block streams the same tiles in the same order as the
    dense kernel: identical O and L."""
    import torch

    import exact_io_aware_amd as fa
    for causal, varlen in ((True, False), (False, False), (True, True)):
        if varlen:
            w = workloads.make_custom(3, 8, 2, 128, "bf16", seed=950, lengths=[100, 1, 300])
        else:
            w = workloads.make_custom(2, 8, 2, 128, "bf16", seed=951, N=333)
        w["Nk"], w["cu_seqlens_k"] = w["N"], w["cu_seqlens"]
        w["causal"], w["scale"] = causal, 128 ** -0.5
        nb = -(-w["N"] // 64)
        ones = np.ones((1, 1, nb, nb), np.uint8)
        G.say(f"all-ones mask vs dense causal={causal} varlen={varlen}")
        O1, L1 = _run(w, mask=ones)
        q, k, v = (G.to_device(w[x], "bf16", "cuda:0") for x in "qkv")
        cu = None if not varlen else torch.from_numpy(w["cu_seqlens"]).to("cuda:0")
        lse = torch.full((w["B"], 8, w["N"]), float("nan"), device="cuda:0")
        o2, l2 = fa.fwd(q, k, v, causal=causal, cu_seqlens=cu,
                        max_seqlen=w["N"] if varlen else None, lse=lse)
        torch.cuda.synchronize()
        assert np.array_equal(O1, o2.double().cpu().numpy())
        assert np.array_equal(np.nan_to_num(L1, nan=7.0),
                              np.nan_to_num(l2.double().cpu().numpy(), nan=7.0))


def test_sparse_empty_mask():
    """No admitted block: every row has O = 0 and L = -inf."""
    w = _make(("bf16", 128, 2, 8, 2, 200, 200, True, "one", 0.5), seed=960)
    G.say("all-zero mask")
    O, L = _run(w, mask=np.zeros_like(w["block_mask"]))
    assert not O.any() and np.isneginf(L).all()


def test_sparse_row_major_matches_packed():
    """fa_fwd_sparse and fa_fwd_sparse_packed: bitwise equal."""
    w = _make(CASES[7], seed=961)
    G.say("fa_fwd_sparse vs fa_fwd_sparse_packed")
    O1, L1 = _run(w)
    O2, L2 = _run(w, packed=True)
    assert np.array_equal(O1, O2)
    assert np.array_equal(np.nan_to_num(L1, nan=7.0), np.nan_to_num(L2, nan=7.0))


def test_streaming_workload_full():
    """The streaming_bf16 workload at full size (B=4, 32 query heads,
    N=4096, sink + 1024-key window), in the launch configuration the bench
    times, against the oracle on every sequence and head."""
    w = workloads.make_inputs("streaming_bf16")
    w["Nk"], w["cu_seqlens_k"] = w["N"], None
    G.say("workload streaming_bf16")
    O, L = _run(w)
    q, k, v = G.f64_inputs(w)
    Oref, Lref = oracle.attention_block_sparse(q, k, v, w["block_mask"], causal=True,
                                               scale=w["scale"],
                                               workers=min(16, oracle.default_workers()))
    assert np.isfinite(O).all() and np.isfinite(L).all()
    eo = np.abs(O - Oref).max()
    el = np.abs(L - Lref).max()
    G.say(f"  errors O {eo:.3e} L {el:.3e}")
    assert eo <= G.O_TOL["bf16"] and el <= G.L_TOL


def test_sparse_longest_tile_list():
    """The longest tile list a workgroup can hold (4096 key tiles: 262144
    keys per sequence).  The last 64-row query block admits every key block;
    every other query block only its own.  Its rows are plain attention over
    all keys (the oracle on those 64 rows); a few diagonal blocks are plain
    attention over their own 64 keys."""
    import torch

    import exact_io_aware_amd as fa
    N, nb = 64 * 4096, 4096
    w = workloads.make_custom(1, 2, 1, 128, "bf16", seed=970, N=N)
    bm = np.eye(nb, dtype=np.uint8)[None, None]
    bm[0, 0, nb - 1, :] = 1
    G.say("sparse: 4096-tile list, N = 262144")
    q, k, v = (G.to_device(w[x], "bf16", "cuda:0") for x in "qkv")
    o, lse = fa.fwd(q, k, v, causal=False, block_mask=torch.from_numpy(bm).to("cuda:0"))
    torch.cuda.synchronize()
    O, L = o.double().cpu().numpy(), lse.double().cpu().numpy()
    qf, kf, vf = G.f64_inputs(w)
    scale = 128 ** -0.5
    Oref, Lref = oracle.attention_qk(qf[:, :, N - 64:], kf, vf, causal=False, scale=scale)
    eo = np.abs(O[:, :, N - 64:] - Oref).max()
    el = np.abs(L[:, :, N - 64:] - Lref).max()
    G.say(f"  last block errors O {eo:.3e} L {el:.3e}")
    assert eo <= G.O_TOL["bf16"] and el <= G.L_TOL
    for i in (0, 1, 2047, 4094):
        sl = slice(64 * i, 64 * i + 64)
        Ob, Lb = oracle.attention(qf[:, :, sl], kf[:, :, sl], vf[:, :, sl], causal=False,
                                  scale=scale)
        assert np.abs(O[:, :, sl] - Ob).max() <= G.O_TOL["bf16"], i
        assert np.abs(L[:, :, sl] - Lb).max() <= G.L_TOL, i
