"""HIP path vs the CPU oracle on the same seeded inputs (needs an MI355X).

Element by element at sizes the oracle finishes in seconds (several tiles,
ragged tails, every dtype / head dim / GQA packing / varlen form), the full
headline workloads, and sampled rows of the largest ones.
"""
from __future__ import annotations

import numpy as np
import pytest

import oracle
import workloads
from tests import gpu_util as G

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def gpu_ready():
    import torch
    assert torch.cuda.is_available(), "GPU tests need a GPU"
    import exact_io_aware_amd as fa
    fa.load()
    name = torch.cuda.get_device_properties(0).gcnArchName
    assert name.startswith("gfx950"), name


def _compare(w, O, L, Oref, Lref, out_dtype="fp32", strict=None, bar=None):
    eo = np.abs(O - Oref)
    if bar is None:
        bar = G.o_bar(w["dtype"], out_dtype, Oref)
    worst_o = float(eo.max()) if eo.size else 0.0
    assert np.isfinite(O).all()
    assert (eo <= bar).all(), f"O error {worst_o:.3e}"
    el = np.abs(L - Lref)
    worst_l = float(np.nanmax(el)) if el.size else 0.0
    assert worst_l <= G.L_TOL, f"L error {worst_l:.3e}"
    if strict is not None:
        assert worst_o <= strict and worst_l <= strict, (worst_o, worst_l)
    return worst_o, worst_l


# (dtype, d, B, Hq, Hkv, N or list of lengths, causal)
MEDIUM = [
    ("bf16", 128, 2, 8, 2, 333, True),
    ("bf16", 128, 2, 8, 2, 333, False),
    ("bf16", 128, 1, 8, 1, 257, True),     # 8 query heads per K/V head
    ("bf16", 64, 1, 4, 4, 517, True),
    ("bf16", 64, 1, 3, 1, 17, False),      # 3 query heads per K/V head
    ("fp16", 64, 2, 6, 6, 300, True),
    ("fp16", 128, 1, 6, 3, 200, False),    # 2 query heads per K/V head
    ("fp16", 128, 1, 2, 2, 1, True),       # a single token
    ("fp16", 64, 1, 2, 1, 129, True),
    ("fp32", 64, 1, 2, 2, 256, False),
    ("fp32", 128, 2, 4, 2, 150, True),
    ("fp32", 64, 1, 4, 4, 70, True),
    ("bf16", 128, 5, 8, 2, [1, 129, 64, 300, 33], True),
    ("bf16", 64, 3, 4, 2, [200, 7, 128], False),
    ("fp16", 128, 3, 4, 4, [65, 1, 190], True),
    ("fp32", 64, 2, 2, 1, [31, 90], True),
    ("bf16", 128, 3, 8, 2, [100, 0, 64], True),      # an empty sequence
    ("fp32", 64, 3, 2, 1, [0, 40, 0], False),
]


def _make(case, seed):
    dtype, d, B, Hq, Hkv, n, causal = case
    if isinstance(n, list):
        w = workloads.make_custom(B, Hq, Hkv, d, dtype, seed=seed, lengths=n)
    else:
        w = workloads.make_custom(B, Hq, Hkv, d, dtype, seed=seed, N=n)
    w["causal"] = causal
    w["scale"] = 1.0 / np.sqrt(d)
    return w


def _oracle(w):
    q, k, v = G.f64_inputs(w)
    return oracle.attention(q, k, v, causal=w["causal"], scale=w["scale"],
                            cu_seqlens=w["cu_seqlens"])


@pytest.mark.parametrize("i", range(len(MEDIUM)), ids=lambda i: "-".join(map(str, MEDIUM[i][:5])))
def test_medium_parity(i):
    case = MEDIUM[i]
    w = _make(case, seed=500 + i)
    Oref, Lref = _oracle(w)
    outs = ["fp32"] if w["dtype"] == "fp32" else ["fp32", w["dtype"]]
    for od in outs:
        G.say(f"medium case {case} out={od}")
        O, L = G.run_gpu(w, out_dtype=G.torch_dtype(od), lse_fill=float("nan"))
        if w["cu_seqlens"] is not None:
            lens = np.diff(w["cu_seqlens"])
            for b, n in enumerate(lens):
                assert np.isnan(L[b, :, n:]).all(), "padded lse rows must stay untouched"
                L[b, :, n:] = Lref[b, :, n:] = 0.0
        strict = G.FP32_STRICT if w["dtype"] == "fp32" else None
        G.say(f"  errors {_compare(w, O, L, Oref, Lref, od, strict)}")


def test_tiny_fp32_workload_full():
    w = workloads.make_inputs("tiny_fp32")
    G.say("workload tiny_fp32")
    O, L = G.run_gpu(w)
    Oref, Lref = _oracle(w)
    G.say(f"  errors {_compare(w, O, L, Oref, Lref, strict=G.FP32_STRICT)}")


@pytest.mark.parametrize("name", ["mha_fp16", "gqa_bf16"])
def test_workload_full(name):
    w = workloads.make_inputs(name)
    G.say(f"workload {name}")
    O, L = G.run_gpu(w)
    q, k, v = G.f64_inputs(w)
    Oref, Lref = oracle.attention(q, k, v, causal=w["causal"], scale=w["scale"],
                                  workers=min(16, oracle.default_workers()))
    G.say(f"  errors {_compare(w, O, L, Oref, Lref)}")


def _picks_fixed(w, rng, per_head=12):
    N = w["N"]
    fixed = [0, 1, 31, 32, 63, 64, 65, 127, 128, N // 2, N - 2, N - 1]
    picks = []
    for b in range(w["B"]):
        for h in range(w["Hq"]):
            rows = set(r for r in fixed if 0 <= r < N)
            rows |= set(rng.integers(0, N, per_head).tolist())
            picks += [(b, h, r) for r in sorted(rows)]
    return picks


def _picks_varlen(w, rng, per_head=4):
    picks = []
    lens = np.diff(w["cu_seqlens"])
    for b, n in enumerate(lens):
        for h in range(w["Hq"]):
            rows = {0, 1, int(n) - 1, int(n) // 2} | set(rng.integers(0, n, per_head).tolist())
            picks += [(b, h, r) for r in sorted(rows) if 0 <= r < n]
    return picks


@pytest.mark.parametrize("name", ["long_bf16", "varlen_bf16"])
def test_workload_sampled_rows(name):
    w = workloads.make_inputs(name)
    G.say(f"workload {name}")
    O, L = G.run_gpu(w, lse_fill=float("nan"))
    rng = np.random.default_rng(99)
    q, k, v = G.f64_inputs(w)
    if w["cu_seqlens"] is None:
        picks = _picks_fixed(w, rng)
        got_o = np.stack([O[b, h, r] for b, h, r in picks])
    else:
        picks = _picks_varlen(w, rng)
        cu = w["cu_seqlens"]
        got_o = np.stack([O[cu[b] + r, h] for b, h, r in picks])
        lens = np.diff(cu)
        for b, n in enumerate(lens):
            assert np.isnan(L[b, :, n:]).all()
            assert np.isfinite(L[b, :, :n]).all()
    got_l = np.array([L[b, h, r] for b, h, r in picks])
    Oref, Lref = oracle.attention_rows(q, k, v, causal=w["causal"], scale=w["scale"],
                                       picks=picks, cu_seqlens=w["cu_seqlens"])
    G.say(f"  {len(picks)} rows, errors {_compare(w, got_o, got_l, Oref, Lref)}")
    assert np.isfinite(O).all()


# --- invariants ------------------------------------------------------------

def test_deterministic_and_overwrites_output():
    import torch

    import exact_io_aware_amd as fa
    w = _make(("bf16", 128, 2, 8, 2, 700, True), seed=1)
    q, k, v = (G.to_device(w[x], "bf16", "cuda:0") for x in "qkv")
    G.say("determinism case")
    out = torch.full(q.shape, float("nan"), device="cuda:0")
    o1, l1 = fa.fwd(q, k, v, causal=True, out=out)
    o2, l2 = fa.fwd(q, k, v, causal=True)
    torch.cuda.synchronize()
    assert not torch.isnan(o1).any()
    assert torch.equal(o1, o2) and torch.equal(l1, l2)


def test_gqa_equals_repeated_heads():
    import torch

    import exact_io_aware_amd as fa
    w = _make(("bf16", 128, 1, 8, 2, 300, True), seed=2)
    q, k, v = (G.to_device(w[x], "bf16", "cuda:0") for x in "qkv")
    G.say("gqa vs repeated heads")
    o1, l1 = fa.fwd(q, k, v, causal=True)
    kr = k.repeat_interleave(4, dim=1).contiguous()
    vr = v.repeat_interleave(4, dim=1).contiguous()
    o2, l2 = fa.fwd(q, kr, vr, causal=True)
    torch.cuda.synchronize()
    assert (o1 - o2).abs().max().item() <= 1e-6
    assert (l1 - l2).abs().max().item() <= 1e-6


def test_varlen_equals_each_sequence_alone():
    import torch

    import exact_io_aware_amd as fa
    lens = [70, 1, 250]
    w = workloads.make_custom(3, 4, 2, 128, "bf16", seed=3, lengths=lens)
    q, k, v = (G.to_device(w[x], "bf16", "cuda:0") for x in "qkv")
    cu = torch.from_numpy(w["cu_seqlens"]).to("cuda:0")
    G.say("varlen vs per-sequence")
    o, l = fa.fwd(q, k, v, causal=True, cu_seqlens=cu, max_seqlen=max(lens))
    for b, n in enumerate(lens):
        s = int(w["cu_seqlens"][b])
        qs, ks, vs = (t[s:s + n].transpose(0, 1).unsqueeze(0).contiguous() for t in (q, k, v))
        ob, lb = fa.fwd(qs, ks, vs, causal=True)
        torch.cuda.synchronize()
        assert (o[s:s + n] - ob[0].transpose(0, 1)).abs().max().item() <= 1e-6
        assert (l[b, :, :n] - lb[0]).abs().max().item() <= 1e-6


def test_causal_row0_is_v0():
    w = _make(("bf16", 128, 2, 8, 2, 129, True), seed=4)
    G.say("causal row 0")
    O, L = G.run_gpu(w)
    q, k, v = G.f64_inputs(w)
    for h in range(8):
        g = h // 4
        assert np.allclose(O[:, h, 0], v[:, g, 0], rtol=1e-6, atol=1e-7)
        assert np.allclose(L[:, h, 0], w["scale"] * np.einsum("bd,bd->b", q[:, h, 0], k[:, g, 0]),
                           atol=1e-5)


def _scaled_case(mult, seed, ramp=False):
    w = workloads.make_custom(1, 4, 2, 128, "bf16", seed=seed, N=600)
    q = workloads.bf16_bits_to_f32(w["q"]) * mult
    k = workloads.bf16_bits_to_f32(w["k"]) * mult
    if ramp:  # later keys score ever higher: the running max moves often
        k = k * np.linspace(0.2, 3.0, 600, dtype=np.float32)[None, None, :, None]
        q = np.abs(q)
        k = np.abs(k)
    w["q"] = workloads.round_to_bf16_bits(q)
    w["k"] = workloads.round_to_bf16_bits(k)
    w["causal"] = True
    w["scale"] = 1.0 / np.sqrt(128)
    return w


@pytest.mark.parametrize("mult,ramp", [(4.0, False), (12.0, False), (1.0, True), (3.0, True)])
def test_large_and_growing_scores(mult, ramp):
    w = _scaled_case(mult, seed=int(mult * 10) + ramp, ramp=ramp)
    G.say(f"scaled scores x{mult} ramp={ramp}")
    O, L = G.run_gpu(w)
    Oref, Lref = _oracle(w)
    q, k, v = G.f64_inputs(w)
    A, _ = oracle.attention(q, k, np.abs(v), causal=w["causal"], scale=w["scale"])
    G.say(f"  errors {_compare(w, O, L, Oref, Lref, bar=G.o_bar_derived('bf16', A))}")


def test_kernel_reported():
    import exact_io_aware_amd as fa
    assert fa.kernel_name(fa.FA_BF16, 128, True, False, fa.FA_F32) == \
        "fa_fwd_mfma_bf16_d128_causal_of32"
    assert fa.kernel_name(fa.FA_F32, 64, False, True, fa.FA_F32) == "fa_fwd_f32_d64_varlen"


# --- packed V (fa_pack_v / fa_fwd_packed / fa_fwd's own workspace) ----------

def _vt_expected(v16: np.ndarray, lens, Hkv: int, d: int, ntiles: int):
    """The packed layout fa.h documents, built with numpy from the uint16
    bit patterns of V ([B, Hkv, N, d] views per sequence).  Returns
    {(b, g, t): uint16 [d, 64]} for the tiles that hold keys."""
    j = np.arange(16)
    key_of_pos = (j % 4) + 8 * ((j // 4) % 2) + 4 * (j // 8)
    order = (16 * (np.arange(64) // 16) + key_of_pos[np.arange(64) % 16])
    out = {}
    for b, n in enumerate(lens):
        for g in range(Hkv):
            for t in range((n + 63) // 64):
                tile = np.zeros((64, d), np.uint16)
                keys = np.arange(64 * t, min(64 * t + 64, n))
                tile[keys - 64 * t] = v16[b][g][keys]
                out[(b, g, t)] = tile[order].T
    return out


@pytest.mark.parametrize("dtype,d,lens,varlen", [
    ("bf16", 128, [130, 130], False), ("fp16", 64, [70, 1, 130], True),
    ("bf16", 64, [64, 200], True), ("fp16", 128, [1], False)])
def test_pack_v_layout(dtype, d, lens, varlen):
    import torch

    import exact_io_aware_amd as fa
    Hkv = 3
    if varlen:
        w = workloads.make_custom(len(lens), Hkv, Hkv, d, dtype, seed=7, lengths=lens)
    else:
        w = workloads.make_custom(len(lens), Hkv, Hkv, d, dtype, seed=7, N=lens[0])
    N = max(lens)
    v16 = np.ascontiguousarray(w["v"]).view(np.uint16)
    if varlen:
        cu = w["cu_seqlens"]
        per = [v16[cu[b]:cu[b + 1]].transpose(1, 0, 2) for b in range(len(lens))]
    else:
        per = [v16[b] for b in range(len(lens))]
    ntiles = (N + 63) // 64
    want = _vt_expected(per, lens, Hkv, d, ntiles)
    v = G.to_device(w["v"], dtype, "cuda:0")
    cu_t = torch.from_numpy(w["cu_seqlens"]).to("cuda:0") if varlen else None
    G.say(f"pack_v {dtype} d={d} lens={lens} varlen={varlen}")
    ws = fa.pack_v(v, cu_seqlens=cu_t, max_seqlen=N if varlen else None)
    torch.cuda.synchronize()
    assert ws.numel() == fa.workspace_bytes(len(lens), Hkv, N, d,
                                            fa.FA_BF16 if dtype == "bf16" else fa.FA_F16)
    got = ws.cpu().numpy().view(np.uint16).reshape(len(lens), Hkv, ntiles, d, 64)
    for (b, g, t), tile in want.items():
        assert np.array_equal(got[b, g, t], tile), (b, g, t)


def test_packed_reuse_and_library_workspace_agree():
    import torch

    import exact_io_aware_amd as fa
    w = _make(("bf16", 128, 2, 8, 2, 333, True), seed=11)
    q, k, v = (G.to_device(w[x], "bf16", "cuda:0") for x in "qkv")
    G.say("packed vt reuse vs fa_fwd workspace")
    o1, l1 = fa.fwd(q, k, v, causal=True)
    vt = fa.pack_v(v)
    o2, l2 = fa.fwd(q, k, None, causal=True, vt=vt)
    o3, l3 = fa.fwd(q, k, None, causal=True, vt=vt)
    o4, l4 = fa.fwd(q, k, v, causal=True, library_workspace=True)
    torch.cuda.synchronize()
    for o, l in ((o2, l2), (o3, l3), (o4, l4)):
        assert torch.equal(o1, o) and torch.equal(l1, l)
    Oref, Lref = _oracle(w)
    _compare(w, o4.double().cpu().numpy(), l4.double().cpu().numpy(), Oref, Lref)


def test_library_workspace_varlen_fp16():
    w = _make(("fp16", 64, 3, 4, 2, [200, 7, 128], True), seed=12)
    Oref, Lref = _oracle(w)
    import torch

    import exact_io_aware_amd as fa
    q, k, v = (G.to_device(w[x], "fp16", "cuda:0") for x in "qkv")
    cu = torch.from_numpy(w["cu_seqlens"]).to("cuda:0")
    G.say("fa_fwd own workspace, varlen fp16")
    o, l = fa.fwd(q, k, v, causal=True, cu_seqlens=cu, max_seqlen=200, library_workspace=True)
    torch.cuda.synchronize()
    L = l.double().cpu().numpy()
    for b, n in enumerate(np.diff(w["cu_seqlens"])):
        L[b, :, n:] = Lref[b, :, n:] = 0.0
    _compare(w, o.double().cpu().numpy(), L, Oref, Lref)


def test_no_score_matrix_in_device_memory():
    """The O(N) memory claim: a call allocates no N x N scores.  With V
    already packed the call allocates nothing beyond o and lse; the default
    path adds only the packed-V workspace (the size of V)."""
    import torch

    import exact_io_aware_amd as fa
    w = workloads.make_inputs("gqa_bf16")
    q, k, v = (G.to_device(w[x], "bf16", "cuda:0") for x in "qkv")
    o = torch.empty(q.shape, dtype=torch.float32, device="cuda:0")
    lse = torch.empty((w["B"], w["Hq"], w["N"]), dtype=torch.float32, device="cuda:0")
    vt = fa.pack_v(v)
    G.say("device memory during a call")
    torch.cuda.synchronize()
    torch.cuda.reset_peak_memory_stats()
    base = torch.cuda.memory_allocated()
    fa.fwd(q, k, None, causal=True, out=o, lse=lse, vt=vt)
    torch.cuda.synchronize()
    assert torch.cuda.max_memory_allocated() - base == 0
    torch.cuda.reset_peak_memory_stats()
    base = torch.cuda.memory_allocated()
    fa.fwd(q, k, v, causal=True, out=o, lse=lse)
    torch.cuda.synchronize()
    delta = torch.cuda.max_memory_allocated() - base
    ws = fa.workspace_bytes(w["B"], w["Hkv"], w["N"], w["d"], fa.FA_BF16)
    assert ws == v.numel() * 2
    assert delta <= ws + (2 << 20)
    scores = w["B"] * w["Hq"] * w["N"] * w["N"] * 2          # one bf16 score matrix
    assert delta * 100 < scores
