"""HIP path vs the CPU oracle on the same seeded inputs (needs an MI355X).

Element by element at sizes the oracle finishes in seconds (several tiles,
ragged tails, every dtype / head dim / GQA packing / varlen form) and all
five workloads in full (every row of every head), in the bench's launch
configuration.
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
    """Element-wise bars.  Every output the oracle defines must have been
    written: O finite everywhere, L finite wherever the oracle's is (callers
    pre-fill L with NaN, so a row the kernel skipped fails here), and no NaN
    can hide in a maximum."""
    assert O.shape == Oref.shape and L.shape == Lref.shape
    assert np.isfinite(O).all(), "non-finite O"
    fin = np.isfinite(Lref)
    assert np.isfinite(L[fin]).all(), "an L row the oracle defines is missing or not finite"
    assert np.array_equal(np.isneginf(L), np.isneginf(Lref)), "rows without keys"
    eo = np.abs(O - Oref)
    if bar is None:
        bar = G.o_bar(w["dtype"], out_dtype, Oref)
    worst_o = float(eo.max()) if eo.size else 0.0
    assert (eo <= bar).all(), f"O error {worst_o:.3e}"
    el = np.abs(np.where(fin, L - Lref, 0.0))
    worst_l = float(el.max()) if el.size else 0.0
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
    # Units (sequence x group of 4 query heads) a multiple of 8: the launch
    # deals each unit's workgroups to one XCD (non-causal, and causal d=64).
    ("bf16", 128, 2, 16, 4, 333, False),
    ("fp16", 64, 4, 8, 2, 200, True),
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


def test_causal_unit_major_varlen():
    """A causal varlen launch more than 4 rounds of workgroups deep takes the
    unit-major order with each unit on one XCD (8 sequences x 8 groups of 4
    query heads, row blocks of 64 rows: 1152 workgroups)."""
    lens = [1100, 700, 1030, 900, 64, 1, 1099, 512]
    w = workloads.make_custom(8, 32, 8, 128, "bf16", seed=520, lengths=lens)
    w["causal"], w["scale"] = True, 128 ** -0.5
    q, k, v = G.f64_inputs(w)
    Oref, Lref = oracle.attention(q, k, v, causal=True, scale=w["scale"],
                                  cu_seqlens=w["cu_seqlens"],
                                  workers=min(16, oracle.default_workers()))
    G.say("causal varlen, unit-major order")
    O, L = G.run_gpu(w, lse_fill=float("nan"))
    for b, n in enumerate(lens):
        assert np.isnan(L[b, :, n:]).all(), "padded lse rows must stay untouched"
        L[b, :, n:] = Lref[b, :, n:] = 0.0
    G.say(f"  errors {_compare(w, O, L, Oref, Lref)}")


@pytest.mark.parametrize("name", ["mha_fp16", "gqa_bf16", "gqa_bf16_tp8"])
def test_workload_full(name):
    w = workloads.make_inputs(name)
    G.say(f"workload {name}")
    O, L = G.run_gpu(w, lse_fill=float("nan"))
    q, k, v = G.f64_inputs(w)
    Oref, Lref = oracle.attention(q, k, v, causal=w["causal"], scale=w["scale"],
                                  workers=min(16, oracle.default_workers()))
    G.say(f"  errors {_compare(w, O, L, Oref, Lref)}")


@pytest.mark.parametrize("name", ["long_bf16", "varlen_bf16"])
def test_workload_full_large(name):
    """The two largest workloads at full size, in the bench's launch
    configuration, element by element against the oracle: every row of
    every query head (the oracle runs over 16 processes, 16 query heads and
    their K/V heads at a time).  Every L row must be written (pre-filled
    with NaN) and padded varlen rows left untouched."""
    w = workloads.make_inputs(name)
    G.say(f"workload {name}")
    O, L = G.run_gpu(w, lse_fill=float("nan"))
    assert np.isfinite(O).all()
    q, k, v = G.f64_inputs(w)
    cu = w["cu_seqlens"]
    if cu is not None:
        for b, n in enumerate(np.diff(cu)):
            assert np.isnan(L[b, :, n:]).all(), "padded lse rows must stay untouched"
            L[b, :, n:] = 0.0
    grp = w["Hq"] // w["Hkv"]
    step = 16
    for h0 in range(0, w["Hq"], step):
        hs, ks = slice(h0, h0 + step), slice(h0 // grp, (h0 + step) // grp)
        Oref, Lref = oracle.attention(np.ascontiguousarray(q[:, hs]),
                                      np.ascontiguousarray(k[:, ks]),
                                      np.ascontiguousarray(v[:, ks]), causal=w["causal"],
                                      scale=w["scale"], cu_seqlens=cu,
                                      workers=min(16, oracle.default_workers()))
        if cu is not None:
            for b, n in enumerate(np.diff(cu)):
                Lref[b, :, n:] = 0.0
        G.say(f"  heads {h0}-{h0 + step - 1}: errors "
              f"{_compare(w, O[:, hs], L[:, hs], Oref, Lref)}")


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


def _store(x: np.ndarray, dtype: str) -> np.ndarray:
    """float values (exactly representable) in the workload's storage form."""
    if dtype == "bf16":
        return workloads.round_to_bf16_bits(x.astype(np.float32))
    return x.astype(np.float16)


@pytest.mark.parametrize("dtype,d", [("bf16", 128), ("fp16", 64)])
def test_shift_invariance(dtype, d):
    """softmax is unchanged when every score of a row moves by one constant:
    with K's first component 1 for every key, setting Q's first component of
    row i to t_i adds scale * t_i to all of row i's scores.  O must stay
    within the bar of the unshifted run (and of the oracle), and L must move
    by exactly scale * t_i (up to fp32 rounding of L itself).  The shifts
    reach +-724 at d = 128 and +-1024 at d = 64 in score units."""
    w = _make((dtype, d, 2, 8, 2, 333, True), seed=51)
    q, k, _ = G.f64_inputs(w)
    k = k.copy()
    k[..., 0] = 1.0
    q0 = q.copy()
    q0[..., 0] = 0.0
    shifts = np.array([0.0, 8192.0, -8192.0, 512.0, -512.0, 64.0])
    t = shifts[np.arange(q0[..., 0].size) % shifts.size].reshape(q0.shape[:-1])
    q1 = q0.copy()
    q1[..., 0] = t
    w0, w1 = dict(w), dict(w)
    w0["k"] = w1["k"] = _store(k, dtype)
    w0["q"], w1["q"] = _store(q0, dtype), _store(q1, dtype)
    G.say(f"shift invariance {dtype} d={d}")
    O0, L0 = G.run_gpu(w0, lse_fill=float("nan"))
    O1, L1 = G.run_gpu(w1, lse_fill=float("nan"))
    Oref, Lref = _oracle(w1)
    G.say(f"  errors {_compare(w1, O1, L1, Oref, Lref)}")
    bar = G.O_TOL[dtype]
    assert np.abs(O1 - O0).max() <= bar
    dl = np.abs((L1 - L0) - w["scale"] * t)
    assert dl.max() <= G.L_TOL + 2e-7 * np.abs(L1).max(), dl.max()


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


@pytest.mark.parametrize("case", [
    ("bf16", 128, 2, 8, 2, 333, True), ("bf16", 128, 2, 8, 2, 333, False),
    ("fp16", 64, 2, 6, 6, 300, True), ("fp16", 64, 1, 4, 2, 130, False),
    ("fp16", 64, 3, 4, 2, [200, 7, 128], True), ("bf16", 128, 3, 8, 2, [100, 0, 64], True)])
def test_row_major_and_packed_agree(case):
    """fa_fwd reads V's rows and transposes them on chip; fa_fwd_packed reads
    V packed by fa_pack_v, reused across calls.  Both feed the same operands,
    in the same order, to the same products: bitwise equal O and L."""
    import torch

    import exact_io_aware_amd as fa
    w = _make(case, seed=11)
    dt = w["dtype"]
    q, k, v = (G.to_device(w[x], dt, "cuda:0") for x in "qkv")
    cu = None if w["cu_seqlens"] is None else torch.from_numpy(w["cu_seqlens"]).to("cuda:0")
    ms = w["N"] if cu is not None else None
    G.say(f"row-major V vs packed V {case}")
    # lse pre-filled with NaN: padded varlen rows stay NaN in every call.
    nanl = lambda: torch.full((w["B"], w["Hq"], w["N"]), float("nan"), device="cuda:0")  # noqa
    o1, l1 = fa.fwd(q, k, v, causal=w["causal"], cu_seqlens=cu, max_seqlen=ms, lse=nanl())
    vt = fa.pack_v(v, cu_seqlens=cu, max_seqlen=ms)
    o2, l2 = fa.fwd(q, k, None, causal=w["causal"], vt=vt, cu_seqlens=cu, max_seqlen=ms,
                    lse=nanl())
    o3, l3 = fa.fwd(q, k, None, causal=w["causal"], vt=vt, cu_seqlens=cu, max_seqlen=ms,
                    lse=nanl())
    torch.cuda.synchronize()
    nan7 = lambda t: torch.nan_to_num(t, nan=7.0)  # noqa: E731 (unwritten padded rows)
    for o, l in ((o2, l2), (o3, l3)):
        assert torch.equal(o1, o) and torch.equal(nan7(l1), nan7(l))


def _device_bytes_in_use():
    """Bytes the device has in use (the HIP runtime's own view, so
    allocations made outside torch's allocator count too)."""
    import torch
    free, total = torch.cuda.mem_get_info()
    return total - free


@pytest.mark.parametrize("name", ["gqa_bf16", "varlen_bf16"])
def test_fa_fwd_allocates_nothing(name):
    """The O(N) memory claim (HolySheep, Chinese edition, "IO 感知的算法设计"):
    fa_fwd allocates nothing at all -- no N x N scores (8 GiB for gqa_bf16's
    32 heads of 4096 x 4096 bf16 scores per sequence) and no workspace --
    with o and lse allocated by the caller.  Checked through torch's
    allocator (delta 0) and the device's own free-memory count (no growth by
    more than the runtime's page rounding)."""
    import torch

    import exact_io_aware_amd as fa
    w = workloads.make_inputs(name)
    q, k, v = (G.to_device(w[x], "bf16", "cuda:0") for x in "qkv")
    cu = None if w["cu_seqlens"] is None else torch.from_numpy(w["cu_seqlens"]).to("cuda:0")
    o = torch.empty(q.shape, dtype=torch.float32, device="cuda:0")
    lse = torch.empty((w["B"], w["Hq"], w["N"]), dtype=torch.float32, device="cuda:0")
    G.say(f"device memory during fa_fwd ({name})")
    torch.cuda.synchronize()
    torch.cuda.reset_peak_memory_stats()
    base = torch.cuda.memory_allocated()
    dev0 = _device_bytes_in_use()
    for _ in range(3):
        fa.fwd(q, k, v, causal=True, out=o, lse=lse, cu_seqlens=cu,
               max_seqlen=w["N"] if cu is not None else None, num_splits=1)
    torch.cuda.synchronize()
    assert torch.cuda.max_memory_allocated() - base == 0
    assert _device_bytes_in_use() - dev0 <= (2 << 20)
    assert torch.isfinite(o).all()


# --- any finite scale, streams, debug checks ----------------------------------

@pytest.mark.parametrize("case", [
    ("bf16", 128, 2, 8, 2, 333, True), ("fp16", 64, 2, 4, 4, 200, False),
    ("fp32", 64, 1, 2, 2, 150, True), ("bf16", 64, 3, 4, 2, [200, 7, 128], False)])
@pytest.mark.parametrize("scale", [-0.125, 0.0, -1.0, 0.3])
def test_any_finite_scale(case, scale):
    """Negative and zero scales: the scores are scale * q.k as written, so a
    negative scale ranks keys in reverse and scale 0 averages V over the
    visible keys (L = ln of their count); checked against the oracle, on the
    default path and (16-bit) with packed V."""
    import torch

    import exact_io_aware_amd as fa
    w = _make(case, seed=600 + int(10 * scale))
    w["scale"] = scale
    Oref, Lref = _oracle(w)
    paths = [False] if w["dtype"] == "fp32" else [False, True]
    for packed in paths:
        G.say(f"scale {scale} case {case} packed={packed}")
        q, k, v = (G.to_device(w[x], w["dtype"], "cuda:0") for x in "qkv")
        cu = None if w["cu_seqlens"] is None else torch.from_numpy(w["cu_seqlens"]).to("cuda:0")
        ms = w["N"] if cu is not None else None
        vt = fa.pack_v(v, cu_seqlens=cu, max_seqlen=ms) if packed else None
        lse = torch.full((w["B"], w["Hq"], w["N"]), float("nan"), device="cuda:0")
        o, l = fa.fwd(q, k, None if packed else v, causal=w["causal"], scale=scale,
                      cu_seqlens=cu, max_seqlen=ms, vt=vt, lse=lse)
        torch.cuda.synchronize()
        O, L = o.double().cpu().numpy(), l.double().cpu().numpy()
        Lr = Lref.copy()
        if cu is not None:
            for b, n in enumerate(np.diff(w["cu_seqlens"])):
                assert np.isnan(L[b, :, n:]).all()
                L[b, :, n:] = Lr[b, :, n:] = 0.0
        strict = G.FP32_STRICT if w["dtype"] == "fp32" else None
        bar = None
        if abs(scale) > w["d"] ** -0.5:
            # Scores larger than the workloads' (|scale| above 1/sqrt(d)): the
            # derived bar of the stress inputs (rounding of P for P.V).
            qf, kf, vf = G.f64_inputs(w)
            A, _ = oracle.attention(qf, kf, np.abs(vf), causal=w["causal"], scale=scale,
                                    cu_seqlens=w["cu_seqlens"])
            bar = G.o_bar_derived(w["dtype"], A)
        G.say(f"  errors {_compare(w, O, L, Oref, Lr, strict=strict, bar=bar)}")


def test_side_stream_matches_default_stream():
    """Forward and backward enqueued on a side stream (tensors made by the
    binding belong to that stream) give the default stream's results."""
    import torch

    import exact_io_aware_amd as fa
    w = _make(("bf16", 128, 2, 8, 2, 300, True), seed=21)
    q, k, v = (G.to_device(w[x], "bf16", "cuda:0") for x in "qkv")
    g = workloads.make_custom(2, 8, 8, 128, "bf16", seed=22, N=300)
    do = G.to_device(g["q"], "bf16", "cuda:0")
    G.say("side stream vs default stream")
    o0, l0 = fa.fwd(q, k, v, causal=True)
    dq0, dk0, dv0 = fa.bwd(q, k, v, o0, l0, do, causal=True)
    torch.cuda.synchronize()
    s = torch.cuda.Stream()
    for _ in range(2):
        o1, l1 = fa.fwd(q, k, v, causal=True, stream=s)
        dq1, dk1, dv1 = fa.bwd(q, k, v, o1, l1, do, causal=True, stream=s)
        # Busy work on the default stream meanwhile must not disturb them.
        junk = torch.empty(1 << 24, device="cuda:0").fill_(3.0)
        del junk
        s.synchronize()
        assert torch.equal(o0, o1) and torch.equal(l0, l1)
        assert torch.equal(dq0, dq1) and torch.equal(dk0, dk1) and torch.equal(dv0, dv1)


def test_debug_mode_rejects_corrupt_offsets():
    """FA_DEBUG=1: every entry point that takes packed offsets checks them on
    the device first; corrupt ones (cu[0] != 0, decreasing, a length above N)
    give FA_ERR_SEQLENS and no attention kernel runs (the NaN-filled outputs
    stay untouched).  All offsets stay inside the buffers.  Runs in a child
    process, since the mode is read once per process."""
    import os
    import subprocess
    import sys
    root = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
    env = dict(os.environ, FA_DEBUG="1")
    G.say("FA_DEBUG=1 child process")
    r = subprocess.run([sys.executable, "-u", "-m", "tests.debug_seqlens_check"], cwd=root,
                       env=env, capture_output=True, text=True, timeout=300)
    print(r.stdout[-3000:], r.stderr[-3000:])
    assert r.returncode == 0 and "DEBUG_SEQLENS_OK" in r.stdout
