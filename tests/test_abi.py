"""The C ABI without a GPU: the library loads, exports what include/fa.h
declares, and rejects every bad argument before touching the device."""
from __future__ import annotations

import ctypes
import os
import re
import subprocess

import pytest

import exact_io_aware_amd as fa
from exact_io_aware_amd import _lib

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "fa.h")


def declared_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"^\s*(?:const\s+)?\w+\s*\*?\s*(fa_\w+)\s*\(", text, re.M)))


def test_header_declares_the_entry_points():
    names = declared_functions()
    assert {"fa_fwd", "fa_fwd_check", "fa_kernel_name", "fa_supported",
            "fa_status_string", "fa_version", "fa_workspace_bytes", "fa_pack_v",
            "fa_fwd_packed", "fa_fwd_kv", "fa_fwd_kv_split", "fa_fwd_kv_split_packed",
            "fa_fwd_sparse", "fa_bwd", "fa_kernel_name_ex", "fa_check_seqlens"} <= set(names)


def test_library_exports_every_declared_symbol():
    lib = fa.load()
    out = subprocess.run(["nm", "-D", "--defined-only", _lib.LIB_PATH],
                         capture_output=True, text=True, check=True).stdout
    exported = set(re.findall(r"\bT\s+(\w+)$", out, re.M))
    for name in declared_functions():
        assert name in exported, name
        assert isinstance(getattr(lib, name), ctypes._CFuncPtr)


def test_status_codes_match_header():
    text = open(HEADER).read()
    for name, value in _lib.STATUS.items():
        assert re.search(rf"\b{name}\s*=\s*{value}\b", text), name
    strings = {fa.status_string(v) for v in _lib.STATUS.values()}
    assert len(strings) == len(_lib.STATUS)
    assert fa.status_string(12345) == "unknown status"


def test_version_and_support():
    assert fa.version() == 10200
    for dt in (fa.FA_F32, fa.FA_F16, fa.FA_BF16):
        for d in (64, 128):
            for c in (False, True):
                assert fa.supported(dt, d, c)
                for vl in (False, True):
                    assert fa.kernel_name(dt, d, c, vl, fa.FA_F32) is not None
                    if dt != fa.FA_F32:
                        assert fa.kernel_name(dt, d, c, vl, dt) is not None
    assert not fa.supported(fa.FA_BF16, 96, True)
    assert not fa.supported(7, 128, True)
    assert fa.kernel_name(fa.FA_BF16, 96, True, False, fa.FA_F32) is None
    assert fa.kernel_name(fa.FA_F32, 64, False, False, fa.FA_BF16) is None


def test_kernel_name_kv_routing():
    """The decode kernel runs exactly where the G query heads of a K/V head
    times the query rows fit one 32-row block (16-bit inputs); elsewhere the
    prefill kernel of fa_kernel_name."""
    pre = fa.kernel_name(fa.FA_BF16, 128, True, False, fa.FA_F32)
    assert fa.kernel_name_kv(fa.FA_BF16, 128, True, False, fa.FA_F32, 32, 8, 8) == \
        "fa_decode_mfma_bf16_d128_causal_of32"                          # G=4, 4*8 = 32
    assert fa.kernel_name_kv(fa.FA_BF16, 128, True, False, fa.FA_F32, 32, 8, 9) == pre
    assert fa.kernel_name_kv(fa.FA_F16, 64, False, True, fa.FA_F16, 8, 8, 32) == \
        "fa_decode_mfma_f16_d64_varlen"                                  # G=1
    assert fa.kernel_name_kv(fa.FA_F16, 64, False, True, fa.FA_F16, 8, 8, 33) == \
        fa.kernel_name(fa.FA_F16, 64, False, True, fa.FA_F16)
    assert fa.kernel_name_kv(fa.FA_F32, 64, False, False, fa.FA_F32, 8, 8, 1) == \
        fa.kernel_name(fa.FA_F32, 64, False, False, fa.FA_F32)          # fp32: no decode kernel
    assert fa.kernel_name_kv(fa.FA_BF16, 96, True, False, fa.FA_F32, 8, 8, 1) is None
    assert fa.kernel_name_kv(fa.FA_BF16, 128, True, False, fa.FA_F32, 8, 0, 1) is None


def test_kernel_name_ex_paths():
    """fa_kernel_name_ex names the instance each entry point runs: the default
    (row-major V) kernels carry no suffix, the *_packed ones "_vtpacked", the
    block-sparse ones "_sparse" (never the decode kernel)."""
    ex = fa.kernel_name_ex
    assert ex(fa.FA_BF16, 128, True, False, fa.FA_F32, 32, 8, 4096) == \
        fa.kernel_name(fa.FA_BF16, 128, True, False, fa.FA_F32)
    assert ex(fa.FA_BF16, 128, True, False, fa.FA_F32, 32, 8, 4096, vt_packed=True) == \
        "fa_fwd_mfma_bf16_d128_causal_of32_vtpacked"
    assert ex(fa.FA_F16, 64, False, True, fa.FA_F16, 8, 2, 300, sparse=True) == \
        "fa_fwd_mfma_f16_d64_varlen_sparse"
    assert ex(fa.FA_BF16, 128, True, False, fa.FA_F32, 32, 8, 1, sparse=True) == \
        "fa_fwd_mfma_bf16_d128_causal_of32_sparse"
    assert ex(fa.FA_BF16, 128, True, False, fa.FA_F32, 32, 8, 1, vt_packed=True) == \
        "fa_decode_mfma_bf16_d128_causal_of32_vtpacked"
    assert ex(fa.FA_BF16, 128, True, False, fa.FA_F32, 32, 8, 1) == \
        "fa_decode_mfma_bf16_d128_causal_of32"
    assert ex(fa.FA_F32, 64, False, False, fa.FA_F32, 2, 2, 256, vt_packed=True) == \
        "fa_fwd_f32_d64"                       # fp32 has no packed path: the plain kernel
    assert ex(fa.FA_BF16, 96, True, False, fa.FA_F32, 8, 8, 1) is None


@pytest.mark.parametrize("cu,B,n,code", [
    ([0], 0, 1, "FA_OK"),
    ([0, 5, 5, 12], 3, 7, "FA_OK"),
    ([0, 5, 5, 12], 3, 6, "FA_ERR_SEQLENS"),         # a length above the bound
    ([1, 5, 9], 2, 8, "FA_ERR_SEQLENS"),             # cu[0] != 0
    ([0, 5, 4], 2, 8, "FA_ERR_SEQLENS"),             # decreasing
    ([0, 2**31 - 1, -2**31], 2, 2**31 - 1, "FA_ERR_SEQLENS"),   # no overflow in the difference
    (None, 2, 8, "FA_ERR_NULL"),
    ([0], -1, 8, "FA_ERR_SHAPE"),
])
def test_check_seqlens(cu, B, n, code):
    """The predicate FA_DEBUG=1 applies on the device, run on host memory."""
    assert fa.check_seqlens(cu, B, n) == S[code]


# Fake, aligned, non-overlapping addresses: the checks never dereference them.
BASE = dict(q=0x100000, k=0x200000, v=0x300000, o=0x400000, lse=0x500000,
            B=2, Hq=8, Hkv=2, N=64, d=128, causal=1, scale=0.125, cu_seqlens=None,
            in_dtype=fa.FA_BF16, out_dtype=fa.FA_F32)


def check(**kw):
    a = dict(BASE, **kw)
    return _lib.fwd_check(a["q"], a["k"], a["v"], a["o"], a["lse"], a["B"], a["Hq"],
                          a["Hkv"], a["N"], a["d"], a["causal"], a["scale"],
                          a["cu_seqlens"], a["in_dtype"], a["out_dtype"])


S = _lib.STATUS


@pytest.mark.parametrize("kw,code", [
    ({}, "FA_OK"),
    ({"cu_seqlens": 0x600000}, "FA_OK"),
    ({"in_dtype": fa.FA_F32}, "FA_OK"),
    ({"out_dtype": fa.FA_BF16}, "FA_OK"),
    ({"q": None}, "FA_ERR_NULL"), ({"k": None}, "FA_ERR_NULL"),
    ({"v": None}, "FA_ERR_NULL"), ({"o": None}, "FA_ERR_NULL"),
    ({"lse": None}, "FA_ERR_NULL"),
    ({"B": 0}, "FA_ERR_SHAPE"), ({"Hq": 0}, "FA_ERR_SHAPE"), ({"Hkv": -1}, "FA_ERR_SHAPE"),
    ({"N": 0}, "FA_ERR_SHAPE"), ({"causal": 2}, "FA_ERR_SHAPE"),
    ({"B": 1 << 20, "N": 1 << 20, "Hq": 1 << 10, "Hkv": 1 << 10}, "FA_ERR_SHAPE"),
    ({"d": 96}, "FA_ERR_HEADDIM"), ({"d": 0}, "FA_ERR_HEADDIM"), ({"d": 256}, "FA_ERR_HEADDIM"),
    ({"Hq": 6, "Hkv": 4}, "FA_ERR_GQA"),
    ({"in_dtype": 3}, "FA_ERR_DTYPE"), ({"in_dtype": -1}, "FA_ERR_DTYPE"),
    ({"out_dtype": fa.FA_F16}, "FA_ERR_DTYPE"),
    ({"in_dtype": fa.FA_F32, "out_dtype": fa.FA_BF16}, "FA_ERR_DTYPE"),
    ({"scale": float("nan")}, "FA_ERR_SCALE"), ({"scale": float("inf")}, "FA_ERR_SCALE"),
    ({"scale": float("-inf")}, "FA_ERR_SCALE"),
    ({"scale": 0.0}, "FA_OK"), ({"scale": -0.1}, "FA_OK"), ({"scale": -0.0}, "FA_OK"),
    ({"q": 0x100008}, "FA_ERR_ALIGN"), ({"o": 0x400004}, "FA_ERR_ALIGN"),
    ({"lse": 0x500002}, "FA_ERR_ALIGN"), ({"cu_seqlens": 0x600001}, "FA_ERR_ALIGN"),
    ({"o": 0x100000}, "FA_ERR_ALIAS"),
    ({"o": 0x300000 + 4096}, "FA_ERR_ALIAS"),           # inside v
    ({"o": 0x500000 - 16}, "FA_ERR_ALIAS"),             # runs into lse
    ({"o": 0x200000, "cu_seqlens": 0x600000}, "FA_ERR_ALIAS"),
])
def test_argument_checks(kw, code):
    assert check(**kw) == S[code]


def test_fwd_rejects_before_any_device_call():
    # fa_fwd runs the same checks first: bad arguments never reach HIP.
    for kw, code in [({"q": None}, "FA_ERR_NULL"), ({"d": 96}, "FA_ERR_HEADDIM"),
                     ({"scale": float("nan")}, "FA_ERR_SCALE"),
                     ({"o": 0x100000}, "FA_ERR_ALIAS")]:
        a = dict(BASE, **kw)
        st = _lib.fwd_raw(a["q"], a["k"], a["v"], a["o"], a["lse"], a["B"], a["Hq"],
                          a["Hkv"], a["N"], a["d"], a["causal"], a["scale"], None, None,
                          a["in_dtype"], a["out_dtype"])
        assert st == S[code]


def test_python_front_end_validates():
    import torch
    q = torch.zeros(1, 2, 8, 64)
    with pytest.raises(ValueError):
        fa.fwd(q, q, q)            # host tensors are refused, nothing falls back
    with pytest.raises(ValueError):
        fa.fwd(q, q.half(), q)


def test_flops_convention():
    assert fa.flops(1, 2, [3], causal=False) == 4 * 2 * 9
    assert fa.flops(2, 4, [3, 1], causal=True) == 4 * 4 * 2 * (6 + 1)
    from workloads import WORKLOADS
    w = WORKLOADS["gqa_bf16"]
    assert abs(fa.flops(w.Hq, w.d, [w.N] * w.B, True) - 5.50e11) / 5.50e11 < 0.01


def test_workspace_bytes():
    # B * Hkv * ceil(N/64) tiles of d rows x 64 keys x 2 bytes; none for fp32.
    assert fa.workspace_bytes(4, 8, 4096, 128, fa.FA_BF16) == 4 * 8 * 64 * 128 * 128
    assert fa.workspace_bytes(2, 3, 65, 64, fa.FA_F16) == 2 * 3 * 2 * 64 * 128
    assert fa.workspace_bytes(1, 1, 1, 128, fa.FA_BF16) == 128 * 128
    assert fa.workspace_bytes(4, 8, 4096, 128, fa.FA_F32) == 0
    assert fa.workspace_bytes(4, 8, 4096, 96, fa.FA_BF16) == 0
    assert fa.workspace_bytes(0, 8, 4096, 128, fa.FA_BF16) == 0


VT = 0x700000
WS = 2 * 2 * 1 * 128 * 128       # workspace of BASE: B=2, Hkv=2, one 64-key tile, d=128


def packed(**kw):
    a = dict(BASE, vt=VT, vt_bytes=WS)
    a.update(kw)
    return _lib.fwd_packed_raw(a["q"], a["k"], a["vt"], a["vt_bytes"], a["o"], a["lse"],
                               a["B"], a["Hq"], a["Hkv"], a["N"], a["d"], a["causal"],
                               a["scale"], a["cu_seqlens"], None, a["in_dtype"],
                               a["out_dtype"])


def pack(**kw):
    a = dict(BASE, vt=VT, vt_bytes=WS)
    a.update(kw)
    return _lib.pack_v_raw(a["v"], a["vt"], a["vt_bytes"], a["B"], a["Hkv"], a["N"], a["d"],
                           a["cu_seqlens"], None, a["in_dtype"])


@pytest.mark.parametrize("kw,code", [
    ({"vt": None}, "FA_ERR_NULL"), ({"q": None}, "FA_ERR_NULL"),
    ({"vt_bytes": WS - 1}, "FA_ERR_WORKSPACE"), ({"vt_bytes": 0}, "FA_ERR_WORKSPACE"),
    ({"vt": VT + 8}, "FA_ERR_ALIGN"),
    ({"in_dtype": fa.FA_F32}, "FA_ERR_DTYPE"),
    ({"d": 96}, "FA_ERR_HEADDIM"), ({"Hq": 6, "Hkv": 4}, "FA_ERR_GQA"),
    ({"scale": float("inf")}, "FA_ERR_SCALE"),
    ({"o": VT}, "FA_ERR_ALIAS"), ({"o": VT + WS - 16}, "FA_ERR_ALIAS"),
])
def test_fwd_packed_rejects_before_any_device_call(kw, code):
    assert packed(**kw) == S[code]


@pytest.mark.parametrize("kw,code", [
    ({"v": None}, "FA_ERR_NULL"), ({"vt": None}, "FA_ERR_NULL"),
    ({"B": 0}, "FA_ERR_SHAPE"), ({"N": 0}, "FA_ERR_SHAPE"), ({"Hkv": 0}, "FA_ERR_SHAPE"),
    ({"B": 1 << 20, "N": 1 << 30, "Hkv": 1 << 10}, "FA_ERR_SHAPE"),
    ({"d": 32}, "FA_ERR_HEADDIM"),
    ({"in_dtype": fa.FA_F32}, "FA_ERR_DTYPE"), ({"in_dtype": 5}, "FA_ERR_DTYPE"),
    ({"v": 0x300004}, "FA_ERR_ALIGN"), ({"vt": VT + 4}, "FA_ERR_ALIGN"),
    ({"cu_seqlens": 0x600002}, "FA_ERR_ALIGN"),
    ({"vt_bytes": WS - 16}, "FA_ERR_WORKSPACE"),
    ({"vt": 0x300000}, "FA_ERR_ALIAS"), ({"vt": 0x300000 + 4096}, "FA_ERR_ALIAS"),
])
def test_pack_v_rejects_before_any_device_call(kw, code):
    assert pack(**kw) == S[code]


def kv(**kw):
    a = dict(BASE, Nk=96, cu_k=None)
    a.update(kw)
    return _lib.fwd_kv_raw(a["q"], a["k"], a["v"], a["o"], a["lse"], a["B"], a["Hq"],
                           a["Hkv"], a["N"], a["Nk"], a["d"], a["causal"], a["scale"],
                           a["cu_seqlens"], a["cu_k"], None, a["in_dtype"], a["out_dtype"])


@pytest.mark.parametrize("kw,code", [
    ({"cu_seqlens": 0x600000}, "FA_ERR_NULL"),            # query offsets without key offsets
    ({"cu_k": 0x600100}, "FA_ERR_NULL"),
    ({"Nk": 0}, "FA_ERR_SHAPE"), ({"N": 0}, "FA_ERR_SHAPE"),
    ({"cu_seqlens": 0x600000, "cu_k": 0x600102}, "FA_ERR_ALIGN"),
    ({"d": 96}, "FA_ERR_HEADDIM"),
    ({"o": 0x200000 + 2 * 96 * 2 * 128 * 2 - 16}, "FA_ERR_ALIAS"),   # runs into k (Nk rows)
])
def test_fwd_kv_rejects_before_any_device_call(kw, code):
    assert kv(**kw) == S[code]


def split(**kw):
    a = dict(BASE, Nk=64, vt=VT, vt_bytes=WS, n=4, part=0x800000, part_bytes=1 << 24)
    a.update(kw)
    return _lib.fwd_kv_split_packed_raw(a["q"], a["k"], a["vt"], a["vt_bytes"], a["o"],
                                        a["lse"], a["B"], a["Hq"], a["Hkv"], a["N"], a["Nk"],
                                        a["d"], a["causal"], a["scale"], a["cu_seqlens"],
                                        a.get("cu_k", a["cu_seqlens"]), a["n"], a["part"],
                                        a["part_bytes"], None, a["in_dtype"], a["out_dtype"])


def split_rm(**kw):
    a = dict(BASE, Nk=64, n=4, part=0x800000, part_bytes=1 << 24)
    a.update(kw)
    return _lib.fwd_kv_split_raw(a["q"], a["k"], a["v"], a["o"], a["lse"], a["B"], a["Hq"],
                                 a["Hkv"], a["N"], a["Nk"], a["d"], a["causal"], a["scale"],
                                 a["cu_seqlens"], a.get("cu_k", a["cu_seqlens"]), a["n"],
                                 a["part"], a["part_bytes"], None, a["in_dtype"],
                                 a["out_dtype"])


def test_split_workspace_bytes():
    assert fa.split_workspace_bytes(2, 8, 64, 128, 4) == 4 * 2 * 8 * 64 * 129 * 4
    assert fa.split_workspace_bytes(2, 8, 64, 128, 1) == 0


@pytest.mark.parametrize("kw,code", [
    ({"n": 0}, "FA_ERR_SHAPE"), ({"n": 257}, "FA_ERR_SHAPE"),
    ({"part": None}, "FA_ERR_NULL"), ({"part": 0x800008}, "FA_ERR_ALIGN"),
    ({"part_bytes": 4 * 2 * 8 * 64 * 129 * 4 - 1}, "FA_ERR_WORKSPACE"),
    ({"part": 0x400000 + 4096}, "FA_ERR_ALIAS"),                 # inside o
    ({"in_dtype": fa.FA_F32}, "FA_ERR_DTYPE"),
])
def test_split_rejects_before_any_device_call(kw, code):
    assert split(**kw) == S[code]
    assert split_rm(**kw) == S[code]        # the row-major-V form checks the same


BWD = dict(q=0x100000, k=0x200000, v=0x300000, o=0x400000, do=0x600000, lse=0x500000,
           dq=0x1000000, dk=0x2000000, dv=0x3000000, ws=0x4000000, ws_bytes=1 << 24,
           B=2, Hq=8, Hkv=2, N=64, d=128, causal=1, scale=0.125, cu=None,
           in_dtype=fa.FA_BF16, o_dtype=fa.FA_F32, g_dtype=fa.FA_F32)


def bwd(**kw):
    a = dict(BWD)
    a.update(kw)
    return _lib.bwd_raw(a["q"], a["k"], a["v"], a["o"], a["do"], a["lse"], a["dq"], a["dk"],
                        a["dv"], a["B"], a["Hq"], a["Hkv"], a["N"], a["d"], a["causal"],
                        a["scale"], a["cu"], a["ws"], a["ws_bytes"], None, a["in_dtype"],
                        a["o_dtype"], a["g_dtype"])


def test_bwd_workspace_bytes():
    rows = 2 * 8 * 64 * 4
    pad = (rows + 255) // 256 * 256
    assert fa.bwd_workspace_bytes(2, 8, 2, 64, 128, fa.FA_BF16) == 2 * pad
    assert fa.bwd_workspace_bytes(2, 8, 2, 64, 128, fa.FA_F32) == 0


@pytest.mark.parametrize("kw,code", [
    ({"do": None}, "FA_ERR_NULL"), ({"dk": None}, "FA_ERR_NULL"), ({"ws": None}, "FA_ERR_NULL"),
    ({"in_dtype": fa.FA_F32, "o_dtype": fa.FA_F32}, "FA_ERR_DTYPE"),
    ({"g_dtype": fa.FA_F16}, "FA_ERR_DTYPE"),
    ({"ws_bytes": 1000}, "FA_ERR_WORKSPACE"),
    ({"dq": 0x1000008}, "FA_ERR_ALIGN"), ({"do": 0x600004}, "FA_ERR_ALIGN"),
    ({"dq": 0x100000}, "FA_ERR_ALIAS"), ({"dk": 0x1000000 + 4096}, "FA_ERR_ALIAS"),
    ({"dv": 0x4000000 + 64}, "FA_ERR_ALIAS"),
    ({"d": 96}, "FA_ERR_HEADDIM"), ({"Hq": 6, "Hkv": 4}, "FA_ERR_GQA"),
    ({"scale": 0.0}, "FA_ERR_SCALE"), ({"scale": -0.5}, "FA_ERR_SCALE"),   # backward: > 0
    ({"scale": float("nan")}, "FA_ERR_SCALE"),
])
def test_bwd_rejects_before_any_device_call(kw, code):
    assert bwd(**kw) == S[code]


def sparse(packed_vt=True, **kw):
    a = dict(BASE, Nk=64, vt=VT, vt_bytes=WS, mask=0x900000, mb=1, mh=1)
    a.update(kw)
    if packed_vt:
        return _lib.fwd_sparse_packed_raw(a["q"], a["k"], a["vt"], a["vt_bytes"], a["o"],
                                          a["lse"], a["B"], a["Hq"], a["Hkv"], a["N"], a["Nk"],
                                          a["d"], a["causal"], a["scale"], a["cu_seqlens"],
                                          a.get("cu_k", a["cu_seqlens"]), a["mask"], a["mb"],
                                          a["mh"], None, a["in_dtype"], a["out_dtype"])
    return _lib.fwd_sparse_raw(a["q"], a["k"], a["v"], a["o"], a["lse"], a["B"], a["Hq"],
                               a["Hkv"], a["N"], a["Nk"], a["d"], a["causal"], a["scale"],
                               a["cu_seqlens"], a.get("cu_k", a["cu_seqlens"]), a["mask"],
                               a["mb"], a["mh"], None, a["in_dtype"], a["out_dtype"])


@pytest.mark.parametrize("packed_vt", [True, False])
@pytest.mark.parametrize("kw,code", [
    ({"mask": None}, "FA_ERR_NULL"),
    ({"in_dtype": fa.FA_F32}, "FA_ERR_DTYPE"),
    ({"mb": 3}, "FA_ERR_SHAPE"), ({"mh": 2}, "FA_ERR_SHAPE"), ({"mh": 0}, "FA_ERR_SHAPE"),
    ({"Nk": 64 * 4096 + 1, "vt_bytes": 1 << 40, "k": 1 << 40, "v": 2 << 40, "vt": 3 << 40},
     "FA_ERR_SHAPE"),                                                 # more than 4096 key tiles
    ({"mask": 0x400000}, "FA_ERR_ALIAS"),                             # the mask is o
    ({"mask": 0x500000 + 64}, "FA_ERR_ALIAS"),                        # inside lse
    ({"d": 96}, "FA_ERR_HEADDIM"),
])
def test_sparse_rejects_before_any_device_call(packed_vt, kw, code):
    if kw.get("in_dtype") == fa.FA_F32 and packed_vt:
        code = "FA_ERR_DTYPE"            # the packed path rejects fp32 first
    assert sparse(packed_vt, **kw) == S[code]


def test_sparse_valid_arguments_reach_the_device_check():
    # Valid arguments pass every check; without a gfx950 device the entry
    # point stops at the device query.
    for packed_vt in (True, False):
        for mb, mh in ((1, 1), (2, 8), (1, 8), (2, 1)):
            st = sparse(packed_vt, mb=mb, mh=mh)
            assert st in (S["FA_ERR_DEVICE"], S["FA_OK"]), st


def test_sparse_flops_count_admitted_pairs():
    """The bench's FLOP count under a block mask equals the oracle's pair
    count (brute force over the admitted blocks)."""
    import numpy as np

    import oracle
    r = np.random.default_rng(5)
    for nq, nk in ((300, 300), (100, 333), (130, 64)):
        for causal in (False, True):
            bm = (r.random((2, 3, -(-nq // 64), -(-nk // 64))) < 0.5).astype(np.uint8)
            want = sum(oracle.sparse_pair_count(bm[b, h], nq, nk, causal)
                       for b in range(2) for h in range(3))
            assert fa.flops(3, 16, [nq, nq], causal, [nk, nk], block_mask=bm) == 4.0 * 16 * want
            one = bm[:1, :1]
            want1 = 6 * oracle.sparse_pair_count(one[0, 0], nq, nk, causal)
            assert fa.flops(3, 16, [nq, nq], causal, [nk, nk], block_mask=one) == 4.0 * 16 * want1


def test_force_order_setting():
    """fa_debug_force_order takes -1 .. 3 and nothing else; no device call."""
    before = fa.debug_forced_order()
    try:
        for order in (-1, 0, 1, 2, 3):
            fa.debug_force_order(order)
            assert fa.debug_forced_order() == order
        for bad in (-2, 4, 1000):
            assert fa.load().fa_debug_force_order(bad) == _lib.STATUS["FA_ERR_SHAPE"]
            assert fa.debug_forced_order() == 3, "a rejected order leaves the setting alone"
    finally:
        fa.debug_force_order(before)


@pytest.mark.parametrize("env,expected", [("2", 2), ("0", 0), ("-1", -1), ("7", -1),
                                          ("rb", -1), ("", -1), (None, -1)])
def test_force_order_from_environment(env, expected):
    """FA_FORCE_ORDER gives the initial setting; anything outside -1 .. 3 is
    ignored.  A fresh process reads it at first use."""
    import sys
    envs = dict(os.environ)
    envs.pop("FA_FORCE_ORDER", None)
    if env is not None:
        envs["FA_FORCE_ORDER"] = env
    code = "import exact_io_aware_amd as fa; print(fa.debug_forced_order())"
    out = subprocess.run([sys.executable, "-c", code], capture_output=True, text=True,
                         check=True, env=envs, cwd=ROOT)
    assert int(out.stdout.strip().splitlines()[-1]) == expected


def test_poisoning_build_is_the_same_interface():
    """libfa_poison.so (the LDS-poisoning test build) exports every declared
    symbol and reports its flag; libfa.so does not."""
    assert fa.load().fa_build_flags() == 0
    out = subprocess.run(["nm", "-D", "--defined-only", _lib.POISON_LIB_PATH],
                         capture_output=True, text=True, check=True).stdout
    exported = set(re.findall(r"\bT\s+(\w+)$", out, re.M))
    assert set(declared_functions()) <= exported
    with _lib.poisoned_lds() as lib:
        assert lib.fa_build_flags() == 1
        assert fa.load() is lib
    assert fa.load().fa_build_flags() == 0
