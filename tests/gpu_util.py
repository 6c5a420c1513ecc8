"""Helpers for the GPU tests: upload seeded inputs, run the HIP path, compare
with the oracle."""
from __future__ import annotations

import sys

import numpy as np

import workloads

# Bars on max |error| (O on the fp32-stored output, L natural log).
O_TOL = {"fp32": 2e-3, "fp16": 2e-3, "bf16": 8e-3}
L_TOL = 1e-3
# fp32 inputs: the computation is fp32 throughout; far below the stated bars.
FP32_STRICT = 1e-5


def say(msg: str) -> None:
    """Name the case before a GPU step, flushed, so a fault is attributable."""
    print(msg, flush=True)
    sys.stdout.flush()


def to_device(arr: np.ndarray, dtype: str, dev):
    import torch
    if dtype == "bf16":
        return torch.from_numpy(np.ascontiguousarray(arr).view(np.int16)).to(dev).view(torch.bfloat16)
    return torch.from_numpy(np.ascontiguousarray(arr)).to(dev)


def torch_dtype(dtype: str):
    import torch
    return {"fp32": torch.float32, "fp16": torch.float16, "bf16": torch.bfloat16}[dtype]


def run_gpu(w: dict, *, out_dtype=None, lse_fill=None, dev="cuda:0"):
    """Run the HIP path on inputs from workloads.make_*; returns (o, lse) as
    float64 numpy arrays (o upcast from out_dtype)."""
    import torch

    import exact_io_aware_amd as fa
    q, k, v = (to_device(w[x], w["dtype"], dev) for x in "qkv")
    cu = None if w["cu_seqlens"] is None else torch.from_numpy(w["cu_seqlens"]).to(dev)
    od = torch.float32 if out_dtype is None else out_dtype
    lse = None
    if lse_fill is not None:
        B = w["B"]
        lse = torch.full((B, w["Hq"], w["N"]), lse_fill, dtype=torch.float32, device=dev)
    o, lse = fa.fwd(q, k, v, causal=w["causal"], scale=w["scale"], cu_seqlens=cu,
                    max_seqlen=w["N"] if cu is not None else None, out_dtype=od, lse=lse)
    torch.cuda.synchronize()
    return o.double().cpu().numpy(), lse.double().cpu().numpy()


def f64_inputs(w: dict):
    return tuple(workloads.to_f64(w[x], w["dtype"]) for x in "qkv")


def o_bar(dtype: str, out_dtype: str, ref: np.ndarray):
    """Elementwise bar on O: the stated bar, plus the rounding of O itself when
    it is stored in 16 bits (half an ulp of the reference value)."""
    bar = O_TOL[dtype]
    if out_dtype == "bf16":
        return bar + np.abs(ref) * 2.0 ** -8
    if out_dtype == "fp16":
        return bar + np.abs(ref) * 2.0 ** -11
    return bar


def o_bar_derived(dtype: str, abs_weighted: np.ndarray):
    """Bar for inputs outside the five workloads (e.g. very peaked softmax).

    The kernel rounds P to the input precision for the P.V contraction, so
    |dO_rj| <= u * sum_c P_rc |V_cj| / l_r, with u the unit roundoff (2^-8
    bf16, 2^-11 fp16, 0 for fp32 where P stays fp32); ``abs_weighted`` is that
    weighted sum, i.e. the oracle's output for values |V|.  1e-3 is added for
    the fp32 score, exp2 and accumulation errors at large score magnitudes.
    The stated bar still applies wherever it is larger.
    """
    u = {"bf16": 2.0 ** -8, "fp16": 2.0 ** -11, "fp32": 0.0}[dtype]
    return np.maximum(O_TOL[dtype], u * abs_weighted + 1e-3)



def grad_bar(dtype: str) -> float:
    """Bar on max |error| of a gradient relative to its largest magnitude.

    The backward rounds P and dS to the input precision for the MFMA
    contractions (unit roundoff u = 2^-8 bf16, 2^-11 fp16) and sums in fp32:
    each gradient element is a sum of terms each carrying a relative error
    <= u, so |error| <= u * sum |terms|.  For N(0,1) inputs the sums of
    absolute terms stay within a few times the largest gradient magnitude;
    4u of it is the bar.
    """
    return 4.0 * {"bf16": 2.0 ** -8, "fp16": 2.0 ** -11}[dtype]


def grad_term_sums(w: dict):
    """Per-element sums of absolute terms of the three gradients, the scale of
    the backward's rounding error element by element (test infrastructure,
    float64 numpy; not the oracle).

    The backward rounds P (for dV = P^T dO) and dS = P (dP - D) (for dK and
    dQ) to the input precision and sums in fp32; D comes from the forward's
    O, which carries that pass's P rounding.  So, with A_r = sum_c |dO_rc|
    (P |V|)_rc (a bound on |D_r| and, times u, on its error):

        |err dV_jc| <~ u * sum_r P_rj |dO_rc|
        |err dK_jc| <~ 3u * |scale| * sum_r P_rj (|dP_rj| + A_r) |Q_rc|
        |err dQ_rc| <~ 3u * |scale| * sum_j P_rj (|dP_rj| + A_r) |K_jc|

    (dS: u from its own rounding and u from P's, each of P |dP - D| <=
    P (|dP| + A_r), plus P |err D_r| <= u P A_r.)

    Returns (T_dQ, T_dK, T_dV) in the layouts of q, k, v (grouped K/V heads
    sum over their query heads)."""
    q, k, v = f64_inputs(w)
    import workloads
    do = workloads.to_f64(w["dout"], w["dtype"])
    scale, causal, cu = w["scale"], w["causal"], w["cu_seqlens"]
    Hq, Hkv = q.shape[-2] if cu is not None else q.shape[1], k.shape[-2] if cu is not None else k.shape[1]
    tq, tk, tv = np.zeros(q.shape), np.zeros(k.shape), np.zeros(v.shape)
    B = len(cu) - 1 if cu is not None else q.shape[0]
    for b in range(B):
        for h in range(Hq):
            g = h // (Hq // Hkv)
            if cu is None:
                qs, ks, vs, ds = q[b, h], k[b, g], v[b, g], do[b, h]
            else:
                a, e = int(cu[b]), int(cu[b + 1])
                qs, ks, vs, ds = q[a:e, h], k[a:e, g], v[a:e, g], do[a:e, h]
            n = qs.shape[0]
            if n == 0:
                continue
            s_ = scale * (qs @ ks.T)
            if causal:
                s_ = np.where(np.tril(np.ones((n, n), dtype=bool)), s_, -np.inf)
            m = s_.max(axis=1, keepdims=True)
            p_ = np.exp(s_ - m)
            p_ /= p_.sum(axis=1, keepdims=True)
            dp = np.abs(ds @ vs.T)
            arow = (np.abs(ds) * (p_ @ np.abs(vs))).sum(axis=1, keepdims=True)
            wgt = p_ * (dp + arow)
            rq = abs(scale) * (wgt @ np.abs(ks))
            rk = abs(scale) * (wgt.T @ np.abs(qs))
            rv = p_.T @ np.abs(ds)
            if cu is None:
                tq[b, h] = rq
                tk[b, g] += rk
                tv[b, g] += rv
            else:
                tq[a:e, h] = rq
                tk[a:e, g] += rk
                tv[a:e, g] += rv
    return tq, tk, tv


def compare_qk(w, O, L, Oref, Lref, out_dtype="fp32", bar=None):
    """Element-wise bars (``bar``, if given, replaces the stated O bar); rows
    that see no key must give O = 0, L = -inf; L rows past a packed
    sequence's query count stay untouched (NaN)."""
    if w["cu_seqlens"] is not None:
        for b, n in enumerate(np.diff(w["cu_seqlens"])):
            assert np.isnan(L[b, :, n:]).all(), "padded lse rows must stay untouched"
            L[b, :, n:] = Lref[b, :, n:] = 0.0
    none = np.isneginf(Lref)
    assert np.array_equal(np.isneginf(L), none), "rows without keys"
    assert np.isfinite(O).all()
    eo = np.abs(O - Oref)
    if bar is None:
        bar = o_bar(w["dtype"], out_dtype, Oref)
    assert (eo <= bar).all(), f"O error {eo.max():.3e}"
    el = np.abs(np.where(none, 0.0, L - Lref))
    assert el.max() <= L_TOL, f"L error {el.max():.3e}"
    if w["dtype"] == "fp32":
        assert eo.max() <= FP32_STRICT and el.max() <= FP32_STRICT
    return float(eo.max()), float(el.max())
