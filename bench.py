"""Benchmark of the exact attention forward on one MI355X.

One step = one forward pass: one launch of the attention kernel (fa_fwd:
grid map, Q load, K/V streaming, QK^T, masking, online softmax, P.V with V
transposed on chip, epilogue) over the headline workload: B=4, Hq=32, Hkv=8,
N=4096, d=128, bf16, causal, fp32 O.  Inputs are resident in HBM before
timing starts.

Prints one JSON line: throughput of the whole step (algorithmic TFLOP/s:
4*d*Hq per visible (query, key) pair), the roofline of the attention kernel
(its average launch time, measured with HIP events recorded on the launch
stream right before and after it), and the CPU oracle timed on a bounded
sample of the same workload on the host cores.
"""
from __future__ import annotations

import argparse
import hashlib
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

METRIC = "attention fwd TFLOP/s at 1 MI355X (% of MFMA peak), bf16 causal d=128 N=4096"
# MI355X dense MFMA peaks by input type (the fp32 path's products run on the
# fp32 MFMA), at the 2.4 GHz peak engine clock, and HBM3E bandwidth.
PEAK_TFLOPS = {"bf16": 2500.0, "fp16": 2500.0, "fp32": 157.3}
PEAK_CLOCK_GHZ = 2.4
PEAK_HBM_GBS = 8000.0
XCDS = 8
# Sources of each kernel family (a counter summary is used only while they
# are unchanged).
_CSRC = os.path.join(ROOT, "exact_io_aware_amd", "csrc")
KERNEL_SRCS = {
    "fa_fwd_mfma": ("fa_fwd_mfma.h", "fa_device.h"),
    "fa_decode_mfma": ("fa_fwd_kernels.hip", "fa_device.h"),
    "fa_fwd_f32": ("fa_fwd_kernels.hip", "fa_device.h"),
    "fa_bwd": ("fa_bwd_kernels.hip", "fa_device.h"),
}


def parse():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=100)
    ap.add_argument("--warmup", type=int, default=30)
    ap.add_argument("--workload", default="gqa_bf16")
    ap.add_argument("--out-dtype", choices=["fp32", "in"], default="fp32")
    ap.add_argument("--pass", dest="which", choices=["fwd", "bwd"], default="fwd",
                    help="bwd: time the backward pass (gradients of sum(O * dO)) instead")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--cpu-sample-heads", type=int, default=0,
                    help="query heads (from the first sequences) the oracle is timed on; "
                         "0 = the whole workload")
    ap.add_argument("--cold", action="store_true",
                    help="overwrite a 512 MiB buffer before every step, so the inputs come "
                         "from HBM and not from the 256 MB last-level cache; the fill is "
                         "outside the attention launch's events but inside ms_per_step")
    ap.add_argument("--calibrate-copy-mib", type=int, default=0,
                    help="after timing, run one plain device copy of this many MiB "
                         "(reads and writes that many bytes once), to scale memory "
                         "counters such as FETCH_SIZE / WRITE_SIZE")
    return ap.parse_args()


def source_digest(kernel: str) -> str:
    """sha256 (first 16 hex digits) of the sources of the kernel's family."""
    fam = next(k for k in KERNEL_SRCS if kernel.startswith(k))
    h = hashlib.sha256()
    for name in KERNEL_SRCS[fam]:
        with open(os.path.join(_CSRC, name), "rb") as f:
            h.update(f.read())
    return h.hexdigest()[:16]


def counters_for(kernel: str, workload: str):
    """The committed counter summary of this kernel on this workload
    (profiles/counters_<workload>.json), if it was taken on the current
    kernel source; else None."""
    path = os.path.join(ROOT, "profiles", f"counters_{workload}.json")
    if not os.path.exists(path):
        return None
    with open(path) as f:
        t = json.load(f)
    if t.get("kernel") != kernel or t.get("kernel_source_sha") != source_digest(kernel):
        return None
    return t


def clock_of(counters, launch_ms: float):
    """Shader clock of the timed launches: the kernel's GPU-active cycles
    per XCD (GRBM_GUI_ACTIVE of the counter run, summed over the XCDs) over
    the live average launch time; None for launches under 50 us."""
    if counters is None or not counters.get("grbm_gui_active_per_dispatch"):
        return None
    if counters.get("dispatch_ns", 0) < 50000:   # a launch's fixed cost dominates
        return None
    return counters["grbm_gui_active_per_dispatch"] / XCDS / (launch_ms * 1e6)


def cpu_baseline(w, heads: int, o_gpu=None, lse_gpu=None):
    """The oracle, as it stands, on the first `heads` query heads (whole
    sequences) of the workload, over a process pool of the host's cores.
    With the timed run's outputs (o_gpu, lse_gpu: host float64 arrays in the
    workload's layout) it also reports their largest differences from the
    oracle on that sample."""
    import numpy as np

    import oracle
    import workloads
    G = w["Hq"] // w["Hkv"]
    if heads <= 0:
        heads = w["B"] * w["Hq"]
    heads = max(G, (heads // G) * G)
    q, k, v = (workloads.to_f64(w[x], w["dtype"]) for x in "qkv")
    nb = min(w["B"], max(1, heads // w["Hq"]))
    hq = min(heads, w["Hq"])
    workers = oracle.default_workers()
    if w["cu_seqlens"] is not None and w.get("cu_seqlens_k") is not None:
        # Packed sequences with their own key counts (the queries are the
        # last tokens of each sequence).
        cu, cuk = w["cu_seqlens"][:nb + 1], w["cu_seqlens_k"][:nb + 1]
        T, Tk = int(cu[-1]), int(cuk[-1])
        qs = np.ascontiguousarray(q[:T, :hq])
        ks = np.ascontiguousarray(k[:Tk, :hq // G])
        vs = np.ascontiguousarray(v[:Tk, :hq // G])
        t0 = time.perf_counter()
        ref = oracle.attention_qk(qs, ks, vs, causal=w["causal"], scale=w["scale"],
                                  cu_seqlens_q=cu, cu_seqlens_k=cuk, workers=workers)
        dt = time.perf_counter() - t0
        fl = hq * 4.0 * w["d"] * sum(oracle.pair_count(int(a), int(c), w["causal"])
                                     for a, c in zip(np.diff(cu), np.diff(cuk)))
        got = None if o_gpu is None else (o_gpu[:T, :hq], lse_gpu[:nb, :hq])
        if got is not None:     # the oracle's L spans the sample's most queries
            got = (got[0], got[1][..., :int(np.diff(cu).max()) if nb else 0])
    elif w["cu_seqlens"] is not None:
        cu = w["cu_seqlens"][:nb + 1]
        T = int(cu[-1])
        qs = np.ascontiguousarray(q[:T, :hq])
        ks = np.ascontiguousarray(k[:T, :hq // G])
        vs = np.ascontiguousarray(v[:T, :hq // G])
        t0 = time.perf_counter()
        ref = oracle.attention(qs, ks, vs, causal=w["causal"], scale=w["scale"], cu_seqlens=cu,
                               workers=workers)
        dt = time.perf_counter() - t0
        fl = hq * sum(oracle.unit_flops(int(n), w["d"], w["causal"]) for n in np.diff(cu))
        got = None if o_gpu is None else (o_gpu[:T, :hq], lse_gpu[:nb, :hq])
        if got is not None:     # the oracle's L spans the sample's longest sequence
            got = (got[0], got[1][..., :int(np.diff(cu).max()) if nb else 0])
    else:
        qs = np.ascontiguousarray(q[:nb, :hq])
        ks = np.ascontiguousarray(k[:nb, :hq // G])
        vs = np.ascontiguousarray(v[:nb, :hq // G])
        t0 = time.perf_counter()
        if w.get("block_mask") is not None:
            ref = oracle.attention_block_sparse(qs, ks, vs, w["block_mask"], causal=w["causal"],
                                                scale=w["scale"], workers=workers)
            fl = nb * hq * 4.0 * w["d"] * oracle.sparse_pair_count(
                w["block_mask"][0, 0], w["N"], w["Nk"], w["causal"])
        elif w["Nk"] != w["N"]:
            ref = oracle.attention_qk(qs, ks, vs, causal=w["causal"], scale=w["scale"],
                                      workers=workers)
            fl = nb * hq * 4.0 * w["d"] * oracle.pair_count(w["N"], w["Nk"], w["causal"])
        else:
            ref = oracle.attention(qs, ks, vs, causal=w["causal"], scale=w["scale"],
                                   workers=workers)
            fl = nb * hq * oracle.unit_flops(w["N"], w["d"], w["causal"])
        dt = time.perf_counter() - t0
        got = None if o_gpu is None else (o_gpu[:nb, :hq], lse_gpu[:nb, :hq])
    rec = {"value": fl / dt / 1e12, "unit": "TFLOP/s", "cores": workers, "kind": "oracle",
           "sample": f"{nb} sequence(s) x {hq} query heads of {w['name']} "
                     f"({nb * hq} of {w['B'] * w['Hq']} head-sequences), float64 numpy, "
                     f"{dt:.2f} s wall"}
    if got is not None:
        # The oracle's L is NaN past a packed sequence's end (no such row)
        # and -inf for a row with no visible key; the kernel's must be -inf
        # exactly there too.
        o_ref, l_ref = ref
        row = ~np.isnan(l_ref)
        fin = np.isfinite(l_ref)
        rec["errors"] = {
            "o_max_abs": float(np.max(np.abs(got[0] - o_ref))) if got[0].size else 0.0,
            "l_max_abs": float(np.max(np.abs(got[1][fin] - l_ref[fin]))) if fin.any() else 0.0,
            "l_neginf_match": bool(np.array_equal(np.isneginf(got[1][row]),
                                                  np.isneginf(l_ref[row]))),
            "of": "the timed run's O and L on the sample above, against the oracle"}
    return rec


def cpu_baseline_bwd(w, heads: int):
    """The oracle's backward (float64 numpy), as it stands, on the first
    query heads of the first sequence (one K/V group at a time), over a
    process pool; rate under the backward's FLOP convention (2.5 x the
    forward's)."""
    import numpy as np

    import oracle
    import workloads
    G = w["Hq"] // w["Hkv"]
    if heads <= 0:
        heads = 2 * G
    heads = max(G, min(w["Hq"], (heads // G) * G))
    q, k, v = (workloads.to_f64(w[x], w["dtype"]) for x in "qkv")
    if w["cu_seqlens"] is not None:
        n0 = int(w["cu_seqlens"][1])
        qs = np.ascontiguousarray(q[:n0, :heads].transpose(1, 0, 2)[None])
        ks = np.ascontiguousarray(k[:n0, :heads // G].transpose(1, 0, 2)[None])
        vs = np.ascontiguousarray(v[:n0, :heads // G].transpose(1, 0, 2)[None])
    else:
        n0 = w["N"]
        qs = np.ascontiguousarray(q[:1, :heads])
        ks = np.ascontiguousarray(k[:1, :heads // G])
        vs = np.ascontiguousarray(v[:1, :heads // G])
    do = np.random.default_rng(w["seed"] + 100).standard_normal(qs.shape)
    workers = oracle.default_workers()
    t0 = time.perf_counter()
    oracle.attention_backward(qs, ks, vs, do, causal=w["causal"], scale=w["scale"],
                              workers=workers)
    dt = time.perf_counter() - t0
    fl = 2.5 * heads * oracle.unit_flops(n0, w["d"], w["causal"])
    return {"value": fl / dt / 1e12, "unit": "TFLOP/s", "cores": workers, "kind": "oracle",
            "sample": f"backward of 1 sequence ({n0} tokens) x {heads} query heads of "
                      f"{w['name']}, float64 numpy, {dt:.2f} s wall"}


def main():
    args = parse()
    if args.gpus != 1:
        print(f"bench.py runs on one GPU only (asked for --gpus {args.gpus}); "
              "multi-GPU runs are not part of this path", file=sys.stderr)
        sys.exit(2)
    import numpy as np
    import torch

    import exact_io_aware_amd as fa
    import workloads

    w = workloads.make_inputs(args.workload)
    dev = torch.device("cuda:0")

    def up(a):
        if w["dtype"] == "bf16":
            return torch.from_numpy(np.ascontiguousarray(a).view(np.int16)).to(dev).view(torch.bfloat16)
        return torch.from_numpy(np.ascontiguousarray(a)).to(dev)

    q, k, v = (up(w[x]) for x in "qkv")
    cu = None if w["cu_seqlens"] is None else torch.from_numpy(w["cu_seqlens"]).to(dev)
    cuk = None if w["cu_seqlens_k"] is None else torch.from_numpy(w["cu_seqlens_k"]).to(dev)
    Nk = w["Nk"]
    out_dtype = torch.float32 if args.out_dtype == "fp32" else q.dtype
    o = torch.empty(q.shape, dtype=out_dtype, device=dev)
    lse = torch.empty((w["B"], w["Hq"], w["N"]), dtype=torch.float32, device=dev)
    lengths = [w["N"]] * w["B"] if cu is None else list(np.diff(w["cu_seqlens"]))
    lengths_k = None
    if Nk != w["N"] or cuk is not None:
        lengths_k = [Nk] * w["B"] if cuk is None else list(np.diff(w["cu_seqlens_k"]))
    bm_np = w.get("block_mask")
    flop = fa.flops(w["Hq"], w["d"], lengths, w["causal"], lengths_k, block_mask=bm_np)
    dt_code = {"fp32": fa.FA_F32, "fp16": fa.FA_F16, "bf16": fa.FA_BF16}[w["dtype"]]
    stream = torch.cuda.current_stream(dev)
    # Decode: the packed V^T is the KV cache's layout, filled once when the
    # cache is built (a decode loop re-packs only the tile holding the new
    # token), so it is packed before timing; a step is the attention alone.
    # Every other workload reads V itself (fa_fwd: one launch per step).
    decode = w["name"].startswith("decode")
    packed = decode and w["dtype"] != "fp32"
    max_seqlen = w["N"] if cu is not None else None
    vt = None
    if packed:
        vt = torch.empty(fa.workspace_bytes(w["B"], w["Hkv"], Nk, w["d"], dt_code),
                         dtype=torch.uint8, device=dev)
    n_splits = fa.num_splits(w["B"], w["Hq"], w["Hkv"], w["N"], Nk, w["d"], dt_code) \
        if w["dtype"] != "fp32" else 1
    bm = None
    if bm_np is not None:          # block-sparse: never split over keys
        bm = torch.from_numpy(np.ascontiguousarray(bm_np)).to(dev)
        n_splits = 1
    kname = fa.kernel_name_ex(dt_code, w["d"], w["causal"], cu is not None,
                              fa.FA_F32 if args.out_dtype == "fp32" else dt_code,
                              w["Hq"], w["Hkv"], w["N"], sparse=bm is not None, vt_packed=packed)
    split_ws = None
    if n_splits > 1:
        split_ws = torch.empty(fa.split_workspace_bytes(w["B"], w["Hq"], w["N"], w["d"],
                                                        n_splits), dtype=torch.uint8, device=dev)

    def pack():
        fa.pack_v(v, cu_seqlens=cuk if cuk is not None else cu,
                  max_seqlen=Nk if cu is not None else None, out=vt, stream=stream)

    if packed and decode:
        pack()

    bwd_state = None
    if args.which == "bwd":
        if w["dtype"] == "fp32" or Nk != w["N"] or cuk is not None:
            raise SystemExit("--pass bwd needs 16-bit inputs with equal query and key counts")
        # dO: seeded N(0,1) like the inputs, query-shaped
        g = workloads.make_custom(w["B"], w["Hq"], w["Hq"], w["d"], w["dtype"], seed=w["seed"] + 100,
                                  **({"N": w["N"]} if cu is None else {"lengths": w["lengths"]}))
        dout = up(g["q"])
        o_f, lse_f = fa.fwd(q, k, v, causal=w["causal"], scale=w["scale"], cu_seqlens=cu,
                            max_seqlen=max_seqlen)
        ws = torch.empty(fa.bwd_workspace_bytes(w["B"], w["Hq"], w["Hkv"], w["N"], w["d"], dt_code),
                         dtype=torch.uint8, device=dev)
        bwd_state = (dout, o_f, lse_f, ws)

    scrub = torch.empty(512 << 20, dtype=torch.uint8, device=dev) if args.cold else None

    def step(mark=None):
        if scrub is not None:
            scrub.fill_(1)     # evicts the inputs from the caches
        if bwd_state is not None:
            dout, o_f, lse_f, ws = bwd_state
            if mark is not None:
                mark[0].record(stream)
            fa.bwd(q, k, v, o_f, lse_f, dout, causal=w["causal"], scale=w["scale"],
                   cu_seqlens=cu, max_seqlen=max_seqlen, workspace=ws, stream=stream)
            if mark is not None:
                mark[1].record(stream)
            return
        if mark is not None:
            mark[0].record(stream)
        fa.fwd(q, k, None if packed else v, causal=w["causal"], scale=w["scale"],
               cu_seqlens=cu, max_seqlen=max_seqlen, out_dtype=out_dtype, out=o, lse=lse,
               stream=stream, vt=vt, cu_seqlens_k=cuk,
               max_seqlen_k=Nk if cu is not None else None,
               num_splits=n_splits if bm is None else None, split_workspace=split_ws,
               block_mask=bm)
        if mark is not None:
            mark[1].record(stream)

    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()

    # Timed region: exactly `steps` steps back to back on one stream,
    # bracketed by device synchronisation.  Events on the launch stream
    # around each attention launch give its duration.
    E = lambda: torch.cuda.Event(enable_timing=True)  # noqa: E731
    ev0, ev1 = E(), E()
    marks = [(E(), E()) for _ in range(args.steps)]
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    ev0.record(stream)
    for i in range(args.steps):
        step(marks[i])
    ev1.record(stream)
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    per = [a.elapsed_time(b) for a, b in marks]
    total_ms = ev0.elapsed_time(ev1)
    ms_per_step = total_ms / args.steps
    if args.which == "bwd":
        flop = 2.5 * flop     # five contractions per visible pair instead of two
    value = flop / (ms_per_step * 1e-3) / 1e12
    avg_launch_ms = sum(per) / len(per)
    achieved = flop / (avg_launch_ms * 1e-3) / 1e12
    # The rest of a step: the gaps between launches.
    gap_ms = [marks[i][1].elapsed_time(marks[i + 1][0]) for i in range(args.steps - 1)]

    ctr = counters_for(kname, w["name"]) if args.which == "fwd" else None
    ghz = clock_of(ctr, avg_launch_ms)
    clock = None
    if ghz is not None:
        clock = {"ghz": round(ghz, 3),
                 "source": "GRBM_GUI_ACTIVE per XCD (committed counter run) / live launch time",
                 "counter_run_ghz": round(ctr["grbm_gui_active_per_dispatch"] / XCDS /
                                          ctr["dispatch_ns"], 3)}
    traffic = ctr["hbm_bytes_per_launch"] if ctr else None
    if decode:
        # HBM-bound: algorithmic bytes = Q, K and the packed V^T read once,
        # O (out dtype) and L written once; per attention call.
        esz = 4 if w["dtype"] == "fp32" else 2
        osz = 4 if args.out_dtype == "fp32" else esz
        qrows = w["B"] * w["N"] if cu is None else int(w["cu_seqlens"][-1])
        krows = w["B"] * Nk if cuk is None else int(w["cu_seqlens_k"][-1])
        nbytes = (qrows * w["Hq"] * w["d"] * (esz + osz) + 2 * krows * w["Hkv"] * w["d"] * esz
                  + w["B"] * w["Hq"] * w["N"] * 4)
        gbs = nbytes / (avg_launch_ms * 1e-3) / 1e9
        roofline = {"bound": "hbm", "achieved": round(gbs, 1), "peak": PEAK_HBM_GBS,
                    "unit": "GB/s", "frac": round(gbs / PEAK_HBM_GBS, 4),
                    "traffic": traffic, "clock": clock,
                    "algorithmic_bytes_per_launch": nbytes, "num_splits": n_splits}
    else:
        peak = PEAK_TFLOPS[w["dtype"]]
        roofline = {"bound": "mfma", "achieved": round(achieved, 2),
                    "peak": peak, "unit": "TFLOP/s",
                    "frac": round(achieved / peak, 4), "traffic": traffic, "clock": clock}
        if ghz is not None:
            # The same fraction against the peak at the measured clock.
            roofline["frac_at_clock"] = round(achieved / (peak * ghz / PEAK_CLOCK_GHZ), 4)
    rec = {
        "metric": (METRIC if args.which == "fwd" and w["name"] == "gqa_bf16" else
                   f"attention {args.which} TFLOP/s at 1 MI355X (% of MFMA peak), {w['name']}"),
        "value": round(value, 2), "unit": "TFLOP/s", "n_gpus": 1,
        "steps": args.steps, "warmup": args.warmup, "ms_per_step": round(ms_per_step, 4),
        "higher_is_better": True, "scaling": "weak", "vs_baseline": None,
        "cache": "cold (512 MiB written before each step)" if args.cold else "warm",
        "dtype": w["dtype"], "data": "synthetic",
        "config": {"workload": w["name"], "B": w["B"], "Hq": w["Hq"], "Hkv": w["Hkv"],
                   "N": w["N"], "Nk": Nk, "d": w["d"], "causal": w["causal"],
                   "out_dtype": args.out_dtype, "pass": args.which,
                   "kernel": kname if args.which == "fwd" else
                   "fa_bwd (fa_bwd_delta, fa_bwd_dkdv, fa_bwd_dq)",
                   "algorithmic_flop_per_step": flop},
        "roofline": roofline,
        "timing": {"attn_launch_ms_avg": round(avg_launch_ms, 4),
                   "attn_launch_ms_min": round(min(per), 4),
                   "attn_launch_ms_median": round(sorted(per)[len(per) // 2], 4),
                   "gap_ms_avg": round(sum(gap_ms) / len(gap_ms), 4) if gap_ms else None,
                   "wall_s": round(wall, 4)},
    }
    if args.calibrate_copy_mib > 0:
        n = args.calibrate_copy_mib * (1 << 20) // 4
        src = torch.ones(n, dtype=torch.float32, device=dev)
        dst = torch.empty_like(src)
        torch.cuda.synchronize()
        torch.mul(src, 1.0, out=dst)   # one elementwise pass: n*4 bytes in, n*4 out
        torch.cuda.synchronize()
        rec["copy_calibration_bytes"] = n * 4
    rec["device"] = {"name": torch.cuda.get_device_properties(dev).name,
                     "arch": torch.cuda.get_device_properties(dev).gcnArchName,
                     "cus": torch.cuda.get_device_properties(dev).multi_processor_count,
                     "hip": torch.version.hip, "torch": torch.__version__,
                     "library_version": fa.version(), "seed": w["seed"],
                     "kernel_source_sha": source_digest(kname) if args.which == "fwd" else
                     source_digest("fa_bwd")}
    if not args.no_cpu_baseline:
        if args.which == "bwd":
            rec["cpu_baseline"] = cpu_baseline_bwd(w, args.cpu_sample_heads)
        else:
            rec["cpu_baseline"] = cpu_baseline(w, args.cpu_sample_heads,
                                               o.double().cpu().numpy(),
                                               lse.double().cpu().numpy())
    print(json.dumps(rec), flush=True)


if __name__ == "__main__":
    main()
