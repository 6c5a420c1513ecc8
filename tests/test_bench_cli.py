"""bench.py's command line without a GPU: more than one GPU is refused with
a message, and the host-side pieces it reports from (FLOP counting, traffic
lookup) behave."""
from __future__ import annotations

import json
import os
import subprocess
import sys

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def test_more_than_one_gpu_is_refused():
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"],
                       capture_output=True, text=True, timeout=120)
    assert r.returncode != 0
    assert "one GPU" in r.stderr


def test_counter_lookup_requires_matching_source(tmp_path, monkeypatch):
    sys.path.insert(0, ROOT)
    import bench
    kernel = "fa_fwd_mfma_bf16_d128_causal_of32"
    rec = {"kernel": kernel, "kernel_source_sha": bench.source_digest(kernel),
           "hbm_bytes_per_launch": 123, "grbm_gui_active_per_dispatch": 8.0e6,
           "dispatch_ns": 500000}
    (tmp_path / "profiles").mkdir()
    (tmp_path / "profiles" / "counters_gqa_bf16.json").write_text(json.dumps(rec))
    monkeypatch.setattr(bench, "ROOT", str(tmp_path))
    got = bench.counters_for(kernel, "gqa_bf16")
    assert got is not None and got["hbm_bytes_per_launch"] == 123
    # 8e6 cycles over 8 XCDs in 0.5 ms: 2 GHz
    assert abs(bench.clock_of(got, 0.5) - 2.0) < 1e-12
    assert bench.counters_for("fa_fwd_mfma_bf16_d64_causal_of32", "gqa_bf16") is None
    assert bench.counters_for(kernel, "no_such_workload") is None
    rec["kernel_source_sha"] = "0" * 16        # taken on another source
    (tmp_path / "profiles" / "counters_gqa_bf16.json").write_text(json.dumps(rec))
    assert bench.counters_for(kernel, "gqa_bf16") is None
    assert bench.clock_of(None, 0.5) is None


def test_committed_counter_summaries_are_well_formed():
    d = os.path.join(ROOT, "profiles")
    for name in sorted(os.listdir(d)):
        if not (name.startswith("counters_") and name.endswith(".json")):
            continue
        with open(os.path.join(d, name)) as f:
            t = json.load(f)
        assert t["workload"] == name[len("counters_"):-len(".json")]
        assert len(t["kernel_source_sha"]) == 16
        for key in ("hbm_bytes_per_launch", "grbm_gui_active_per_dispatch", "dispatch_ns"):
            assert t[key] > 0, (name, key)
        assert t["commands"], name


def _custom(lengths_q=None, lengths_k=None, N=None, Nk=None):
    import workloads
    w = workloads.make_custom_qk(2, 4, 2, 64, "bf16", seed=5, Nq=N, Nk=Nk,
                                 lengths_q=lengths_q, lengths_k=lengths_k)
    w.update(causal=True, scale=0.125, name="custom", seed=5)
    return w


def test_cpu_baseline_reports_the_timed_outputs_errors():
    """The CPU-baseline leg compares the outputs it is handed with the oracle
    on its sample: exact outputs give zero error; a disturbed O entry, an L
    row or a missing -inf show up (fixed, packed, and packed with separate
    key counts)."""
    import numpy as np

    import bench
    import oracle
    import workloads
    cases = [dict(N=70, Nk=70), dict(N=30, Nk=90),
             dict(lengths_q=[33, 5], lengths_k=[33, 5]),
             dict(lengths_q=[8, 20], lengths_k=[40, 0])]
    for kw in cases:
        w = _custom(**kw)
        q, k, v = (workloads.to_f64(w[x], "bf16") for x in "qkv")
        if w["cu_seqlens"] is None:
            O, L = oracle.attention_qk(q, k, v, causal=True, scale=0.125)
        else:
            O, L = oracle.attention_qk(q, k, v, causal=True, scale=0.125,
                                       cu_seqlens_q=w["cu_seqlens"],
                                       cu_seqlens_k=w["cu_seqlens_k"])
            if kw["lengths_q"] == kw["lengths_k"]:
                w["cu_seqlens_k"] = None     # equal counts: the plain packed form
        Lg = np.where(np.isnan(L), 7.0, L)  # the kernel leaves padding rows alone
        e = bench.cpu_baseline(w, 0, O, Lg)["errors"]
        assert e["o_max_abs"] == 0.0 and e["l_max_abs"] == 0.0 and e["l_neginf_match"], kw
        O2 = O.copy()
        O2.reshape(-1)[5] += 1e-3
        L2 = Lg.copy()
        fin = np.argwhere(np.isfinite(L))[0]
        L2[tuple(fin)] += 2e-3
        e = bench.cpu_baseline(w, 0, O2, L2)["errors"]
        assert abs(e["o_max_abs"] - 1e-3) < 1e-12 and abs(e["l_max_abs"] - 2e-3) < 1e-12, kw
        if np.isneginf(L).any():
            L3 = Lg.copy()
            L3[np.isneginf(L)] = 0.0
            assert not bench.cpu_baseline(w, 0, O, L3)["errors"]["l_neginf_match"], kw
