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
