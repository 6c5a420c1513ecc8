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


def test_traffic_lookup_requires_matching_source():
    sys.path.insert(0, ROOT)
    import bench
    path = os.path.join(ROOT, "profiles", "traffic_gqa_bf16.json")
    with open(path) as f:
        t = json.load(f)
    got = bench.traffic_for(t["kernel"], "gqa_bf16")
    if t["kernel_source_sha"] == bench.source_digest():
        assert got == t["hbm_bytes_per_launch"]
    else:
        assert got is None
    assert bench.traffic_for("some_other_kernel", "gqa_bf16") is None
    assert bench.traffic_for(t["kernel"], "no_such_workload") is None
