"""Host-side checks of the benchmark (no GPU): the one-GPU refusal, the
per-token byte table, and that the committed counter records were taken on
the kernel sources as they are now (a kernel change without new counters
would silently turn `roofline.traffic` into null)."""
import json
import os
import subprocess
import sys

import pytest

import bench
from oracle import oracle as O

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def test_more_than_one_gpu_is_refused():
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"], capture_output=True,
                       text=True, timeout=120, cwd=ROOT)
    assert r.returncode == 2
    line = json.loads(r.stdout.strip().splitlines()[-1])
    assert "one GPU" in line["error"]


def test_tier_token_bytes_follow_the_tier_table():
    # radius (2) + angle and magnitude codes (8 * (tb + sb)) + values
    # (fp16: 256; V8: 4 scale bytes + 128 codes)
    for t, (tb, sb) in O.TIER_BITS.items():
        assert bench.TIER_TOKEN_BYTES[t] == 2 + 8 * (tb + sb) + (132 if t >= 3 else 256), t


@pytest.mark.parametrize("workload", ["llama8b", "llama8b_v8", "long256k", "ragged", "rdr128k"])
def test_committed_counters_match_the_kernel_sources(workload):
    path = os.path.join(ROOT, "profiles", f"ada_decode_partials_{workload}_pmc.json")
    rec = json.load(open(path))
    assert rec["kernel_source_hash"] == bench.kernel_source_hash()
    traffic = bench.measured_traffic(workload)
    assert traffic == rec["hbm_bytes_per_launch"]
    # HBM bytes within a few percent above the algorithmic bytes
    assert 1.0 <= traffic / rec["algorithmic_bytes_per_launch"] < 1.15
