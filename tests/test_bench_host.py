"""Host-side checks of bench.py and the workload table (CPU only)."""

import json
import os
import subprocess
import sys

import pytest

from video_dit_block_bsa_amd import WORKLOADS, effective_flops

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def test_more_than_one_gpu_exits_with_a_message():
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"],
                       capture_output=True, text=True, timeout=120)
    assert r.returncode == 2
    assert "one GPU" in r.stderr


@pytest.mark.parametrize("name,kept_per_row,want_tflop", [
    ("tiny", 2, 0.134e-3),     # 512 tokens, 2 heads, k = 2
    ("480p", 11, 0.496),
    ("720p", 45, 8.70),
    ("long", 105, 47.35),
])
def test_effective_flops_closed_form(name, kept_per_row, want_tflop):
    """4 * N * kept_keys * d per head: with top-k every query block keeps k
    key blocks of 128 tokens."""
    w = WORKLOADS[name]
    kept = w.heads * w.batch * w.num_blocks * kept_per_row
    got = effective_flops(w, kept)
    assert got == 4.0 * w.seq_len * kept_per_row * 128 * 128 * w.heads * w.batch
    assert abs(got / 1e12 - want_tflop) <= 0.005 * want_tflop


def test_traffic_record_matches_kernel_source():
    """The counter record bench.py reports as roofline traffic was taken on
    the attention kernel as it stands (the record carries the source hash)."""
    sys.path.insert(0, ROOT)
    import bench

    with open(bench.TRAFFIC_FILE) as f:
        rec = json.load(f)
    assert rec["kernel_source_sha"] == bench.kernel_source_hash()
    for name in ("long", "720p", "480p", "vc"):
        assert bench.traffic_for(name) > 0
