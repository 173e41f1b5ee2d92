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


@pytest.mark.parametrize("grid,chunk,key_chunk", [
    ((6, 6, 12), (4, 4, 8), ()),
    ((10, 20, 36), (4, 4, 8), (4, 8, 8)),
    ((93, 45, 80), (4, 4, 8), (2, 4, 8)),
    ((56, 48, 80), (4, 4, 8), ()),
])
def test_workload_block_counts_match_the_library(grid, chunk, key_chunk):
    """bench.py sizes idx and cnt from Workload.num_blocks: on a grid the
    chunk does not divide it must count partial blocks as the library does
    (ceilings), or bsa_select would write past the end of idx."""
    from video_dit_block_bsa_amd import binding as B
    from video_dit_block_bsa_amd.workloads import Workload

    w = Workload("t", *grid, heads=2, chunk=chunk, key_chunk=key_chunk)
    p = B.Problem.from_workload(w)
    assert w.num_blocks == p.num_blocks
    assert w.num_key_blocks == p.num_key_blocks
    # The library's own counts, read back from its workspace size (the layout
    # documented in bsa.h: pooled Q and pooled K, fp32, each part rounded up
    # to 256 bytes).
    nb, nk = w.num_blocks, w.num_key_blocks
    a = lambda x: -(-x // 256) * 256
    want = a(2 * nb * 512) + a(2 * nk * 512)
    assert B.select_workspace_bytes(p, B.SelectParams.topk(3)) == want


def test_roofline_names_the_closer_roof():
    """The record reports both fractions and binds to the larger one."""
    sys.path.insert(0, ROOT)
    import bench

    r = bench.roofline_record(47.352e12, 46.37, 328.2e9)  # 215K tokens, round-one figures
    assert r["bound"] == "hbm" and r["unit"] == "GB/s" and r["peak"] == 8000.0
    assert abs(r["frac_mfma"] - 47.352e12 / 46.37e-3 / 2.5e15) < 1e-4
    assert abs(r["frac_hbm"] - 328.2e9 / 46.37e-3 / 8e12) < 1e-4
    assert r["frac"] == r["frac_hbm"]
    r = bench.roofline_record(47.352e12, 46.37, 100e9)
    assert r["bound"] == "mfma" and r["frac"] == r["frac_mfma"]
    r = bench.roofline_record(47.352e12, 46.37, None)
    assert r["bound"] == "mfma" and r["frac_hbm"] is None


def test_attention_launch_count_mirrors_the_library():
    """bench.py divides the step's attention time and flops by the launches
    one bsa_attention call makes: the library sends sparse calls as launches
    of 7,680 workgroups (one per query block, or per t-adjacent pair of
    64-token query blocks)."""
    sys.path.insert(0, ROOT)
    import bench
    from video_dit_block_bsa_amd import WORKLOADS

    assert bench.LAUNCH_WORKGROUPS == 7680
    assert bench.attention_launches(WORKLOADS["long"]) == 7        # 32 x 1680 = 53,760
    assert bench.attention_launches(WORKLOADS["long_k64"]) == 7
    assert bench.attention_launches(WORKLOADS["long_k256"]) == 7
    assert bench.attention_launches(WORKLOADS["long_q64"]) == 7    # 32 x 1680 pairs
    assert bench.attention_launches(WORKLOADS["720p"]) == 3        # 32 x 720 = 23,040
    assert bench.attention_launches(WORKLOADS["vc"]) == 2          # 32 x 480 = 15,360
    assert bench.attention_launches(WORKLOADS["480p"]) == 1        # 32 x 168 = 5,376
    assert bench.attention_launches(WORKLOADS["tiny"]) == 1
    src = open(os.path.join(ROOT, "video_dit_block_bsa_amd", "csrc", "attention.hip")).read()
    assert "kLaunchWorkgroups = 15 * 512;" in src
    assert "(size_t)g.bh * g.nb <= 32768" in src and "kGroupHeads = 8" in src
