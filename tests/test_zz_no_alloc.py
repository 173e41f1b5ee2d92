"""bsa_select_noalloc (the allocation-free selection, workspace in the
library's static device scratch) through the C ABI, against bsa_select with
a caller workspace: idx and cnt must be bit-identical. Two calls in a row,
the second on a smaller problem, so anything the first call leaves in the
shared scratch would show."""

from __future__ import annotations

import numpy as np
import pytest

import parity as PT
from video_dit_block_bsa_amd import binding as B
from video_dit_block_bsa_amd.binding import Problem, SelectParams
from video_dit_block_bsa_amd.inputs import make_qkv

pytestmark = pytest.mark.gpu


def _both(problem, params, q, k):
    import torch

    qd, kd = PT.to_device(q), PT.to_device(k)
    idx_ref, cnt_ref = PT.run_select(problem, params, qd, kd)
    stride = B.index_stride(problem, params)
    rows = problem.batch * problem.heads * problem.num_blocks
    idx = torch.full((rows, stride), -7, dtype=torch.int32, device="cuda")
    cnt = torch.full((rows,), -7, dtype=torch.int32, device="cuda")
    B.bsa_select_noalloc(problem, params, qd, kd, idx, cnt)
    torch.cuda.synchronize()
    return idx_ref.cpu().numpy(), cnt_ref.cpu().numpy(), idx.cpu().numpy(), cnt.cpu().numpy()


CASES = [
    # 480p coarse-stage grid, 32 heads, top-11 (the larger call first)
    (dict(T=12, H=32, W=56, heads=32), SelectParams.topk(11), 1),
    # then a smaller grid with condition frames and CDF selection
    (dict(T=8, H=16, W=32, heads=2, cond_frames=4), SelectParams.cdf(0.9, 2, 12), 7),
    # and a cut grid (partial blocks), smaller again
    (dict(T=6, H=6, W=12, heads=2), SelectParams.topk(3), 43),
]


def test_noalloc_matches_select_on_consecutive_calls():
    for kw, params, seed in CASES:
        problem = Problem.make(**kw)
        assert B.select_workspace_bytes(problem, params) <= B.select_noalloc_max_workspace_bytes()
        q, k, _ = make_qkv(kw["T"], kw["H"], kw["W"], kw["heads"], kind="field", seed=seed)
        idx_ref, cnt_ref, idx, cnt = _both(problem, params, q, k)
        print(f"{kw}: {int(cnt.sum())} kept pairs", flush=True)
        assert np.array_equal(cnt, cnt_ref)
        assert np.array_equal(idx, idx_ref)


def test_noalloc_rejects_a_problem_beyond_the_scratch():
    problem = Problem.make(56, 48, 80, 32, batch=4)
    params = SelectParams.topk(105)
    assert B.select_workspace_bytes(problem, params) > B.select_noalloc_max_workspace_bytes()
    with pytest.raises(B.BSAError, match="static scratch"):
        B.bsa_select_noalloc(problem, params, 0x10000, 0x10000, 0x10000, 0x10000)
