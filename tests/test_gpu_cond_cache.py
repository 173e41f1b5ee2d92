"""GPU tests of the condition-KV cache path (bsa_pool_cond_keys,
bsa_select_noisy, bsa_attention_noisy) through the C ABI.

Two denoising steps are simulated: the condition tokens (the first
cond_frames latent frames) keep their Q/K/V, the noisy tokens are redrawn.
On each step the cached path's noisy rows of idx, cnt and o must be
bit-identical to the full path's (bsa_select + bsa_attention on the same
tensors), its condition rows must be left untouched, and a sample of noisy
query blocks is compared with the oracle (max-abs <= 2e-2, mean-abs <= 1e-3,
the tolerances of the forward parity tests).
"""

from __future__ import annotations

import math

import numpy as np
import pytest

import oracle.bsa_oracle as O
import parity as PT
from video_dit_block_bsa_amd.binding import Problem, SelectParams
from video_dit_block_bsa_amd.inputs import make_qkv

pytestmark = pytest.mark.gpu

SCALE = 1.0 / math.sqrt(128)


def _log(*a):
    print(*a, flush=True)


def _step_tensors(T, H, W, heads, cond_frames, seed0, seed1):
    """Step 0 draws all tokens; step 1 keeps the condition tokens of step 0
    and redraws the noisy ones."""
    a = make_qkv(T, H, W, heads, kind="field", seed=seed0)
    b = make_qkv(T, H, W, heads, kind="field", seed=seed1)
    n_cond = cond_frames * H * W
    step1 = []
    for x0, x1 in zip(a, b):
        x = x1.copy()
        x[:, :, :n_cond] = x0[:, :, :n_cond]
        step1.append(x)
    return a, tuple(step1)


@pytest.mark.parametrize("grid,chunk,key_chunk,params,cond", [
    ((16, 16, 32), (4, 4, 8), None, SelectParams.topk(6), 4),
    ((16, 16, 32), (4, 4, 8), None, SelectParams.cdf(0.8, 2, 10), 4),
    ((16, 16, 32), (4, 4, 8), (2, 4, 8), SelectParams.topk(9), 4),
    ((16, 16, 32), (4, 4, 8), (4, 8, 8), SelectParams.topk(3), 4),
    # 64-token query blocks: the noisy rows start on an even t-row (paired
    # blocks) or on an odd one (one block per workgroup)
    ((16, 16, 32), (2, 4, 8), (4, 4, 8), SelectParams.topk(5), 4),
    ((16, 16, 32), (2, 4, 8), (2, 8, 8), SelectParams.topk(5), 4),
    ((16, 16, 32), (2, 4, 8), (2, 8, 8), SelectParams.cdf(0.8, 2, 8), 2),
    # partial blocks along t, h and w
    ((14, 18, 36), (4, 4, 8), None, SelectParams.topk(6), 4),
    ((14, 18, 36), (4, 4, 8), (4, 8, 8), SelectParams.cdf(0.8, 1, 8), 4),
])
def test_noisy_rows_match_full_path(grid, chunk, key_chunk, params, cond):
    import torch

    from video_dit_block_bsa_amd import binding as B

    (T, H, W), heads = grid, 2
    problem = Problem.make(T, H, W, heads, chunk=chunk, cond_frames=cond, key_chunk=key_chunk)
    g = PT.geometry(problem)
    nb, cq = g.num_blocks, g.cond_blocks
    stride = B.index_stride(problem, params)
    steps = _step_tensors(T, H, W, heads, cond, 51, 52)
    cache = torch.full((max(B.cond_cache_bytes(problem), 16) // 4,), float("nan"), dtype=torch.float32,
                       device="cuda")
    ws = torch.empty(B.select_workspace_bytes(problem, params), dtype=torch.uint8, device="cuda")
    wsa = torch.empty(16, dtype=torch.uint8, device="cuda")
    for step, (q, k, v) in enumerate(steps):
        qd, kd, vd = PT.to_device(q), PT.to_device(k), PT.to_device(v)
        if step == 0:
            B.bsa_pool_cond_keys(problem, kd, cache)
        # Full path.
        idx_f, cnt_f = PT.run_select(problem, params, qd, kd)
        o_f = PT.run_attention(problem, qd, kd, vd, idx_f, cnt_f, stride)
        # Cached path; condition rows carry sentinels that must survive.
        idx_c = torch.full_like(idx_f, -7)
        cnt_c = torch.full_like(cnt_f, -7)
        B.bsa_select_noisy(problem, params, qd, kd, cache, idx_c, cnt_c, ws)
        o_c = torch.full_like(qd, float("nan"))
        B.bsa_attention_noisy(problem, qd, kd, vd, idx_c, cnt_c, stride, o_c, wsa)
        torch.cuda.synchronize()
        rows_f = idx_f.view(heads, nb, stride)
        rows_c = idx_c.view(heads, nb, stride)
        assert torch.equal(rows_c[:, cq:], rows_f[:, cq:]), "noisy idx rows differ"
        assert torch.equal(cnt_c.view(heads, nb)[:, cq:], cnt_f.view(heads, nb)[:, cq:])
        assert bool((rows_c[:, :cq] == -7).all()) and bool((cnt_c.view(heads, nb)[:, :cq] == -7).all())
        of = PT.from_device(o_f).reshape(q.shape)
        oc = PT.from_device(o_c).reshape(q.shape)
        n_cond = cond * H * W
        assert np.array_equal(oc[:, :, n_cond:], of[:, :, n_cond:]), "noisy o rows differ"
        assert np.all(np.isnan(O.bf16_bits_to_f64(oc[:, :, :n_cond]))), "condition rows written"
        # The oracle on a sample of noisy query blocks (the GPU's lists, which
        # the full path's parity tests validate against the oracle selection).
        idx_n = idx_c.cpu().numpy()
        cnt_n = cnt_c.cpu().numpy()
        items = [(p, i) for p in range(heads) for i in (cq, cq + 1, nb // 2, nb - 1)]
        mx, mean, nvals = PT.compare_outputs(
            oc, q, k, v, g, lambda p, i: idx_n[p * nb + i, : cnt_n[p * nb + i]], SCALE, items)
        _log(f"step {step}: noisy rows bit-identical; oracle max-abs {mx:.3e}, mean-abs {mean:.3e}")
        assert mx <= PT.MAX_ABS and mean <= PT.MEAN_ABS


def test_vc_workload_full_size():
    """The video-continuation workload (61,440 tokens, 4 condition frames,
    32 heads, CDF 0.9 in [4, 64]) in the configuration the benchmark times:
    the cached path's noisy rows equal the full path's, bit for bit."""
    import torch

    from video_dit_block_bsa_amd import WORKLOADS
    from video_dit_block_bsa_amd import binding as B

    w = WORKLOADS["vc"]
    problem = Problem.from_workload(w)
    params = SelectParams.from_workload(w)
    stride = B.index_stride(problem, params)
    g = PT.geometry(problem)
    nb, cq = g.num_blocks, g.cond_blocks
    q, k, v = make_qkv(w.T, w.H, w.W, w.heads, kind=w.kind, seed=w.seed)
    qd, kd, vd = PT.to_device(q), PT.to_device(k), PT.to_device(v)
    idx_f, cnt_f = PT.run_select(problem, params, qd, kd)
    o_f = PT.run_attention(problem, qd, kd, vd, idx_f, cnt_f, stride)
    cache = torch.empty(B.cond_cache_bytes(problem) // 4, dtype=torch.float32, device="cuda")
    ws = torch.empty(B.select_workspace_bytes(problem, params), dtype=torch.uint8, device="cuda")
    B.bsa_pool_cond_keys(problem, kd, cache)
    idx_c = torch.full_like(idx_f, -7)
    cnt_c = torch.full_like(cnt_f, -7)
    B.bsa_select_noisy(problem, params, qd, kd, cache, idx_c, cnt_c, ws)
    o_c = torch.full_like(qd, float("nan"))
    B.bsa_attention_noisy(problem, qd, kd, vd, idx_c, cnt_c, stride, o_c, ws)
    torch.cuda.synchronize()
    h = w.heads
    assert torch.equal(idx_c.view(h, nb, stride)[:, cq:], idx_f.view(h, nb, stride)[:, cq:])
    assert torch.equal(cnt_c.view(h, nb)[:, cq:], cnt_f.view(h, nb)[:, cq:])
    n_cond = w.cond_frames * w.H * w.W
    assert torch.equal(o_c[:, :, n_cond:].view(torch.int16), o_f[:, :, n_cond:].view(torch.int16))
    assert bool(torch.isnan(o_c[:, :, :n_cond].float()).all())


def test_noisy_path_many_heads_launch_groups():
    """Many heads: both attention paths go out as launches of 7,680
    workgroups (the full path's 33,280 in five, the noisy path's 16,640, one
    per noisy query block, in three). 1040 heads are 65 copies of 16 seeded
    heads; the cached path's noisy rows equal the full path's, and every
    head's output equals its base head's in a 16-head problem (one launch),
    bit for bit."""
    import torch

    from video_dit_block_bsa_amd import binding as B

    T, H, W, base, copies, cond = 8, 16, 32, 16, 65, 4
    params = SelectParams.topk(4)
    q, k, v = make_qkv(T, H, W, base, kind="field", seed=61)
    qb, kb, vb = PT.to_device(q), PT.to_device(k), PT.to_device(v)
    small = Problem.make(T, H, W, base, cond_frames=cond)
    big = Problem.make(T, H, W, base * copies, cond_frames=cond)
    g = PT.geometry(big)
    nb, cq = g.num_blocks, g.cond_blocks
    assert big.heads * (nb - cq) > 2 * 7680
    stride = B.index_stride(big, params)
    idx_s, cnt_s = PT.run_select(small, params, qb, kb)
    o_s = PT.run_attention(small, qb, kb, vb, idx_s, cnt_s, stride)
    qd, kd, vd = (t.repeat(1, copies, 1, 1).contiguous() for t in (qb, kb, vb))
    del qb, kb, vb
    idx_f, cnt_f = PT.run_select(big, params, qd, kd)
    o_f = PT.run_attention(big, qd, kd, vd, idx_f, cnt_f, stride)
    cache = torch.empty((max(B.cond_cache_bytes(big), 16) // 4,), dtype=torch.float32, device="cuda")
    ws = torch.empty(B.select_workspace_bytes(big, params), dtype=torch.uint8, device="cuda")
    B.bsa_pool_cond_keys(big, kd, cache)
    idx_c = torch.full_like(idx_f, -7)
    cnt_c = torch.full_like(cnt_f, -7)
    B.bsa_select_noisy(big, params, qd, kd, cache, idx_c, cnt_c, ws)
    o_c = torch.full_like(qd, float("nan"))
    B.bsa_attention_noisy(big, qd, kd, vd, idx_c, cnt_c, stride, o_c, torch.empty(16, dtype=torch.uint8,
                                                                                     device="cuda"))
    torch.cuda.synchronize()
    n_cond = cond * H * W
    of = o_f.view(torch.int16).view(copies, base, -1, 128)
    oc = o_c.view(torch.int16).view(copies, base, -1, 128)
    os_ = o_s.view(torch.int16).view(1, base, -1, 128)
    assert torch.equal(of, os_.expand_as(of)), "grouped launches changed a head's output"
    assert torch.equal(oc[:, :, n_cond:], of[:, :, n_cond:]), "noisy o rows differ"
    rows_f = idx_f.view(-1, nb, stride)
    rows_c = idx_c.view(-1, nb, stride)
    assert torch.equal(rows_c[:, cq:], rows_f[:, cq:])
