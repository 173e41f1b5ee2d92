"""64-token query blocks taken in t-adjacent pairs (GPU against the oracle).

With 128-token key blocks, the sparse kernel and dQ run one workgroup per
pair of query blocks at t-rows 2m and 2m+1 (after an odd number of rows the
last one alone) and walk the union of the two key lists. These cases check
that each block still attends exactly to its own list: selections from the
select kernel, hand-made lists (unordered, ids outside [0, Nk), a list
that one block of a pair has and the other lacks, empty lists), random
shuffled lists, the log-normaliser output, and grids with an odd number of
t-rows. The dense baseline runs 64-token chunks on boxes of twice their
depth where those tile the grid; its cases come last.
"""

from __future__ import annotations

import math

import numpy as np
import pytest

import parity as PT
from oracle import bsa_oracle as O
from test_gpu_parity import _run_and_compare
from video_dit_block_bsa_amd.binding import Problem, SelectParams
from video_dit_block_bsa_amd.inputs import make_grad, make_qkv

pytestmark = pytest.mark.gpu

SCALE = 1.0 / math.sqrt(128)


def _log(*a):
    print(*a, flush=True)


@pytest.mark.parametrize("grid,chunk,key_chunk,params,cond", [
    ((12, 16, 32), (2, 4, 8), (4, 4, 8), SelectParams.cdf(0.8, 2, 9), 4),   # paired, condition rows
    ((8, 8, 32), (1, 8, 8), (2, 8, 8), SelectParams.topk(3), 0),            # paired, another chunk
    ((4, 32, 64), (2, 4, 8), (2, 8, 8), SelectParams.topk(7), 0),           # one pair of t-rows
    ((6, 16, 32), (2, 4, 8), (2, 8, 8), SelectParams.topk(3), 0),           # odd t-rows: last alone
])
def test_pairs_select_and_attend(grid, chunk, key_chunk, params, cond):
    T, H, W = grid
    _log(f"grid {grid} chunk {chunk} key chunk {key_chunk} cond {cond}")
    q, k, v = make_qkv(T, H, W, 2, kind="field", seed=83)
    problem = Problem.make(T, H, W, 2, chunk=chunk, cond_frames=cond, key_chunk=key_chunk)
    _run_and_compare(problem, params, q, k, v)


def _attend_lists(problem, q, k, v, idx, cnt, stride):
    """Run bsa_attention on host lists and compare every block with the
    oracle over the valid ids of its clamped list."""
    import torch

    g = PT.geometry(problem)
    nbk = O.key_geometry(g).num_blocks
    qd, kd, vd = PT.to_device(q), PT.to_device(k), PT.to_device(v)
    idx_d = torch.from_numpy(np.ascontiguousarray(idx, dtype=np.int32)).to("cuda")
    cnt_d = torch.from_numpy(np.ascontiguousarray(cnt, dtype=np.int32)).to("cuda")
    out = PT.from_device(PT.run_attention(problem, qd, kd, vd, idx_d, cnt_d, stride)).reshape(q.shape)
    nb = g.num_blocks

    def blocks(p, i):
        row = idx[p * nb + i, : min(max(int(cnt[p * nb + i]), 0), stride)]
        return [int(b) for b in row if 0 <= b < nbk]

    pairs = q.shape[0] * q.shape[1]
    empty = [(p, i) for p in range(pairs) for i in range(nb) if not blocks(p, i)]
    items = [(p, i) for p in range(pairs) for i in range(nb) if blocks(p, i)]
    mx, mean, nvals = PT.compare_outputs(out, q, k, v, g, blocks, SCALE, items)
    _log(f"outputs: max-abs {mx:.3e}, mean-abs {mean:.3e} over {nvals} values; {len(empty)} empty rows")
    assert mx <= PT.MAX_ABS and mean <= PT.MEAN_ABS
    perm = O.block_token_order(g)
    for p, i in empty:
        b, h = divmod(p, q.shape[1])
        assert np.all(out[b, h][O.block_tokens(perm, i, g.n)] == 0)


def test_pairs_lone_last_row_lists():
    """Grid 6x8x16, query chunk (2,4,8): three t-rows of 4 blocks, pairs
    (0,4), (1,5), (2,6), (3,7) and blocks 8..11 alone; shuffled lists."""
    T, H, W = 6, 8, 16
    q, k, v = make_qkv(T, H, W, 1, kind="iid", seed=91)
    problem = Problem.make(T, H, W, 1, chunk=(2, 4, 8), key_chunk=(2, 8, 8))
    nbk = 3 * 1 * 2
    rng = np.random.default_rng(792)
    idx = np.stack([rng.permutation(nbk)[:4] for _ in range(12)]).astype(np.int32)
    cnt = rng.integers(0, 5, size=12).astype(np.int32)
    cnt[8] = 4
    _attend_lists(problem, q, k, v, idx, cnt, 4)


def test_pairs_hand_lists():
    """Grid 4x8x16, query chunk (2,4,8): 8 query blocks in pairs (0,4),
    (1,5), (2,6), (3,7); key chunk (4,4,8): 4 key blocks."""
    T, H, W = 4, 8, 16
    q, k, v = make_qkv(T, H, W, 1, kind="iid", seed=84)
    problem = Problem.make(T, H, W, 1, chunk=(2, 4, 8), key_chunk=(4, 4, 8))
    idx = np.array([
        [3, 0, 2, -1],    # 0: unordered
        [1, 3, 0, 0],     # 1: only its first two count (cnt 2)
        [-1, 3, 99, 1],   # 2: ids outside the key grid between valid ones
        [2, 0, 0, 0],     # 3
        [0, 2, 3, 1],     # 4: partly ascending, shares 0, 2, 3 with block 0
        [1, 2, 3, 0],     # 5: cnt 0, gets zeros
        [1, 3, -1, -1],   # 6: the same set as block 2 in another order
        [3, 2, 1, 0],     # 7: descending, all four
    ], dtype=np.int32)
    cnt = np.array([3, 2, 4, 1, 4, 0, 2, 9], dtype=np.int32)  # 9 is clamped to the stride
    _attend_lists(problem, q, k, v, idx, cnt, 4)


@pytest.mark.parametrize("seed", [0, 1])
def test_pairs_random_shuffled_lists(seed):
    """Random distinct ids per block, shuffled, with random counts (empty
    rows included) and some ids outside [0, Nk)."""
    T, H, W, heads = 8, 16, 32, 2
    q, k, v = make_qkv(T, H, W, heads, kind="iid", seed=85 + seed)
    problem = Problem.make(T, H, W, heads, chunk=(2, 4, 8), key_chunk=(4, 4, 8))
    g = PT.geometry(problem)
    nbk = O.key_geometry(g).num_blocks
    rows, stride = heads * g.num_blocks, 12
    rng = np.random.default_rng(700 + seed)
    idx = np.full((rows, stride), -1, dtype=np.int32)
    cnt = rng.integers(0, stride + 1, size=rows).astype(np.int32)
    for r in range(rows):
        ids = rng.choice(nbk, size=stride, replace=False).astype(np.int32)
        bad = rng.random(stride) < 0.15
        ids[bad] = rng.choice([-7, -1, nbk, nbk + 40], size=int(bad.sum()))
        idx[r] = ids
    _attend_lists(problem, q, k, v, idx, cnt, stride)


def test_pairs_lse():
    """bsa_attention_lse on paired blocks: the same o as bsa_attention and
    lse against the oracle's."""
    import torch

    from video_dit_block_bsa_amd import binding as B

    T, H, W = 8, 16, 32
    q, k, v = make_qkv(T, H, W, 2, kind="field", seed=86)
    problem = Problem.make(T, H, W, 2, chunk=(2, 4, 8), key_chunk=(4, 4, 8), cond_frames=4)
    g = PT.geometry(problem)
    qd, kd, vd = PT.to_device(q), PT.to_device(k), PT.to_device(v)
    params = SelectParams.topk(5)
    stride = B.index_stride(problem, params)
    idx_d, cnt_d = PT.run_select(problem, params, qd, kd)
    o1 = PT.run_attention(problem, qd, kd, vd, idx_d, cnt_d, stride)
    o2 = torch.full_like(qd, float("nan"))
    lse = torch.full(q.shape[:3], float("nan"), dtype=torch.float32, device="cuda")
    B.bsa_attention_lse(problem, qd, kd, vd, idx_d, cnt_d, stride, o2, lse,
                        torch.empty(16, dtype=torch.uint8, device="cuda"))
    torch.cuda.synchronize()
    assert torch.equal(o1.view(torch.int16), o2.view(torch.int16))
    idx = idx_d.cpu().numpy()
    cnt = cnt_d.cpu().numpy()
    nb = g.num_blocks
    for h in range(2):
        _, lse_r = O.forward_lse_head(*(O.bf16_bits_to_f64(a[0, h]) for a in (q, k, v)), g,
                                      idx[h * nb:(h + 1) * nb], cnt[h * nb:(h + 1) * nb], SCALE)
        err = np.abs(lse[0, h].cpu().numpy() - lse_r).max()
        _log(f"lse head {h}: max-abs {err:.3e}")
        assert err <= 2.5e-3


# Backward: dQ takes the same pairs (dK/dV is unchanged); every gradient
# element against the oracle, on the oracle's selection and on shuffled
# random lists with invalid ids and empty rows.
@pytest.mark.parametrize("grid,chunk,key_chunk,k_sel,cond", [
    ((8, 16, 32), (2, 4, 8), (4, 4, 8), 5, 4),    # paired, condition rows
    ((8, 8, 32), (1, 8, 8), (2, 8, 8), 3, 0),     # paired, another chunk
    ((6, 16, 32), (2, 4, 8), (2, 8, 8), 3, 0),    # odd t-rows: last alone
])
def test_pairs_backward_selection(grid, chunk, key_chunk, k_sel, cond):
    from test_gpu_backward import _case

    _case(*grid, 2, k_sel, chunk=chunk, kind="field", seed=87, cond_frames=cond,
          key_chunk=key_chunk)


def test_pairs_backward_shuffled_lists():
    from test_gpu_backward import compare_all

    T, H, W, heads = 8, 16, 32, 2
    q, k, v = make_qkv(T, H, W, heads, kind="field", seed=88)
    do = make_grad(T, H, W, heads, seed=88)
    problem = Problem.make(T, H, W, heads, chunk=(2, 4, 8), key_chunk=(4, 4, 8))
    g = PT.geometry(problem)
    nbk = O.key_geometry(g).num_blocks
    rows, stride = heads * g.num_blocks, 10
    rng = np.random.default_rng(789)
    idx = np.full((rows, stride), -1, dtype=np.int32)
    cnt = rng.integers(0, stride + 1, size=rows).astype(np.int32)
    for r in range(rows):
        ids = rng.choice(nbk, size=stride, replace=False).astype(np.int32)
        bad = rng.random(stride) < 0.15
        ids[bad] = rng.choice([-2, nbk, nbk + 9], size=int(bad.sum()))
        idx[r] = ids
    compare_all(problem, q, k, v, do, idx, cnt, stride)


# Dense baseline with 64-token query chunks: boxes of twice the chunk's depth
# when they tile the grid and the condition rows, the chunk itself otherwise.
@pytest.mark.parametrize("grid,chunk,cond,batch,heads", [
    ((8, 16, 32), (2, 4, 8), 0, 1, 2),     # doubled boxes
    ((8, 8, 32), (1, 8, 8), 2, 2, 3),      # doubled boxes, condition rows, batch 2
    ((12, 16, 16), (4, 2, 8), 4, 1, 2),    # three t-rows: the chunk itself
    ((8, 16, 32), (2, 4, 8), 2, 1, 2),     # one condition row: the chunk itself
])
def test_dense_64_token_chunks(grid, chunk, cond, batch, heads):
    T, H, W = grid
    q, k, v = make_qkv(T, H, W, heads, batch=batch, kind="field", seed=92)
    problem = Problem.make(T, H, W, heads, batch=batch, chunk=chunk, cond_frames=cond)
    g = PT.geometry(problem)
    out = PT.from_device(PT.run_dense(problem, *(PT.to_device(a) for a in (q, k, v))))
    out = out.reshape(q.shape)
    for b in range(batch):
        for h in range(heads):
            ref = O.dense_head(*(O.bf16_bits_to_f64(a[b, h]) for a in (q, k, v)), g, SCALE)
            err = np.abs(O.bf16_bits_to_f64(out[b, h]) - ref)
            _log(f"dense ({b},{h}): max-abs {err.max():.3e}, mean-abs {err.mean():.3e}")
            assert err.max() <= PT.MAX_ABS and err.mean() <= PT.MEAN_ABS
