"""GPU parity: the HIP path (through the C ABI) against the CPU oracle.

Small problems are compared element by element over every query block;
the full-size workloads compare every index row and a seeded sample of
query blocks' outputs. Tolerances: index sets exact up to near-ties of
1e-5 in pooled score; outputs max-abs <= 2e-2 and mean-abs <= 1e-3.
"""

from __future__ import annotations

import math

import numpy as np
import pytest

import oracle.bsa_oracle as O
import parity as PT
from video_dit_block_bsa_amd import WORKLOADS
from video_dit_block_bsa_amd.binding import Problem, SelectParams
from video_dit_block_bsa_amd.inputs import make_qkv

pytestmark = pytest.mark.gpu

SCALE = 1.0 / math.sqrt(128)


def _log(*a):
    print(*a, flush=True)


def _run_and_compare(problem, params, q, k, v, all_outputs=True, sample=None, seed=0):
    g = PT.geometry(problem)
    sp = PT.oracle_params(params)
    stride = O.index_stride(sp)
    qd, kd, vd = PT.to_device(q), PT.to_device(k), PT.to_device(v)
    idx_d, cnt_d = PT.run_select(problem, params, qd, kd)
    o_d = PT.run_attention(problem, qd, kd, vd, idx_d, cnt_d, stride)
    idx = idx_d.cpu().numpy()
    cnt = cnt_d.cpu().numpy()
    out = PT.from_device(o_d).reshape(q.shape)
    rows = PT.oracle_select_all(q, k, g, sp, SCALE)
    exact, ties, fails = PT.check_selection(idx, cnt, rows, g, sp, stride)
    _log(f"selection: {exact} exact rows, {ties} near-tie rows, {len(fails)} failures")
    assert not fails, fails[:5]
    nb = g.num_blocks
    pairs = q.shape[0] * q.shape[1]
    if all_outputs:
        items = [(p, i) for p in range(pairs) for i in range(nb)]
    else:
        rng = np.random.default_rng(seed)
        heads = sorted(rng.choice(pairs, size=min(sample[0], pairs), replace=False).tolist())
        items = []
        for p in heads:
            blocks = set(rng.choice(nb, size=min(sample[1], nb), replace=False).tolist())
            blocks |= {0, nb - 1}
            if g.cond_blocks:
                blocks |= {g.cond_blocks - 1, g.cond_blocks}
            items += [(p, i) for i in sorted(blocks)]
    mx, mean, nvals = PT.compare_outputs(
        out, q, k, v, g, lambda p, i: idx[p * nb + i, : cnt[p * nb + i]], SCALE, items)
    _log(f"outputs: max-abs {mx:.3e}, mean-abs {mean:.3e} over {nvals} values")
    assert mx <= PT.MAX_ABS and mean <= PT.MEAN_ABS
    return idx, cnt, out, o_d


def test_tiny_topk2():
    w = WORKLOADS["tiny"]
    q, k, v = make_qkv(w.T, w.H, w.W, w.heads, kind=w.kind, seed=w.seed)
    _run_and_compare(Problem.from_workload(w), SelectParams.topk(2), q, k, v)


def test_tiny_all_blocks_equals_dense():
    """k = all blocks: BSA equals the oracle's dense attention and the GPU's
    own dense kernel."""
    w = WORKLOADS["tiny"]
    q, k, v = make_qkv(w.T, w.H, w.W, w.heads, kind=w.kind, seed=w.seed)
    problem = Problem.from_workload(w)
    _, _, out, o_sparse = _run_and_compare(problem, SelectParams.topk(4), q, k, v)
    g = PT.geometry(problem)
    o_dense = PT.run_dense(problem, PT.to_device(q), PT.to_device(k), PT.to_device(v))
    dense = PT.from_device(o_dense).reshape(q.shape)
    for h in range(w.heads):
        ref = O.dense_head(O.bf16_bits_to_f64(q[0, h]), O.bf16_bits_to_f64(k[0, h]),
                           O.bf16_bits_to_f64(v[0, h]), g, SCALE)
        err = np.abs(O.bf16_bits_to_f64(dense[0, h]) - ref)
        assert err.max() <= PT.MAX_ABS and err.mean() <= PT.MEAN_ABS
    # same tile engine, same key order: the two GPU results agree bitwise
    assert np.array_equal(dense, out)


@pytest.mark.parametrize(
    "grid,heads,k",
    [((8, 12, 40), 3, 5),     # 30 blocks: fewer than one 64-wide selection chunk
     ((12, 16, 48), 2, 7),    # 72 blocks: a ragged second chunk
     ((4, 4, 8), 2, 3)],      # a single block: k clamps to 1
)
def test_small_field_topk(grid, heads, k):
    T, H, W = grid
    q, k_, v = make_qkv(T, H, W, heads, kind="field", seed=T * 100 + W)
    _run_and_compare(Problem.make(T, H, W, heads), SelectParams.topk(k), q, k_, v)


@pytest.mark.parametrize(
    "chunk,grid",
    [((2, 8, 8), (6, 16, 24)),     # 36 blocks
     ((8, 4, 4), (16, 12, 8)),     # 12 blocks, deep in time
     ((1, 8, 16), (5, 16, 32)),    # 20 blocks, one frame per block
     ((4, 8, 4), (8, 16, 12)),     # 12 blocks
     ((1, 1, 128), (3, 4, 256))],  # 24 blocks, one row of 128 tokens each
)
def test_other_chunk_shapes(chunk, grid):
    """Block shapes other than [4,4,8]: every power-of-two chunk of 128
    tokens goes through the same tile-address arithmetic."""
    T, H, W = grid
    q, k, v = make_qkv(T, H, W, 2, kind="field", seed=sum(grid) + chunk[0])
    problem = Problem.make(T, H, W, 2, chunk=chunk)
    _run_and_compare(problem, SelectParams.topk(5), q, k, v)


def test_batch_two_three_heads():
    """batch > 1: rows and heads are laid out (batch, head, block)."""
    T, H, W = 8, 16, 32  # 16 blocks
    q, k, v = make_qkv(T, H, W, 3, batch=2, kind="field", seed=91)
    problem = Problem.make(T, H, W, 3, batch=2, cond_frames=4)
    _run_and_compare(problem, SelectParams.topk(6), q, k, v)


def test_small_cdf_block_causal():
    T, H, W = 12, 16, 32  # 48 blocks, 16 condition blocks
    q, k, v = make_qkv(T, H, W, 2, kind="field", seed=77)
    problem = Problem.make(T, H, W, 2, cond_frames=4)
    idx, cnt, _, _ = _run_and_compare(problem, SelectParams.cdf(0.9, 2, 12), q, k, v)
    assert cnt.min() >= 2 and cnt.max() <= 12


def test_small_topk_block_causal_clamp():
    """k above the condition block count clamps condition rows."""
    T, H, W = 8, 8, 16  # 8 blocks, 4 condition blocks
    q, k, v = make_qkv(T, H, W, 2, kind="iid", seed=78)
    problem = Problem.make(T, H, W, 2, cond_frames=4)
    idx, cnt, _, _ = _run_and_compare(problem, SelectParams.topk(6), q, k, v)
    cnt = cnt.reshape(2, 8)
    assert np.all(cnt[:, :4] == 4) and np.all(cnt[:, 4:] == 6)


def test_q_zero_closed_form():
    """Q = 0: all pooled scores tie, so blocks 0..k-1 are kept and every query
    averages V over their tokens."""
    T, H, W, heads, kk = 8, 16, 16, 2, 3
    _, k, v = make_qkv(T, H, W, heads, kind="iid", seed=5)
    q = np.zeros_like(k)
    problem = Problem.make(T, H, W, heads)
    qd, kd, vd = PT.to_device(q), PT.to_device(k), PT.to_device(v)
    idx_d, cnt_d = PT.run_select(problem, SelectParams.topk(kk), qd, kd)
    idx = idx_d.cpu().numpy()
    assert np.all(idx == np.arange(kk)) and np.all(cnt_d.cpu().numpy() == kk)
    out = O.bf16_bits_to_f64(PT.from_device(PT.run_attention(problem, qd, kd, vd, idx_d, cnt_d, kk)))
    g = PT.geometry(problem)
    perm = O.block_token_order(g)
    for h in range(heads):
        vv = O.bf16_bits_to_f64(v[0, h])
        mean_v = vv[perm[: kk * g.n]].mean(axis=0)
        err = np.abs(out.reshape(q.shape)[0, h] - mean_v)
        assert err.max() < 8e-3


def test_constant_v():
    """V constant: every output equals it (weights sum to one)."""
    T, H, W, heads = 8, 16, 16, 2
    q, k, _ = make_qkv(T, H, W, heads, kind="iid", seed=6)
    v = np.full_like(q, 0x3F00)  # bf16 0.5
    problem = Problem.make(T, H, W, heads)
    qd, kd, vd = PT.to_device(q), PT.to_device(k), PT.to_device(v)
    idx_d, cnt_d = PT.run_select(problem, SelectParams.topk(5), qd, kd)
    out = O.bf16_bits_to_f64(PT.from_device(PT.run_attention(problem, qd, kd, vd, idx_d, cnt_d, 5)))
    assert np.abs(out - 0.5).max() < 4e-3


def test_deterministic():
    T, H, W, heads = 8, 16, 24, 2
    q, k, v = make_qkv(T, H, W, heads, kind="field", seed=8)
    problem = Problem.make(T, H, W, heads, cond_frames=4)
    params = SelectParams.cdf(0.8, 1, 6)
    qd, kd, vd = PT.to_device(q), PT.to_device(k), PT.to_device(v)
    res = []
    for _ in range(2):
        idx_d, cnt_d = PT.run_select(problem, params, qd, kd)
        o = PT.run_attention(problem, qd, kd, vd, idx_d, cnt_d, 6)
        res.append((idx_d.cpu().numpy(), cnt_d.cpu().numpy(), PT.from_device(o)))
    for a, b in zip(res[0], res[1]):
        assert np.array_equal(a, b)


def test_block_causal_independence():
    """Condition rows' indices and outputs do not change, bit for bit, when
    every noisy token's Q, K and V is replaced."""
    T, H, W, heads = 12, 16, 16, 2
    q, k, v = make_qkv(T, H, W, heads, kind="field", seed=9)
    q2, k2, v2 = make_qkv(T, H, W, heads, kind="field", seed=10)
    cond_tokens = 4 * H * W
    for a, b in ((q2, q), (k2, k), (v2, v)):
        a[:, :, :cond_tokens] = b[:, :, :cond_tokens]
    problem = Problem.make(T, H, W, heads, cond_frames=4)
    params = SelectParams.topk(4)
    outs = []
    for qq, kk, vv in ((q, k, v), (q2, k2, v2)):
        qd, kd, vd = PT.to_device(qq), PT.to_device(kk), PT.to_device(vv)
        idx_d, cnt_d = PT.run_select(problem, params, qd, kd)
        o = PT.run_attention(problem, qd, kd, vd, idx_d, cnt_d, 4)
        outs.append((idx_d.cpu().numpy().reshape(heads, -1, 4), PT.from_device(o)))
    nb_cond = 4  # (4/4) * (16/4) * (16/8)
    assert np.array_equal(outs[0][0][:, :nb_cond], outs[1][0][:, :nb_cond])
    assert np.array_equal(outs[0][1][:, :, :cond_tokens], outs[1][1][:, :, :cond_tokens])


def test_skips_invalid_ids_and_clamps_cnt():
    """bsa_attention skips ids outside [0, Nb) and clamps cnt to the stride;
    a row with no valid block gives zeros."""
    import torch

    T, H, W, heads = 8, 8, 16, 1
    q, k, v = make_qkv(T, H, W, heads, kind="iid", seed=12)
    problem = Problem.make(T, H, W, heads)
    qd, kd, vd = PT.to_device(q), PT.to_device(k), PT.to_device(v)
    idx = torch.tensor([[0, 5, -3, 2], [99, -1, -1, -1], [1, 3, 0, 0], [7, 6, 5, 4],
                        [4, 4, 4, 4], [0, 1, 2, 3], [2, 2, 2, 2], [3, 1, 0, 2]],
                       dtype=torch.int32, device="cuda")
    cnt = torch.tensor([4, 1, 2, 9, 0, -5, 1, 4], dtype=torch.int32, device="cuda")
    out = O.bf16_bits_to_f64(PT.from_device(PT.run_attention(problem, qd, kd, vd, idx, cnt, 4)))
    g = PT.geometry(problem)
    perm = O.block_token_order(g)
    qf, kf, vf = (O.bf16_bits_to_f64(a[0, 0]) for a in (q, k, v))
    want_blocks = {0: [0, 5, 2], 2: [1, 3], 3: [7, 6, 5, 4], 6: [2], 7: [3, 1, 0, 2]}
    for i in range(g.num_blocks):
        got = out[0, 0][perm[i * g.n : (i + 1) * g.n]]
        if i in want_blocks:
            ref = O.attend_query_block(qf, kf, vf, g, i, want_blocks[i], SCALE, perm)
            assert np.abs(got - ref).max() <= PT.MAX_ABS
        else:
            assert np.all(got == 0.0)


@pytest.mark.parametrize("grid,chunk,key_chunk,params,cond", [
    ((8, 16, 32), (4, 4, 8), (2, 4, 8), SelectParams.topk(5), 0),    # 64-token keys, odd count
    ((8, 16, 32), (4, 4, 8), (2, 4, 8), SelectParams.topk(6), 0),    # 64-token keys, even count
    ((8, 16, 32), (4, 4, 8), (4, 8, 8), SelectParams.topk(3), 0),    # 256
    ((8, 16, 32), (4, 4, 8), (8, 8, 16), SelectParams.topk(2), 0),   # 1024
    ((8, 16, 32), (2, 8, 8), (4, 8, 16), SelectParams.topk(3), 0),   # 512, another query chunk
    ((8, 16, 32), (4, 4, 8), (4, 8, 8), SelectParams.cdf(0.8, 1, 6), 4),
    ((8, 16, 32), (4, 4, 8), (2, 4, 8), SelectParams.cdf(0.7, 1, 9), 4),
    # 64-token query blocks (key-half split): with 64-, 128- and 256-token keys.
    ((8, 16, 32), (2, 4, 8), None, SelectParams.topk(5), 0),
    ((8, 16, 32), (2, 4, 8), (4, 4, 8), SelectParams.topk(4), 0),
    ((8, 16, 32), (2, 4, 8), (4, 8, 8), SelectParams.topk(3), 0),
    ((8, 16, 32), (4, 2, 8), (2, 4, 8), SelectParams.cdf(0.7, 1, 7), 4),
])
def test_key_chunks(grid, chunk, key_chunk, params, cond):
    """Key blocks cut with their own chunk (64 to 1024 tokens), and query
    blocks of 64 tokens: every index row and every output against the
    oracle."""
    T, H, W = grid
    q, k, v = make_qkv(T, H, W, 2, kind="field", seed=17)
    problem = Problem.make(T, H, W, 2, chunk=chunk, cond_frames=cond, key_chunk=key_chunk)
    _run_and_compare(problem, params, q, k, v)


@pytest.mark.parametrize("cond", [4, 2])
def test_query_chunk_64_dense_and_lse(cond):
    """64-token query blocks: dense attention against the oracle's dense
    (block-causal) attention, and bsa_attention_lse: the same o as
    bsa_attention and lse against the oracle's. With an even number of
    condition t-rows the dense kernel runs on boxes of twice the chunk's
    depth; with an odd one (cond 2) on the chunk itself."""
    import torch

    from video_dit_block_bsa_amd import binding as B

    T, H, W = 8, 16, 32
    q, k, v = make_qkv(T, H, W, 2, kind="field", seed=29)
    problem = Problem.make(T, H, W, 2, chunk=(2, 4, 8), cond_frames=cond)
    g = PT.geometry(problem)
    qd, kd, vd = PT.to_device(q), PT.to_device(k), PT.to_device(v)
    o = O.bf16_bits_to_f64(PT.from_device(PT.run_dense(problem, qd, kd, vd)).reshape(q.shape))
    for h in range(2):
        ref = O.dense_head(*(O.bf16_bits_to_f64(a[0, h]) for a in (q, k, v)), g, SCALE)
        err = np.abs(o[0, h] - ref)
        _log(f"dense q64 head {h}: max-abs {err.max():.3e}, mean-abs {err.mean():.3e}")
        assert err.max() <= PT.MAX_ABS and err.mean() <= PT.MEAN_ABS
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
        assert np.abs(lse[0, h].cpu().numpy() - lse_r).max() <= 2.5e-3


@pytest.mark.parametrize("key_chunk", [(2, 4, 8), (4, 8, 8)])
def test_key_chunks_invalid_ids_and_clamps(key_chunk):
    """With 64- and 256-token key blocks: ids outside [0, Nk) are skipped, cnt
    is clamped to the stride, a lone last 64-token block is handled, and a
    row with no valid block gives zeros."""
    import torch

    T, H, W = 8, 8, 16
    q, k, v = make_qkv(T, H, W, 1, kind="iid", seed=23)
    problem = Problem.make(T, H, W, 1, key_chunk=key_chunk)
    g = PT.geometry(problem)
    nk = g.num_key_blocks
    qd, kd, vd = PT.to_device(q), PT.to_device(k), PT.to_device(v)
    rows = [[0, nk + 2, 1, nk - 1], [nk, -1, -1, -1], [1, nk - 2, 0, 0], [3, 2, 1, 0],
            [0, 0, 0, 0], [0, 1, 2, 3], [2, -7, 2, 2], [nk - 1, 1, 0, 2]]
    cnt_l = [4, 1, 3, 9, 0, -5, 3, 4]
    idx = torch.tensor([[min(x, 10**6) for x in r] for r in rows], dtype=torch.int32, device="cuda")
    cnt = torch.tensor(cnt_l, dtype=torch.int32, device="cuda")
    out = O.bf16_bits_to_f64(PT.from_device(PT.run_attention(problem, qd, kd, vd, idx, cnt, 4)))
    perm = O.block_token_order(g)
    kperm = O.block_token_order(O.key_geometry(g))
    qf, kf, vf = (O.bf16_bits_to_f64(a[0, 0]) for a in (q, k, v))
    for i in range(g.num_blocks):
        c = min(max(cnt_l[i], 0), 4)
        want = [x for x in rows[i][:c] if 0 <= x < nk]
        got = out[0, 0][perm[i * g.n:(i + 1) * g.n]]
        if want:
            ref = O.attend_query_block(qf, kf, vf, g, i, want, SCALE, perm, kperm)
            assert np.abs(got - ref).max() <= PT.MAX_ABS, (i, want)
        else:
            assert np.all(got == 0.0)


# Grids that a chunk does not divide: the pages' block counts are ceilings,
# so the last block along a cut axis holds only the tokens of its box inside
# the grid (pooled over those tokens, attended over those tokens).
@pytest.mark.parametrize("grid,chunk,key_chunk,params,cond", [
    ((6, 6, 12), (4, 4, 8), None, SelectParams.topk(3), 0),          # every axis cut, 8 blocks
    ((10, 20, 36), (4, 4, 8), None, SelectParams.topk(7), 0),
    ((10, 20, 36), (4, 4, 8), None, SelectParams.cdf(0.8, 2, 9), 4),
    ((10, 20, 36), (4, 4, 8), (2, 4, 8), SelectParams.topk(9), 0),    # 64-token keys
    ((10, 20, 36), (4, 4, 8), (4, 8, 8), SelectParams.topk(4), 0),    # 256
    ((10, 20, 36), (4, 4, 8), (8, 8, 16), SelectParams.topk(2), 0),   # 1024: whole units outside
    ((10, 20, 36), (2, 4, 8), None, SelectParams.topk(5), 0),         # 64-token queries
    ((10, 20, 36), (2, 4, 8), (4, 4, 8), SelectParams.topk(4), 4),
    ((10, 20, 36), (4, 2, 8), (2, 4, 8), SelectParams.cdf(0.7, 1, 7), 4),
    ((16, 30, 52), (4, 4, 8), None, SelectParams.topk(14), 0),        # uneven latent frame
])
def test_partial_blocks(grid, chunk, key_chunk, params, cond):
    """Partial blocks at the grid's far edge: every index row and every
    output against the oracle."""
    T, H, W = grid
    q, k, v = make_qkv(T, H, W, 2, kind="field", seed=37)
    problem = Problem.make(T, H, W, 2, chunk=chunk, cond_frames=cond, key_chunk=key_chunk)
    _run_and_compare(problem, params, q, k, v)


# Block grids one block wide (or one block per frame): the kernels divide
# block ids by nW and nH*nW, and a divisor of 1 takes its own path.
@pytest.mark.parametrize("grid,chunk,key_chunk,params,cond", [
    ((8, 4, 8), (4, 4, 8), None, SelectParams.topk(2), 0),            # nH = nW = 1
    ((9, 10, 16), (1, 8, 16), None, SelectParams.cdf(0.7, 2, 6), 0),  # nW = 1, cut along h
    ((6, 21, 32), (2, 2, 16), (1, 8, 32), SelectParams.topk(6), 2),   # key grid one block wide
    ((12, 5, 7), (4, 4, 8), (2, 4, 8), SelectParams.topk(3), 4),      # cut to one block per frame
])
def test_one_block_wide_grids(grid, chunk, key_chunk, params, cond):
    T, H, W = grid
    q, k, v = make_qkv(T, H, W, 2, kind="iid", seed=71)
    problem = Problem.make(T, H, W, 2, chunk=chunk, cond_frames=cond, key_chunk=key_chunk)
    _run_and_compare(problem, params, q, k, v)
    dense = PT.from_device(PT.run_dense(problem, *(PT.to_device(a) for a in (q, k, v))))
    g = PT.geometry(problem)
    for h in range(2):
        ref = O.dense_head(*(O.bf16_bits_to_f64(a[0, h]) for a in (q, k, v)), g, SCALE)
        err = np.abs(O.bf16_bits_to_f64(dense.reshape(q.shape)[0, h]) - ref)
        assert err.max() <= PT.MAX_ABS and err.mean() <= PT.MEAN_ABS


@pytest.mark.parametrize("chunk", [(4, 4, 8), (2, 4, 8)])
def test_partial_blocks_dense_and_lse(chunk):
    """Partial grid with condition frames: dense attention against the
    oracle's dense (block-causal) attention; bsa_attention_lse writes the same
    o as bsa_attention and an lse within 2.5e-3 of the oracle's for every
    token."""
    import torch

    from video_dit_block_bsa_amd import binding as B

    T, H, W = 10, 20, 36
    q, k, v = make_qkv(T, H, W, 2, kind="field", seed=41)
    problem = Problem.make(T, H, W, 2, chunk=chunk, cond_frames=4)
    g = PT.geometry(problem)
    qd, kd, vd = PT.to_device(q), PT.to_device(k), PT.to_device(v)
    o = O.bf16_bits_to_f64(PT.from_device(PT.run_dense(problem, qd, kd, vd)).reshape(q.shape))
    for h in range(2):
        ref = O.dense_head(*(O.bf16_bits_to_f64(a[0, h]) for a in (q, k, v)), g, SCALE)
        err = np.abs(o[0, h] - ref)
        _log(f"dense partial {chunk} head {h}: max-abs {err.max():.3e}, mean-abs {err.mean():.3e}")
        assert err.max() <= PT.MAX_ABS and err.mean() <= PT.MEAN_ABS
    params = SelectParams.topk(6)
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
        got = lse[0, h].cpu().numpy()
        assert np.isfinite(got).all()
        assert np.abs(got - lse_r).max() <= 2.5e-3


def test_longest_sequence_sampled():
    """The longest sequence the boundary accepts (T*H*W < 2^24):
    255 x 256 x 256 = 16,711,680 tokens, one head, so a head's K or V spans
    4.28 GB and the tile loads' 32-bit byte offsets come within 17 MB of
    2^32; the last row of blocks along t is partial (3 of 4 frames). Random
    lists of 3 key blocks per query block (the last query block keeps the
    last three key blocks, which sit at the top of the address range);
    sampled query blocks against the oracle."""
    import torch

    from video_dit_block_bsa_amd.inputs import uniform_block_lists

    T, H, W = 255, 256, 256
    problem = Problem.make(T, H, W, 1)
    g = PT.geometry(problem)
    nb = g.num_blocks
    assert nb == 64 * 64 * 32 and g.seq_len < (1 << 24)
    _log(f"generating {T}x{H}x{W} ({g.seq_len} tokens), one head")
    q, k, v = make_qkv(T, H, W, 1, kind="iid", seed=61)
    idx, cnt = uniform_block_lists(nb, nb, 3, seed=62)
    idx[nb - 1] = [nb - 3, nb - 2, nb - 1]
    idx[0] = [0, nb // 2, nb - 1]
    qd, kd, vd = PT.to_device(q), PT.to_device(k), PT.to_device(v)
    out = PT.from_device(PT.run_attention(problem, qd, kd, vd, torch.from_numpy(idx).cuda(),
                                          torch.from_numpy(cnt).cuda(), 3))
    del qd, kd, vd
    rng = np.random.default_rng(63)
    sample = sorted({0, 1, nb // 2, nb - 33, nb - 2, nb - 1} |
                    set(rng.choice(nb, size=6, replace=False).tolist()))
    perm = O.block_token_order(g)
    worst = 0.0
    for i in sample:
        blocks = [int(x) for x in idx[i]]
        # Widen only the rows this query block touches; the oracle reads them
        # through a block order remapped onto the widened rows.
        need = [i] + blocks
        sub_perm = np.full_like(perm, -1)
        pos = 0
        for b in dict.fromkeys(need):
            t_b = O.block_tokens(perm, b, g.n)
            slots = np.nonzero(perm[b * g.n:(b + 1) * g.n] >= 0)[0] + b * g.n
            sub_perm[slots] = np.arange(pos, pos + t_b.size)
            pos += t_b.size
        uniq = np.concatenate([O.block_tokens(perm, b, g.n) for b in dict.fromkeys(need)])
        qs, ks, vs = (O.bf16_bits_to_f64(a[0, 0][uniq]) for a in (q, k, v))
        ref = O.attend_query_block(qs, ks, vs, g, i, blocks, SCALE, sub_perm, sub_perm)
        got = O.bf16_bits_to_f64(out.reshape(q.shape)[0, 0][O.block_tokens(perm, i, g.n)])
        err = np.abs(got - ref)
        assert np.isfinite(got).all()
        worst = max(worst, err.max())
        assert err.max() <= PT.MAX_ABS and err.mean() <= PT.MEAN_ABS, (i, blocks)
    _log(f"longest sequence: {len(sample)} sampled query blocks, max-abs {worst:.3e}")


@pytest.mark.parametrize("name", ["480p", "720p", "long", "vc", "long_k64", "long_k256", "long_q64"])
def test_full_size_workload(name):
    """Full-size workloads in the configuration the benchmark times: every
    index row against the oracle, outputs on a seeded sample."""
    w = WORKLOADS[name]
    _log(f"generating {name}: {w.T}x{w.H}x{w.W}, {w.heads} heads")
    q, k, v = make_qkv(w.T, w.H, w.W, w.heads, kind=w.kind, seed=w.seed)
    _, cnt, _, _ = _run_and_compare(Problem.from_workload(w), SelectParams.from_workload(w),
                                    q, k, v, all_outputs=False, sample=(4, 10), seed=w.seed)
    if w.mode == "cdf":
        _log(f"CDF counts: min {cnt.min()}, mean {cnt.mean():.2f}, max {cnt.max()}")
        assert cnt.min() >= w.k_min and cnt.max() <= w.k_max


@pytest.mark.parametrize("params,cond", [(SelectParams.topk(352), 0),
                                          (SelectParams.cdf(0.9, 4, 64), 4)])
def test_more_than_4096_key_blocks(params, cond):
    """The pages' 720p x 93-frame token count (93 x 45 x 80 = 334,800 tokens;
    deep dive, "VAE, Text Encoder, and Token Spaces") cut into 128-token query blocks and
    64-token key blocks: 2,880 query blocks, 5,640 key blocks (the last t- and
    h-rows partial), more than a row's scores fit in registers, so the
    selection searches them in LDS. Top-k at the pages' ratio r = N_k/16, and
    CDF with condition frames. Every index row against the oracle, outputs
    on a sample."""
    T, H, W = 93, 45, 80
    problem = Problem.make(T, H, W, 2, key_chunk=(2, 4, 8), cond_frames=cond)
    assert problem.num_key_blocks == 5640 and problem.num_blocks == 2880
    q, k, v = make_qkv(T, H, W, 2, kind="field", seed=91)
    _, cnt, _, _ = _run_and_compare(problem, params, q, k, v, all_outputs=False, sample=(2, 6),
                                    seed=92)
    _log(f"counts: min {cnt.min()}, mean {cnt.mean():.2f}, max {cnt.max()}")


def test_dense_720p_sampled():
    """Dense baseline at 720p x 93f on sampled query blocks."""
    w = WORKLOADS["720p"]
    q, k, v = make_qkv(w.T, w.H, w.W, w.heads, kind=w.kind, seed=w.seed, head_subset=[0, 17])
    problem = Problem.make(w.T, w.H, w.W, 2)
    o = PT.from_device(PT.run_dense(problem, PT.to_device(q), PT.to_device(k), PT.to_device(v)))
    g = PT.geometry(problem)
    items = [(p, i) for p in range(2) for i in (0, 1, 359, 719)]
    mx, mean, _ = PT.compare_outputs(o.reshape(q.shape), q, k, v, g,
                                     lambda p, i: range(g.num_blocks), SCALE, items)
    _log(f"dense 720p: max-abs {mx:.3e}, mean-abs {mean:.3e}")
    assert mx <= PT.MAX_ABS and mean <= PT.MEAN_ABS


@pytest.mark.parametrize("batch,heads,H", [(1, 1040, 16), (3, 347, 16), (1, 160, 28), (3, 53, 28)])
@pytest.mark.parametrize("with_lse", [False, True])
def test_many_heads_launch_groups(batch, heads, H, with_lse):
    """A sparse call of more than 7,680 query-block workgroups goes out as
    launches of 7,680 workgroups, numbered across the launches: every (batch,
    head) pair's output (and lse) is bit-identical to the same head computed
    in a small single-launch problem. The pairs are copies of 16 seeded
    heads, pair p a copy of base head p % 16, so a range offset that lands on
    the wrong head shows. With 32 query blocks per head the ranges start at
    head boundaries (33,280 and 33,312 workgroups: five launches); with 56
    they start inside a head (7,680 = 137 x 56 + 8)."""
    import torch

    from video_dit_block_bsa_amd import binding as B

    T, W, base = 8, 32, 16
    bh = batch * heads
    copies = -(-bh // base)
    q, k, v = make_qkv(T, H, W, base, kind="field", seed=21)
    qb, kb, vb = PT.to_device(q), PT.to_device(k), PT.to_device(v)
    small = Problem.make(T, H, W, base)
    params = SelectParams.topk(5)
    stride = B.index_stride(small, params)
    idx_s, cnt_s = PT.run_select(small, params, qb, kb)
    big = Problem.make(T, H, W, heads, batch=batch)
    nq8 = -(-big.num_blocks // 8) * 8
    assert base * nq8 <= 7680 < bh * nq8
    assert H == 16 or 7680 % nq8 != 0
    qd, kd, vd = (t.repeat(1, copies, 1, 1)[:, :bh].reshape(batch, heads, -1, 128).contiguous()
                  for t in (qb, kb, vb))
    idx_b, cnt_b = PT.run_select(big, params, qd, kd)
    per = big.num_blocks * stride
    assert torch.equal(idx_b.view(-1)[: bh * per].view(bh, per),
                       idx_s.view(base, per).repeat(copies, 1)[:bh])
    assert torch.equal(cnt_b.view(bh, -1), cnt_s.view(base, -1).repeat(copies, 1)[:bh])

    def attend(problem, qq, kk, vv, idx, cnt):
        o = torch.full_like(qq, float("nan"))
        ws = torch.empty(max(B.attention_workspace_bytes(problem), 1), dtype=torch.uint8,
                         device="cuda")
        if not with_lse:
            B.bsa_attention(problem, qq, kk, vv, idx, cnt, stride, o, ws)
            torch.cuda.synchronize()
            return o, None
        lse = torch.full(qq.shape[:3], float("nan"), dtype=torch.float32, device="cuda")
        B.bsa_attention_lse(problem, qq, kk, vv, idx, cnt, stride, o, lse, ws)
        torch.cuda.synchronize()
        return o, lse

    o_s, l_s = attend(small, qb, kb, vb, idx_s, cnt_s)
    o_b, l_b = attend(big, qd, kd, vd, idx_b, cnt_b)
    want = o_s.view(torch.int16).view(base, -1).repeat(copies, 1)[:bh]
    assert torch.equal(o_b.view(torch.int16).view(bh, -1), want)
    if with_lse:
        assert torch.equal(l_b.view(bh, -1), l_s.view(base, -1).repeat(copies, 1)[:bh])


@pytest.mark.parametrize("kind", ["dense", "paired_q64"])
def test_many_heads_dense_and_paired_blocks(kind):
    """1,041 (batch, head) pairs (3 x 347, copies of 16 seeded heads) give
    every pair's output bit-identical to its base head's in a 16-head
    single-launch problem, for the two other launch splits: dense calls of
    more than 32,768 workgroups go out as 130 launches of 8 pairs and a last
    one of one pair; paired 64-token query blocks (one workgroup per
    t-adjacent pair, 33,312 workgroups) as five launches of up to 7,680."""
    import torch

    from video_dit_block_bsa_amd import binding as B

    T, H, W, base, batch, heads = 8, 16, 32, 16, 3, 347
    chunk = (4, 4, 8) if kind == "dense" else (2, 4, 8)
    bh = batch * heads
    copies = -(-bh // base)
    q, k, v = make_qkv(T, H, W, base, kind="field", seed=23)
    qb, kb, vb = PT.to_device(q), PT.to_device(k), PT.to_device(v)
    small = Problem.make(T, H, W, base, chunk=chunk, key_chunk=(4, 4, 8))
    big = Problem.make(T, H, W, heads, batch=batch, chunk=chunk, key_chunk=(4, 4, 8))
    assert bh * big.num_blocks > 32768 and bh % 8 == 1
    qd, kd, vd = (t.repeat(1, copies, 1, 1)[:, :bh].reshape(batch, heads, -1, 128).contiguous()
                  for t in (qb, kb, vb))
    if kind == "dense":
        o_s = PT.run_dense(small, qb, kb, vb)
        o_b = PT.run_dense(big, qd, kd, vd)
    else:
        params = SelectParams.topk(5)
        stride = B.index_stride(small, params)
        idx_s, cnt_s = PT.run_select(small, params, qb, kb)
        idx_b, cnt_b = PT.run_select(big, params, qd, kd)
        o_s = PT.run_attention(small, qb, kb, vb, idx_s, cnt_s, stride)
        o_b = PT.run_attention(big, qd, kd, vd, idx_b, cnt_b, stride)
    want = o_s.view(torch.int16).view(base, -1).repeat(copies, 1)[:bh]
    assert torch.equal(o_b.view(torch.int16).view(bh, -1), want)
