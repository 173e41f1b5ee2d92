"""GPU parity of the backward pass (bsa_attention_lse + bsa_attention_bwd,
through the C ABI) against the float64 oracle (forward_lse_head,
backward_head).

Selections are inputs here: they come from the oracle's own selection
(select_head) or from seeded random lists, never from the GPU.

Tolerances. Every gradient element is an fp32 sum of products of bf16
operands: P and dS are rounded to bf16 before their products (relative error
up to 2^-9 = 0.2% each; the dK/dV kernel also forms dS from the bf16 P) and
the result is rounded to bf16 (2^-9). dK and dV stay at that level (measured
up to 0.3% mean, 0.8% max):
  max |gpu - oracle| <= 1.5e-2 * max |oracle|,  mean <= 5e-3 * mean |oracle|.
dQ carries one more error: D = rowsum(dO * O) is formed from the forward's
bf16 O (relative error 2^-9 per element). dS = P (dP - D) cancels where the
softmax is peaked (dP - D is small next to D), and dQ = s dS K inherits the
absolute error s P dD K, which is a larger fraction of a smaller dQ. On the
smooth-field inputs this doubles to triples the relative error (measured up
to 0.6% mean, 2.2% max), and more where blocks are small and the softmax
sharper: on the 6 x 6 x 12 grid (partial blocks of 16 to 64 tokens) the
numpy model of exactly these roundings in tests/bf16_error_model.py (bf16 P,
dS, O and dQ, fp64 otherwise) gives 1.04-1.08% mean and 2.7% max against the
float64 oracle; tests/test_tolerance_model.py derives the bound below from
it on the CPU. dQ takes
  max <= 4e-2 * max |oracle|,  mean <= 1.5e-2 * mean |oracle|.
lse: |gpu - oracle| <= 2.5e-3. The forward sums bf16-rounded probabilities,
each within a relative 2^-9, so the sum and its log are off by at most
log(1 + 2^-9) = 1.95e-3, plus fp32 rounding of the scores.
"""

from __future__ import annotations

import math

import numpy as np
import pytest

import oracle.bsa_oracle as O
import parity as PT
from video_dit_block_bsa_amd import WORKLOADS
from video_dit_block_bsa_amd.binding import Problem, SelectParams
from video_dit_block_bsa_amd.inputs import make_grad, make_qkv, random_block_lists

pytestmark = pytest.mark.gpu

SCALE = 1.0 / math.sqrt(128)
TOL = {"dq": (4e-2, 1.5e-2), "dk": (1.5e-2, 5e-3), "dv": (1.5e-2, 5e-3)}  # (max, mean) relative
LSE_ABS = 2.5e-3


def _log(*a):
    print(*a, flush=True)


def run_backward(problem, q, k, v, do, idx, cnt, stride):
    """Forward with lse, then the backward, on the GPU. Inputs are numpy
    (bf16 bits / int32). Returns numpy (o, o_plain, lse, dq, dk, dv)."""
    import torch

    from video_dit_block_bsa_amd import binding as B

    qd, kd, vd, dod = (PT.to_device(a) for a in (q, k, v, do))
    idx_d = torch.from_numpy(np.ascontiguousarray(idx, dtype=np.int32)).cuda()
    cnt_d = torch.from_numpy(np.ascontiguousarray(cnt, dtype=np.int32)).cuda()
    o = torch.full_like(qd, float("nan"))
    lse = torch.full(q.shape[:3], float("nan"), dtype=torch.float32, device="cuda")
    ws = torch.empty(max(B.attention_workspace_bytes(problem), 1), dtype=torch.uint8, device="cuda")
    B.bsa_attention_lse(problem, qd, kd, vd, idx_d, cnt_d, stride, o, lse, ws)
    o_plain = PT.run_attention(problem, qd, kd, vd, idx_d, cnt_d, stride)
    grads = [torch.full_like(qd, float("nan")) for _ in range(3)]
    wsb = torch.full((max(B.attention_bwd_workspace_bytes(problem), 16),), 0x5A, dtype=torch.uint8,
                     device="cuda")
    B.bsa_attention_bwd(problem, qd, kd, vd, o, dod, lse, idx_d, cnt_d, stride, *grads, wsb)
    torch.cuda.synchronize()
    return (PT.from_device(o).reshape(q.shape), PT.from_device(o_plain).reshape(q.shape),
            lse.cpu().numpy(), *(PT.from_device(t).reshape(q.shape) for t in grads))


def clean_lists(idx, cnt, nbk, stride):
    """The valid ids of each row (the forward skips ids outside [0, nbk), nbk
    the number of key blocks, and clamps cnt to [0, stride])."""
    out = []
    for r in range(idx.shape[0]):
        c = min(max(int(cnt[r]), 0), stride)
        out.append([int(x) for x in idx[r, :c] if 0 <= x < nbk])
    return out


def oracle_pair(q, k, v, do, g, lists, b, h, query_blocks=None):
    nb = g.num_blocks
    Hh = q.shape[1]
    rows = lists[(b * Hh + h) * nb:(b * Hh + h + 1) * nb]
    stride = max(1, max(len(r) for r in rows))
    idx = np.full((nb, stride), -1, dtype=np.int64)
    cnt = np.zeros(nb, dtype=np.int64)
    for i, r in enumerate(rows):
        idx[i, :len(r)] = r
        cnt[i] = len(r)
    qf, kf, vf, dof = (O.bf16_bits_to_f64(a[b, h]) for a in (q, k, v, do))
    out, lse = O.forward_lse_head(qf, kf, vf, g, idx, cnt, SCALE)
    dq, dk, dv = O.backward_head(qf, kf, vf, dof, g, idx, cnt, SCALE, query_blocks=query_blocks)
    return out, lse, dq, dk, dv


def check_close(name, got_bits, ref):
    got = O.bf16_bits_to_f64(got_bits)
    assert np.isfinite(got).all(), f"{name}: non-finite values"
    err = np.abs(got - ref)
    mx, mean = err.max(), err.mean()
    ref_max, ref_mean = np.abs(ref).max(), np.abs(ref).mean()
    _log(f"{name}: max-abs {mx:.3e} (ref max {ref_max:.3e}), mean-abs {mean:.3e} "
         f"(ref mean {ref_mean:.3e}); ratios {mx / ref_max:.4f} {mean / ref_mean:.4f}")
    max_rel, mean_rel = TOL[name.split()[0]]
    assert mx <= max_rel * ref_max + 1e-6, name
    assert mean <= mean_rel * ref_mean + 1e-7, name


def compare_all(problem, q, k, v, do, idx, cnt, stride):
    g = PT.geometry(problem)
    nb = g.num_blocks
    o, o_plain, lse, dq, dk, dv = run_backward(problem, q, k, v, do, idx, cnt, stride)
    assert np.array_equal(o, o_plain), "bsa_attention_lse changed o"
    lists = clean_lists(idx, cnt, g.num_key_blocks, stride)
    for b in range(q.shape[0]):
        for h in range(q.shape[1]):
            out_r, lse_r, dq_r, dk_r, dv_r = oracle_pair(q, k, v, do, g, lists, b, h)
            fin = np.isfinite(lse_r)
            assert np.array_equal(np.isfinite(lse[b, h]), fin)
            assert np.all(lse[b, h][~fin] == -np.inf)
            if fin.any():
                e = np.abs(lse[b, h][fin] - lse_r[fin]).max()
                _log(f"lse ({b},{h}): max-abs {e:.3e}")
                assert e <= LSE_ABS
            for name, got, ref in (("dq", dq, dq_r), ("dk", dk, dk_r), ("dv", dv, dv_r)):
                if np.abs(ref).max() == 0:
                    assert np.all(O.bf16_bits_to_f64(got[b, h]) == 0), name
                else:
                    check_close(f"{name} ({b},{h})", got[b, h], ref)
    return dq, dk, dv


def oracle_selection(problem, params, q, k):
    g = PT.geometry(problem)
    sp = PT.oracle_params(params)
    stride = O.index_stride(sp)
    rows = PT.oracle_select_all(q, k, g, sp, SCALE)
    idx = np.concatenate([r[0] for r in rows]).astype(np.int32)
    cnt = np.concatenate([r[1] for r in rows]).astype(np.int32)
    return idx.reshape(-1, stride), cnt.reshape(-1), stride


def _case(T, H, W, heads, k_sel, batch=1, chunk=(4, 4, 8), kind="iid", seed=0, cond_frames=0,
          params=None, key_chunk=None):
    problem = Problem.make(T, H, W, heads, batch=batch, chunk=chunk, cond_frames=cond_frames,
                           key_chunk=key_chunk)
    params = params or SelectParams.topk(k_sel)
    q, k, v = make_qkv(T, H, W, heads, batch=batch, kind=kind, seed=seed)
    do = make_grad(T, H, W, heads, batch=batch, seed=seed)
    idx, cnt, stride = oracle_selection(problem, params, q, k)
    _log(f"case {T}x{H}x{W} chunk {chunk} batch {batch} heads {heads}: "
         f"{int(cnt.sum())} kept pairs")
    return compare_all(problem, q, k, v, do, idx, cnt, stride)


def test_tiny_topk2():
    w = WORKLOADS["tiny"]
    _case(w.T, w.H, w.W, w.heads, 2, kind=w.kind, seed=w.seed)


def test_tiny_all_blocks():
    w = WORKLOADS["tiny"]
    _case(w.T, w.H, w.W, w.heads, 4, kind=w.kind, seed=w.seed)


@pytest.mark.parametrize("kind", ["iid", "field"])
def test_small_topk(kind):
    _case(8, 16, 32, 2, 6, kind=kind, seed=11)


@pytest.mark.parametrize("chunk,grid", [((2, 8, 8), (4, 16, 16)), ((8, 4, 4), (16, 8, 8)),
                                        ((1, 8, 16), (2, 16, 32)), ((1, 1, 128), (2, 2, 256))])
def test_other_chunk_shapes(chunk, grid):
    _case(*grid, 1, 3, chunk=chunk, seed=5)


def test_batch_two_three_heads():
    _case(8, 16, 16, 3, 4, batch=2, kind="field", seed=9)


def test_block_causal_cdf():
    _case(16, 16, 16, 2, 0, kind="field", seed=13, cond_frames=4,
          params=SelectParams.cdf(0.9, 2, 12))


@pytest.mark.parametrize("key_chunk,k_sel,cond", [((4, 8, 8), 3, 0), ((8, 8, 16), 2, 0),
                                                  ((4, 8, 8), 4, 4)])
def test_key_chunks(key_chunk, k_sel, cond):
    """Key blocks of 256 and 1024 tokens (walked in 128-key units by dQ, one
    dK/dV workgroup per unit), with and without condition frames."""
    _case(8, 16, 32, 2, k_sel, kind="field", seed=19, cond_frames=cond, key_chunk=key_chunk)


@pytest.mark.parametrize("grid,key_chunk,k_sel,cond", [
    ((6, 6, 12), None, 3, 0),             # every axis cut, 8 blocks
    ((10, 20, 36), None, 6, 4),
    ((10, 20, 36), (4, 8, 8), 4, 0),      # 256-token keys cut along h and w
    ((10, 20, 36), (8, 8, 16), 2, 0),     # 1024: units wholly outside the grid
])
def test_partial_blocks(grid, key_chunk, k_sel, cond):
    """Partial blocks at the grid's far edge: every gradient element against
    the oracle (slots outside the grid take no part, in queries or keys)."""
    _case(*grid, 2, k_sel, kind="field", seed=43, cond_frames=cond, key_chunk=key_chunk)


@pytest.mark.parametrize("grid,chunk,key_chunk,k_sel,cond", [
    ((8, 16, 32), (4, 4, 8), (2, 4, 8), 5, 0),     # 64-token keys, odd counts
    ((8, 16, 32), (4, 4, 8), (2, 4, 8), 6, 4),     # even counts, condition frames
    ((8, 16, 32), (2, 4, 8), None, 5, 0),          # 64-token queries and keys
    ((8, 16, 32), (2, 4, 8), (4, 4, 8), 4, 4),     # 64-token queries, 128-token keys
    ((8, 16, 32), (4, 2, 8), (4, 8, 8), 3, 0),     # 64-token queries, 256-token keys
    ((6, 12, 24), (2, 4, 8), (2, 4, 8), 4, 0),     # odd block counts, partial blocks
])
def test_64_token_blocks(grid, chunk, key_chunk, k_sel, cond):
    """Query blocks of 64 tokens (dQ: four key parts per query slice; dK/dV:
    two query blocks per step) and key blocks of 64 tokens (two per dQ unit
    and per dK/dV workgroup), every gradient element against the oracle."""
    _case(*grid, 2, k_sel, chunk=chunk, kind="field", seed=47, cond_frames=cond,
          key_chunk=key_chunk)


@pytest.mark.parametrize("grid,chunk,key_chunk,k_sel,cond", [
    ((8, 4, 8), (4, 4, 8), None, 2, 0),          # nH = nW = 1
    ((9, 10, 16), (1, 8, 16), None, 3, 0),       # nW = 1, cut along h
    ((6, 21, 32), (2, 2, 16), (1, 8, 32), 4, 2), # key grid one block wide
])
def test_one_block_wide_grids(grid, chunk, key_chunk, k_sel, cond):
    """Block grids one block wide: block ids divided by 1 take their own path."""
    _case(*grid, 2, k_sel, chunk=chunk, seed=73, cond_frames=cond, key_chunk=key_chunk)


def test_many_blocks_one_key_block_popular():
    """One key block kept by every query block (long mask rows) and rows of
    different lengths."""
    T, H, W = 16, 32, 32  # 128 blocks
    problem = Problem.make(T, H, W, 1)
    nb = problem.num_blocks
    q, k, v = make_qkv(T, H, W, 1, kind="iid", seed=21)
    do = make_grad(T, H, W, 1, seed=21)
    stride = 9
    counts = np.random.default_rng(4).integers(1, stride, size=nb)
    idx, cnt = random_block_lists([nb] * nb, stride, counts, seed=22)
    for r in range(nb):  # put key block 37 in every row
        row = [x for x in idx[r, :cnt[r]] if x != 37][: stride - 1] + [37]
        row.sort()
        idx[r, :] = -1
        idx[r, :len(row)] = row
        cnt[r] = len(row)
    compare_all(problem, q, k, v, do, idx, cnt, stride)


def test_invalid_ids_empty_rows_and_clamped_counts():
    """Ids outside [0, nb) are skipped, cnt is clamped to [0, stride], rows
    with no key block give zero dq and never touch dk, dv."""
    T, H, W = 8, 16, 32  # 32 blocks
    problem = Problem.make(T, H, W, 2)
    nb = problem.num_blocks
    q, k, v = make_qkv(T, H, W, 2, kind="iid", seed=31)
    do = make_grad(T, H, W, 2, seed=31)
    stride = 6
    rng = np.random.default_rng(32)
    idx, cnt = random_block_lists([nb] * (2 * nb), stride, rng.integers(0, stride + 1, size=2 * nb),
                                  seed=33)
    for r in range(nb):      # key blocks 1 and 2 of head 0: kept by no query block
        row = [x for x in idx[r, :cnt[r]] if x not in (1, 2)]
        idx[r, :] = -1
        idx[r, :len(row)] = row
        cnt[r] = len(row)
    idx[3, :] = -1
    idx[3, :3] = [nb + 5, 4, 9]  # out of range: skipped
    cnt[3] = 3
    idx[4, :] = -1
    idx[4, :3] = [0, -3, 12]     # negative: skipped
    cnt[4] = 3
    idx[5, :] = -1
    idx[5, :2] = [3, 5]
    cnt[5] = stride + 7          # clamped to stride; the trailing -1 entries are skipped
    cnt[6] = -2                  # clamped to 0: empty row
    cnt[7] = 0
    dq, dk, dv = compare_all(problem, q, k, v, do, idx, cnt, stride)
    g = PT.geometry(problem)
    perm = O.block_token_order(g)
    for blk in (6, 7):
        assert np.all(dq[0, 0][perm[blk * 128:(blk + 1) * 128]] == 0)
    for kb in (1, 2):
        assert np.all(dk[0, 0][perm[kb * 128:(kb + 1) * 128]] == 0)
        assert np.all(dv[0, 0][perm[kb * 128:(kb + 1) * 128]] == 0)


def test_deterministic():
    T, H, W = 8, 16, 32
    problem = Problem.make(T, H, W, 2)
    q, k, v = make_qkv(T, H, W, 2, kind="field", seed=41)
    do = make_grad(T, H, W, 2, seed=41)
    idx, cnt, stride = oracle_selection(problem, SelectParams.topk(8), q, k)
    a = run_backward(problem, q, k, v, do, idx, cnt, stride)
    b = run_backward(problem, q, k, v, do, idx, cnt, stride)
    for x, y in zip(a[3:], b[3:]):
        assert np.array_equal(x, y)


@pytest.mark.timeout(600)
@pytest.mark.parametrize("name", ["long", "long_q64", "long_k64", "long_k256", "vc"])
def test_full_size_sampled(name):
    """Full-size workloads, 32 heads (the configurations the benchmark times:
    215,040 tokens with 128-token blocks, 64-token query blocks taken in pairs
    by dQ, 64- and 256-token key blocks; 61,440 tokens with condition frames
    and CDF selection). The backward runs on every head; the oracle checks dq
    of sampled query blocks and dk, dv of sampled key blocks (visiting every
    query block that kept them) on two heads. The selection is the oracle's
    own."""
    import torch

    w = WORKLOADS[name]
    _log(f"generating {name}: {w.T}x{w.H}x{w.W}, {w.heads} heads")
    q, k, v = make_qkv(w.T, w.H, w.W, w.heads, kind=w.kind, seed=w.seed)
    do = make_grad(w.T, w.H, w.W, w.heads, seed=w.seed)
    problem = Problem.from_workload(w)
    params = SelectParams.from_workload(w)
    g = PT.geometry(problem)
    kg = O.key_geometry(g)
    nb, nbk = g.num_blocks, kg.num_blocks
    heads = [0, 19]
    sp = PT.oracle_params(params)
    stride = O.index_stride(sp)
    # The oracle selection for the sampled heads; the other heads take the
    # GPU's own selection (their outputs are not compared, only run).
    qd, kd = PT.to_device(q), PT.to_device(k)
    idx_d, cnt_d = PT.run_select(problem, params, qd, kd)
    idx = idx_d.cpu().numpy()
    cnt = cnt_d.cpu().numpy()
    del qd, kd, idx_d, cnt_d
    torch.cuda.empty_cache()
    rows = {}
    for h in heads:
        oi, oc, _ = O.select_head(O.bf16_bits_to_f64(q[0, h]), O.bf16_bits_to_f64(k[0, h]), g, sp,
                                  SCALE)
        idx[h * nb:(h + 1) * nb] = oi
        cnt[h * nb:(h + 1) * nb] = oc
        rows[h] = (oi, oc)
    _log("running forward + backward on the GPU")
    o, o_plain, lse, dq, dk, dv = run_backward(problem, q, k, v, do, idx, cnt, stride)
    assert np.array_equal(o, o_plain)
    perm = O.block_token_order(g)
    kperm = O.block_token_order(kg)
    rng = np.random.default_rng(7)
    for h in heads:
        oi, oc = rows[h]
        qbs = sorted(set(rng.choice(nb, size=2, replace=False).tolist()) | {0, nb - 1})
        kbs = sorted(rng.choice(nbk, size=2, replace=False).tolist())
        keepers = sorted({i for i in range(nb) for kb in kbs if kb in set(oi[i, :oc[i]].tolist())})
        _log(f"head {h}: query blocks {qbs}, key blocks {kbs} kept by {len(keepers)} query blocks")
        qf, kf, vf, dof = (O.bf16_bits_to_f64(a[0, h]) for a in (q, k, v, do))
        _, lse_r = O.forward_lse_head(qf, kf, vf, g, oi, oc, SCALE, query_blocks=qbs)
        dq_r, dk_r, dv_r = O.backward_head(qf, kf, vf, dof, g, oi, oc, SCALE,
                                           query_blocks=sorted(set(qbs) | set(keepers)))
        for i in qbs:
            tok = O.block_tokens(perm, i, g.n)
            assert np.abs(lse[0, h][tok] - lse_r[tok]).max() <= LSE_ABS
            check_close(f"dq head {h} block {i}", dq[0, h][tok], dq_r[tok])
        for kb in kbs:
            tok = O.block_tokens(kperm, kb, kg.n)
            if not any(kb in set(oi[i, :oc[i]].tolist()) for i in range(nb)):
                assert np.all(dk[0, h][tok] == 0) and np.all(dv[0, h][tok] == 0)
                continue
            check_close(f"dk head {h} block {kb}", dk[0, h][tok], dk_r[tok])
            check_close(f"dv head {h} block {kb}", dv[0, h][tok], dv_r[tok])
    for a in (dq, dk, dv):
        assert np.isfinite(O.bf16_bits_to_f64(a[:, :: 7])).all()
