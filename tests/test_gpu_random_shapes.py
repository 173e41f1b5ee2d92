"""Seeded sweep over random problem shapes (GPU against the oracle).

Each case draws a latent grid (often one that the chunks do not divide), a
query chunk of 64 or 128 tokens, a key chunk of 64 to 1024 tokens or none,
condition frames, batch and heads, and a top-k or CDF rule. The forward is
checked on every index row and every output (the rules of the parity tests),
and the dense baseline on every output; the backward, on the oracle's own
selection, on every gradient element (the tolerances of the backward tests).
Inputs are i.i.d. N(0, 1).
"""

from __future__ import annotations

import math

import numpy as np
import pytest

import oracle.bsa_oracle as O
import parity as PT
from test_gpu_backward import compare_all, oracle_selection
from test_gpu_parity import _run_and_compare
from video_dit_block_bsa_amd.binding import Problem, SelectParams
from video_dit_block_bsa_amd.inputs import make_grad, make_qkv

pytestmark = pytest.mark.gpu

SCALE = 1.0 / math.sqrt(128)

QUERY_CHUNKS = [(4, 4, 8), (2, 4, 8), (4, 2, 8), (2, 8, 8), (8, 4, 4), (1, 8, 16), (4, 8, 4), (2, 2, 16)]
KEY_CHUNKS = [None, None, (2, 4, 8), (4, 4, 8), (4, 8, 8), (2, 8, 16), (8, 8, 16), (1, 8, 32)]


def _case(seed):
    rng = np.random.default_rng(1000 + seed)
    chunk = QUERY_CHUNKS[rng.integers(len(QUERY_CHUNKS))]
    key_chunk = KEY_CHUNKS[rng.integers(len(KEY_CHUNKS))]
    kc = key_chunk or chunk
    T = int(rng.integers(2, 13))
    H = int(rng.integers(4, 25))
    W = int(rng.integers(8, 41))
    if T * H * W > 6000:
        W = max(8, 6000 // (T * H))
    step = math.lcm(chunk[0], kc[0])
    cond = step * int(rng.integers(0, 2)) if T > step else 0
    problem = Problem.make(T, H, W, int(rng.integers(1, 3)), batch=int(rng.integers(1, 3)),
                           chunk=chunk, cond_frames=cond, key_chunk=key_chunk)
    nk = problem.num_key_blocks
    if rng.random() < 0.6:
        params = SelectParams.topk(int(rng.integers(1, max(2, nk // 2))))
    else:
        kmin = int(rng.integers(1, 4))
        params = SelectParams.cdf(float(rng.uniform(0.3, 0.95)), kmin, kmin + int(rng.integers(0, 8)))
    return problem, params


@pytest.mark.parametrize("seed", range(24))
def test_forward_random_shape(seed):
    problem, params = _case(seed)
    print(f"case {seed}: grid {problem.T}x{problem.H}x{problem.W}, chunk "
          f"({problem.ct},{problem.ch},{problem.cw}), key chunk {problem.key_chunk}, cond "
          f"{problem.cond_frames}, batch {problem.batch}, heads {problem.heads}, mode {params.mode} "
          f"k {params.k}", flush=True)
    q, k, v = make_qkv(problem.T, problem.H, problem.W, problem.heads, batch=problem.batch,
                       kind="iid", seed=2000 + seed)
    _run_and_compare(problem, params, q, k, v)
    dense = PT.from_device(PT.run_dense(problem, *(PT.to_device(a) for a in (q, k, v))))
    dense = dense.reshape(q.shape)
    g = PT.geometry(problem)
    for b in range(problem.batch):
        for h in range(problem.heads):
            ref = O.dense_head(*(O.bf16_bits_to_f64(a[b, h]) for a in (q, k, v)), g, SCALE)
            err = np.abs(O.bf16_bits_to_f64(dense[b, h]) - ref)
            assert err.max() <= PT.MAX_ABS and err.mean() <= PT.MEAN_ABS, (b, h, err.max())


@pytest.mark.parametrize("seed", range(12))
def test_backward_random_shape(seed):
    problem, params = _case(100 + seed)
    print(f"case {100 + seed}: grid {problem.T}x{problem.H}x{problem.W}, chunk "
          f"({problem.ct},{problem.ch},{problem.cw}), key chunk {problem.key_chunk}, cond "
          f"{problem.cond_frames}, batch {problem.batch}, heads {problem.heads}", flush=True)
    q, k, v = make_qkv(problem.T, problem.H, problem.W, problem.heads, batch=problem.batch,
                       kind="iid", seed=3000 + seed)
    do = make_grad(problem.T, problem.H, problem.W, problem.heads, batch=problem.batch,
                   seed=3000 + seed)
    idx, cnt, stride = oracle_selection(problem, params, q, k)
    compare_all(problem, q, k, v, do, idx, cnt, stride)
