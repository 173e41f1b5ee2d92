"""Seeded synthetic Q/K/V generators for the BSA workloads.

This module only draws random numbers and shapes them into inputs; it holds
none of the attention or selection arithmetic. Both the GPU path and the CPU
oracle's tests consume its output (bfloat16 bit patterns as uint16), so the
two sides see identical inputs by construction.

Recipes
-------
* ``"iid"``:   Q, K, V i.i.d. N(0, 1).
* ``"field"``: a smooth random field F shared by Q and K stands in for the
  spatio-temporal redundancy of video latents that block selection exploits.
  For every (batch, head, channel), F is i.i.d. N(0, 1) over the T x H x W
  grid, filtered by a separable Gaussian (sigma = 2 tokens on each axis,
  truncated at 4 sigma, periodic boundary), then scaled to unit standard
  deviation per channel. Q = F + 0.3 N(0,1), K = F + 0.3 N(0,1), V = N(0,1).

* ``make_grad``: the output gradient dL/dO of the backward workloads, i.i.d.
  N(0, 1) per element, from its own seed sequence.
* ``random_block_lists``, ``uniform_block_lists``: key-block lists drawn
  uniformly without replacement (for tests that fix the selection instead
  of deriving it from Q and K).

All values are rounded from float32 to bfloat16 with round-to-nearest-even.
Each (batch, head) draws from its own child of ``SeedSequence(seed)``, so any
subset of heads can be regenerated alone and heads can be produced in
parallel threads.
"""

from __future__ import annotations

import os
from concurrent.futures import ThreadPoolExecutor

import numpy as np

SIGMA = 2.0
TRUNCATE = 4.0
NOISE = 0.3


def f32_to_bf16_bits(x: np.ndarray) -> np.ndarray:
    """Round float32 to bfloat16 (nearest, ties to even); returns uint16 bits.
    Works through the array in slices so that the temporaries stay small."""
    u = np.ascontiguousarray(x, dtype=np.float32).view(np.uint32)
    flat = u.reshape(-1)
    out = np.empty(flat.shape, dtype=np.uint16)
    step = 1 << 24
    for i in range(0, flat.size, step):
        c = flat[i:i + step]
        bias = np.uint32(0x7FFF) + ((c >> np.uint32(16)) & np.uint32(1))
        out[i:i + step] = (c + bias) >> np.uint32(16)
    return out.reshape(u.shape)


def _circulant_gauss(n: int) -> np.ndarray:
    radius = int(TRUNCATE * SIGMA + 0.5)
    offs = np.arange(-radius, radius + 1)
    w = np.exp(-0.5 * (offs / SIGMA) ** 2)
    w /= w.sum()
    g = np.zeros((n, n), dtype=np.float64)
    for i in range(n):
        for o, wo in zip(offs, w):
            g[i, (i + o) % n] += wo
    return g.astype(np.float32)


def _smooth_field(rng: np.random.Generator, T: int, H: int, W: int, d: int) -> np.ndarray:
    """Gaussian-filtered white noise, [T*H*W, d] float32, unit std per channel."""
    x = rng.standard_normal((T, H, W, d), dtype=np.float32)
    gt, gh, gw = _circulant_gauss(T), _circulant_gauss(H), _circulant_gauss(W)
    x = np.matmul(gw, x.reshape(T * H, W, d))  # filter along w
    x = x.reshape(T, H, W, d).transpose(0, 2, 1, 3).reshape(T * W, H, d)
    x = np.matmul(gh, x).reshape(T, W, H, d).transpose(0, 2, 1, 3)  # along h
    x = np.ascontiguousarray(x).reshape(T, H * W * d)
    x = (gt @ x).reshape(T * H * W, d)  # along t
    std = x.std(axis=0, dtype=np.float64).astype(np.float32)
    x /= np.maximum(std, np.float32(1e-12))
    return x


def _one_head(kind: str, seq: np.random.SeedSequence, T: int, H: int, W: int, d: int):
    s_f, s_q, s_k, s_v = seq.spawn(4)
    S = T * H * W
    if kind == "iid":
        # Three independent streams: drawn (and rounded) in parallel threads,
        # with the same values as drawing them one after the other.
        def draw(stream):
            return f32_to_bf16_bits(np.random.default_rng(stream).standard_normal((S, d), dtype=np.float32))

        with ThreadPoolExecutor(max_workers=3) as ex:
            q, k, v = ex.map(draw, (s_q, s_k, s_v))
        return q, k, v
    elif kind == "field":
        f = _smooth_field(np.random.default_rng(s_f), T, H, W, d)
        q = np.random.default_rng(s_q).standard_normal((S, d), dtype=np.float32)
        q *= np.float32(NOISE)
        q += f
        k = np.random.default_rng(s_k).standard_normal((S, d), dtype=np.float32)
        k *= np.float32(NOISE)
        k += f
        del f
    else:
        raise ValueError(f"unknown input kind {kind!r}")
    v = np.random.default_rng(s_v).standard_normal((S, d), dtype=np.float32)
    return f32_to_bf16_bits(q), f32_to_bf16_bits(k), f32_to_bf16_bits(v)


def make_qkv(
    T: int,
    H: int,
    W: int,
    heads: int,
    head_dim: int = 128,
    batch: int = 1,
    kind: str = "field",
    seed: int = 0,
    head_subset=None,
    threads: int | None = None,
):
    """Generate Q, K, V as uint16 bfloat16 bits, each [batch, n, S, head_dim]
    where n = heads (or len(head_subset)); tokens in latent order
    s = (t*H + h)*W + w. ``head_subset`` lists (batch, head) pairs or head
    ids (batch 0) to generate alone; values equal the full draw's."""
    root = np.random.SeedSequence(seed)
    children = root.spawn(batch * heads)
    if head_subset is None:
        pairs = [(b, h) for b in range(batch) for h in range(heads)]
        shape_b, shape_h = batch, heads
    else:
        pairs = [p if isinstance(p, tuple) else (0, int(p)) for p in head_subset]
        shape_b, shape_h = 1, len(pairs)
    S = T * H * W
    out = [np.empty((shape_b, shape_h, S, head_dim), dtype=np.uint16) for _ in range(3)]

    def work(slot):
        b, h = pairs[slot]
        q, k, v = _one_head(kind, children[b * heads + h], T, H, W, head_dim)
        ob, oh = (b, h) if head_subset is None else (0, slot)
        out[0][ob, oh] = q
        out[1][ob, oh] = k
        out[2][ob, oh] = v

    n_threads = threads or min(16, os.cpu_count() or 1)
    with ThreadPoolExecutor(max_workers=max(1, n_threads)) as ex:
        list(ex.map(work, range(len(pairs))))
    return out[0], out[1], out[2]


def make_grad(T: int, H: int, W: int, heads: int, head_dim: int = 128, batch: int = 1,
              seed: int = 0, threads: int | None = None):
    """Output gradient dO, uint16 bfloat16 bits [batch, heads, S, head_dim],
    i.i.d. N(0, 1); head (b, h) draws from child b*heads + h of
    SeedSequence([seed, 0x644F])."""
    children = np.random.SeedSequence([seed, 0x644F]).spawn(batch * heads)
    S = T * H * W
    out = np.empty((batch, heads, S, head_dim), dtype=np.uint16)

    def work(i):
        b, h = divmod(i, heads)
        x = np.random.default_rng(children[i]).standard_normal((S, head_dim), dtype=np.float32)
        out[b, h] = f32_to_bf16_bits(x)

    n_threads = threads or min(16, os.cpu_count() or 1)
    with ThreadPoolExecutor(max_workers=max(1, n_threads)) as ex:
        list(ex.map(work, range(batch * heads)))
    return out


def uniform_block_lists(rows: int, n_blocks: int, count: int, seed: int = 0):
    """`count` distinct ids per row drawn uniformly from range(n_blocks), in
    ascending order (for very many rows: vectorised draws, rows with a
    repeated id drawn again). Returns (idx int32 [rows, count], cnt int32 [rows])."""
    rng = np.random.default_rng(seed)
    idx = np.sort(rng.integers(0, n_blocks, size=(rows, count)), axis=1)
    while True:
        bad = np.nonzero((np.diff(idx, axis=1) == 0).any(axis=1))[0]
        if bad.size == 0:
            break
        idx[bad] = np.sort(rng.integers(0, n_blocks, size=(bad.size, count)), axis=1)
    return idx.astype(np.int32), np.full(rows, count, dtype=np.int32)


def random_block_lists(allowed, stride: int, counts, seed: int = 0):
    """Key-block lists for len(allowed) rows: row i holds counts[i] distinct
    ids drawn uniformly from range(allowed[i]) (at most allowed[i] and
    stride of them), in ascending order, padded with -1 to `stride`.
    Returns (idx int32 [rows, stride], cnt int32 [rows])."""
    rng = np.random.default_rng(seed)
    rows = len(allowed)
    idx = np.full((rows, stride), -1, dtype=np.int32)
    cnt = np.zeros(rows, dtype=np.int32)
    for i in range(rows):
        c = int(min(counts[i], allowed[i], stride))
        if c > 0:
            idx[i, :c] = np.sort(rng.choice(int(allowed[i]), size=c, replace=False))
        cnt[i] = c
    return idx, cnt
