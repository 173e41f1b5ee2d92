"""A numpy model of the roundings the HIP backward makes, used to derive the
dQ tolerance of the GPU parity tests (test infrastructure only).

The GPU computes every product from bf16 operands with fp32 accumulation.
The roundings that matter for dQ are, in order:
  * O, written by the forward in bf16, from which D = rowsum(dO * O) is formed;
  * P = exp(scale q.k - lse), rounded to bf16 as an MFMA operand;
  * dS = P * (dP - D), rounded to bf16 as an MFMA operand;
  * dQ itself, written in bf16.
``dq_with_gpu_roundings`` applies exactly these four roundings (round to
nearest even) to the oracle's float64 definition of the gradient and keeps
everything else in float64, so its distance to the oracle's dQ is the error
the tolerance has to admit, apart from fp32 accumulation (2^-24 per add).
"""

from __future__ import annotations

import numpy as np

import oracle.bsa_oracle as O


def round_bf16(x: np.ndarray) -> np.ndarray:
    """Round float64 values to the nearest bfloat16 (ties to even), through
    float32 as the GPU does, and return them as float64."""
    f32 = np.asarray(x, dtype=np.float64).astype(np.float32)
    u = f32.view(np.uint32).astype(np.uint64)
    u = (u + 0x7FFF + ((u >> 16) & 1)) & 0xFFFF0000
    return u.astype(np.uint32).view(np.float32).astype(np.float64)


def dq_with_gpu_roundings(q, k, v, do, g, idx, cnt, scale):
    """dQ of L = sum(dO * O) for fixed selections with the HIP path's bf16
    roundings of O, P, dS and dQ; float64 otherwise."""
    perm = O.block_token_order(g)
    kperm = O.block_token_order(O.key_geometry(g))
    q, k, v, do = (np.asarray(a, np.float64) for a in (q, k, v, do))
    dq = np.zeros_like(q)
    n, nk = g.n, g.nk
    for i in range(g.num_blocks):
        blocks = [int(j) for j in idx[i, : cnt[i]]]
        if not blocks:
            continue
        qt = O.block_tokens(perm, i, n)
        kt = np.concatenate([O.block_tokens(kperm, j, nk) for j in blocks])
        logits = (q[qt] @ k[kt].T) * scale
        m = logits.max(axis=1, keepdims=True)
        e = np.exp(logits - m)
        p = e / e.sum(axis=1, keepdims=True)
        o = round_bf16(p @ v[kt])                      # forward output, bf16
        delta = (do[qt] * o).sum(axis=1, keepdims=True)
        dp = do[qt] @ v[kt].T
        ds = round_bf16(round_bf16(p) * (dp - delta))  # P and dS as bf16 operands
        dq[qt] = scale * (ds @ k[kt])
    return round_bf16(dq)
