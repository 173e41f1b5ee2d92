"""CPU oracle for 3D Block Sparse Attention (BSA) -- TEST INFRASTRUCTURE ONLY.

This module is the parity reference for the HIP path. It is a plain, slow,
step-by-step numpy implementation in float64. It shares no code with the
product library; only ``tests/``, ``__graft_entry__.smoke()`` and the
``cpu_baseline`` leg of ``bench.py`` may import it. The product path never
calls it.

Sources (cited by page and section; the pages are the LongCat-Video
Technical Report and four write-ups about it):

* [DeepDive] "LongCat-Video Technical Report" (paper-graph-ui deep dive),
  section "Block Sparse Attention": paragraphs "3D block partitioning",
  "Pooled block similarity computation" (the Q_pool / K_pool equations),
  "Block selection via pooled attention scores" (the S_pool equation, top-r,
  mask M), "Sparse attention computation" (softmax(QK^T/sqrt(d) (.) M) V with
  non-selected positions set to -inf), and "Implementation details and design
  trade-offs" (Top-r mode and CDF-p mode).
* [DeepDive-KV] same page, section "Block Attention with KV-Cache for
  Efficient Multi-Task Inference", paragraph "Attention structure"
  (X_cond / X_noisy equations).
* [Notes] "LongCat-Video Technical Report" (zhaifeiyue paper notes),
  section 3 (architecture / method), subsection "3D Block Sparse Attention":
  default chunk shape [4, 4, 8]; Top-K, CDF-threshold and combined selection.

Readings where the pages are silent or inconsistent (each one is also listed
with its reason in the design notes of the repository):

* Block shape: (t, h, w) = (4, 4, 8) as in [Notes]; any positive shape is
  accepted here.
* Pooling index: 0-based, block b covers block-ordered slots b*n .. b*n+n-1.
* Partial blocks: [DeepDive] "3D block partitioning" counts blocks with
  ceilings (N_T = ceil(T / t), ...). A block at the far edge of a grid that
  its chunk does not divide holds only the tokens of its box that lie inside
  the grid; there are no padding tokens. Its pooled vector is the mean of
  the tokens it holds (the pooling equation's 1/n with n that block's token
  count), and a query block that selects it attends to those tokens only.
* Mask: additive -inf on non-selected keys (the prose of [DeepDive]), not a
  multiplicative (.) M.
* Top-k ranks pooled scores (softmax is monotone, so ranking P is the same);
  ties are broken towards the lower key-block id.
* CDF: order by (P descending, id ascending); keep the smallest prefix whose
  cumulative probability reaches p (the crossing block is kept); then clamp
  the count to [k_min, min(k_max, allowed)]. If no prefix reaches p (rounding
  when p = 1), every allowed block is the prefix.
* Block-causal: the X_cond / X_noisy equations of [DeepDive-KV] are applied at
  block granularity. Condition frames are the first ``cond_frames`` latent
  frames (a multiple of the block's t extent), so condition tokens fill the
  first key blocks. A condition query block may select only condition key
  blocks; a noisy query block may select any block. Softmax and selection run
  over the allowed blocks only.
* k larger than the number of allowed blocks is clamped to that number.
* Decoupled query and key blocks ([DeepDive] "Implementation details and
  design trade-offs" reports query blocks of 64 or 128 tokens and key blocks
  of 64 to 1024 tokens): queries are cut with the query chunk (ct, ch, cw)
  and keys with the key chunk (ctk, chk, cwk); each is pooled over its own
  blocks, S_pool is N_q x N_k, and a query block attends to the tokens of the
  key blocks it selects. Block order and intra-block order follow the same
  [N_T, N_H, N_W] / [t, h, w] rule for both. Condition frames must be a
  multiple of both t extents; condition key blocks are the leading ones.

Backward pass (the gradients of the attention step for fixed selections):
[DeepDive] "Implementation details and design trade-offs" states that the
operator has both a forward and a backward pass, and [Notes] section 7
("实现 cross-reference", on the same zhaifeiyue notes page) lists separate
dQ and dK/dV backward kernels and a forward-to-backward transpose of the
block index lists. The pages print no
backward formulas; ``backward_head`` differentiates the forward above
(softmax over the gathered keys) by the chain rule, and treats the block
selection as a constant (it is a discrete choice with no gradient).

Every function works on one (batch, head) slice: arrays are [S, d] in the
latent grid's own memory order (token s = (t*H + h)*W + w).
"""

from __future__ import annotations

from dataclasses import dataclass

import numpy as np

__all__ = [
    "Geometry",
    "SelectParams",
    "bf16_bits_to_f64",
    "block_token_order",
    "block_tokens",
    "pool_blocks",
    "pooled_scores",
    "allowed_key_blocks",
    "softmax_allowed",
    "select_topk",
    "select_cdf",
    "select_head",
    "attend_query_block",
    "bsa_head",
    "dense_head",
    "index_stride",
    "forward_lse_head",
    "backward_head",
    "key_geometry",
]


def _ceil_div(a: int, b: int) -> int:
    return -(-a // b)


@dataclass(frozen=True)
class Geometry:
    """Latent grid T x H x W cut into blocks of ct x ch x cw tokens.

    [DeepDive] "3D block partitioning": blocks of t x h x w tokens, N_T x N_H x
    N_W of them. [Notes] gives the default chunk shape [4, 4, 8].
    ``cond_frames`` is the number of leading latent frames that are condition
    tokens ([DeepDive-KV]); 0 disables block-causal attention.
    """

    T: int
    H: int
    W: int
    ct: int = 4
    ch: int = 4
    cw: int = 8
    cond_frames: int = 0
    # Key chunk; 0 means the same as the query chunk.
    ctk: int = 0
    chk: int = 0
    cwk: int = 0

    def __post_init__(self):
        for name in ("T", "H", "W", "ct", "ch", "cw"):
            if getattr(self, name) <= 0:
                raise ValueError(f"{name} must be positive")
        if (self.ctk, self.chk, self.cwk) != (0, 0, 0):
            if min(self.ctk, self.chk, self.cwk) <= 0:
                raise ValueError("key chunk extents must all be positive (or all 0)")
        if self.cond_frames < 0 or self.cond_frames % self.ct or (
            self.cond_frames and self.cond_frames >= self.T
        ):
            raise ValueError("cond_frames must be a multiple of ct and < T")
        if self.cond_frames % self.key_chunk[0]:
            raise ValueError("cond_frames must be a multiple of the key chunk's t extent")

    @property
    def key_chunk(self) -> tuple:
        if (self.ctk, self.chk, self.cwk) == (0, 0, 0):
            return (self.ct, self.ch, self.cw)
        return (self.ctk, self.chk, self.cwk)

    @property
    def nk(self) -> int:
        """Tokens per key block."""
        a, b, c = self.key_chunk
        return a * b * c

    @property
    def num_key_blocks(self) -> int:
        a, b, c = self.key_chunk
        return _ceil_div(self.T, a) * _ceil_div(self.H, b) * _ceil_div(self.W, c)

    @property
    def cond_key_blocks(self) -> int:
        """Key blocks made of condition tokens (the first ones in key-block order)."""
        a, b, c = self.key_chunk
        return (self.cond_frames // a) * _ceil_div(self.H, b) * _ceil_div(self.W, c)

    @property
    def n(self) -> int:
        return self.ct * self.ch * self.cw

    @property
    def nT(self) -> int:
        return _ceil_div(self.T, self.ct)

    @property
    def nH(self) -> int:
        return _ceil_div(self.H, self.ch)

    @property
    def nW(self) -> int:
        return _ceil_div(self.W, self.cw)

    @property
    def num_blocks(self) -> int:
        return self.nT * self.nH * self.nW

    @property
    def seq_len(self) -> int:
        return self.T * self.H * self.W

    @property
    def cond_blocks(self) -> int:
        """Query blocks made of condition tokens (the first ones in block order)."""
        return (self.cond_frames // self.ct) * self.nH * self.nW


def key_geometry(g: Geometry) -> Geometry:
    """The same grid cut with the key chunk: its blocks are g's key blocks."""
    a, b, c = g.key_chunk
    return Geometry(g.T, g.H, g.W, a, b, c, g.cond_frames)


@dataclass(frozen=True)
class SelectParams:
    """Selection rule. mode 'topk' keeps k blocks; mode 'cdf' keeps blocks by
    cumulative softmax mass p with the count clamped to [k_min, k_max]
    ([DeepDive] "Implementation details and design trade-offs"; [Notes]
    Top-K / CDF / combined)."""

    mode: str = "topk"
    k: int = 1
    p: float = 0.9
    k_min: int = 1
    k_max: int = 64

    def __post_init__(self):
        if self.mode not in ("topk", "cdf"):
            raise ValueError("mode must be 'topk' or 'cdf'")
        if self.mode == "topk" and self.k < 1:
            raise ValueError("k must be >= 1")
        if self.mode == "cdf":
            if not (0.0 < self.p <= 1.0):
                raise ValueError("p must be in (0, 1]")
            if self.k_min < 1 or self.k_max < self.k_min:
                raise ValueError("need 1 <= k_min <= k_max")


def index_stride(params: SelectParams) -> int:
    """Row length of the index list: k for top-k, k_max for CDF."""
    return params.k if params.mode == "topk" else params.k_max


def bf16_bits_to_f64(bits: np.ndarray) -> np.ndarray:
    """Exact widening of bfloat16 bit patterns (uint16) to float64.

    bfloat16 is the upper half of an IEEE-754 binary32, so the pattern moved
    into the high 16 bits of a 32-bit word is that float32 exactly (the pages
    fix no input precision; the inputs here are bf16 tensors)."""
    u32 = np.asarray(bits, dtype=np.uint16).astype(np.uint32) << np.uint32(16)
    return u32.view(np.float32).astype(np.float64)


def block_token_order(g: Geometry) -> np.ndarray:
    """perm[i*n + j] = latent-order token index of slot j of block i, or -1
    where slot j of a partial block lies outside the grid.

    [DeepDive] "3D block partitioning": tokens of a block are contiguous with
    intra-block order [t, h, w]; blocks are in [N_T, N_H, N_W] order, with
    N_T = ceil(T / t) and so on.
    """
    perm = np.full(g.num_blocks * g.n, -1, dtype=np.int64)
    pos = 0
    for bt in range(g.nT):
        for bh in range(g.nH):
            for bw in range(g.nW):
                for it in range(g.ct):
                    for ih in range(g.ch):
                        t = bt * g.ct + it
                        h = bh * g.ch + ih
                        w0 = bw * g.cw
                        if t < g.T and h < g.H:
                            run = min(g.cw, g.W - w0)
                            row = (t * g.H + h) * g.W + w0
                            perm[pos : pos + run] = np.arange(row, row + run)
                        pos += g.cw
    return perm


def block_tokens(perm: np.ndarray, i: int, n: int) -> np.ndarray:
    """Latent-order tokens of block i in slot order (slots outside the grid
    left out)."""
    t = perm[i * n : (i + 1) * n]
    return t[t >= 0]


def pool_blocks(x: np.ndarray, perm: np.ndarray, n: int) -> np.ndarray:
    """Mean of each block's tokens: X_pool[b] = (1/n_b) sum_j X[b*n + j] in
    block order, over the n_b slots of block b that lie inside the grid (all
    n of them unless b is partial) ([DeepDive] "Pooled block similarity
    computation")."""
    x = np.asarray(x, dtype=np.float64)
    nblk = perm.shape[0] // n
    out = np.empty((nblk, x.shape[-1]))
    for b in range(nblk):
        out[b] = x[block_tokens(perm, b, n)].mean(axis=0)
    return out


def pooled_scores(q_pool: np.ndarray, k_pool: np.ndarray, scale: float) -> np.ndarray:
    """S_pool = Q_pool K_pool^T / sqrt(d) ([DeepDive] "Block selection via
    pooled attention scores"); ``scale`` is 1/sqrt(d) unless overridden."""
    return (q_pool @ k_pool.T) * scale


def allowed_key_blocks(g: Geometry, i: int) -> int:
    """How many leading key blocks query block i may attend to.

    Block-causal ([DeepDive-KV] "Attention structure"): condition queries see
    condition keys only; noisy queries see all keys. Condition tokens are the
    first frames, so they occupy key blocks 0 .. cond_key_blocks-1.
    """
    if g.cond_frames and i < g.cond_blocks:
        return g.cond_key_blocks
    return g.num_key_blocks


def softmax_allowed(scores_row: np.ndarray, n_allowed: int) -> np.ndarray:
    """Softmax of one pooled-score row over its first n_allowed entries."""
    s = np.asarray(scores_row[:n_allowed], dtype=np.float64)
    e = np.exp(s - s.max())
    return e / e.sum()


def _rank_order(values: np.ndarray) -> np.ndarray:
    """Ids sorted by value descending, then id ascending."""
    ids = np.arange(values.shape[0])
    return np.lexsort((ids, -values))


def select_topk(scores_row: np.ndarray, n_allowed: int, k: int) -> np.ndarray:
    """Top-r mode: the min(k, n_allowed) allowed key blocks with the highest
    pooled scores, returned in ascending id order ([DeepDive] "Block selection
    via pooled attention scores")."""
    order = _rank_order(np.asarray(scores_row[:n_allowed], dtype=np.float64))
    keep = min(k, n_allowed)
    return np.sort(order[:keep])


def select_cdf(
    scores_row: np.ndarray, n_allowed: int, p: float, k_min: int, k_max: int
) -> np.ndarray:
    """CDF-p mode: walk key blocks in descending softmax probability until the
    cumulative probability reaches p; clamp the count to [k_min, k_max]
    ([DeepDive] "Implementation details and design trade-offs"; the clamps are
    the combined mode of [Notes])."""
    probs = softmax_allowed(scores_row, n_allowed)
    order = _rank_order(probs)
    cum = np.cumsum(probs[order])
    reached = np.nonzero(cum >= p)[0]
    count = int(reached[0]) + 1 if reached.size else n_allowed
    hi = min(k_max, n_allowed)
    count = min(max(count, k_min), hi)
    return np.sort(order[:count])


def select_head(
    q: np.ndarray, k: np.ndarray, g: Geometry, params: SelectParams, scale: float
):
    """Block selection for one (batch, head).

    Returns (idx, cnt, scores): idx is int32 [Nb, stride] with ascending
    key-block ids padded by -1, cnt is int32 [Nb], scores is the float64
    [Nb, Nk] pooled score matrix with -inf where a key block is not allowed.
    """
    qp = pool_blocks(q, block_token_order(g), g.n)
    kp = pool_blocks(k, block_token_order(key_geometry(g)), g.nk)
    s = pooled_scores(qp, kp, scale)
    nb = g.num_blocks
    stride = index_stride(params)
    idx = np.full((nb, stride), -1, dtype=np.int32)
    cnt = np.zeros(nb, dtype=np.int32)
    masked = np.full_like(s, -np.inf)
    for i in range(nb):
        na = allowed_key_blocks(g, i)
        masked[i, :na] = s[i, :na]
        if params.mode == "topk":
            sel = select_topk(s[i], na, params.k)
        else:
            sel = select_cdf(s[i], na, params.p, params.k_min, params.k_max)
        cnt[i] = sel.size
        idx[i, : sel.size] = sel
    return idx, cnt, masked


def attend_query_block(
    q: np.ndarray,
    k: np.ndarray,
    v: np.ndarray,
    g: Geometry,
    i: int,
    key_blocks,
    scale: float,
    perm: np.ndarray | None = None,
    kperm: np.ndarray | None = None,
) -> np.ndarray:
    """Attention of query block i restricted to the given key blocks.

    [DeepDive] "Sparse attention computation": O = softmax(QK^T/sqrt(d) with
    non-selected keys at -inf) V. Keys outside the selected blocks contribute
    exp(-inf) = 0, so softmax over the gathered keys is the same thing.
    ``perm`` / ``kperm`` are the query and key block orders (computed when
    not given). Returns float64 rows for the block's tokens in slot order
    ([n, d] unless the block is partial; a partial key block contributes its
    tokens inside the grid only).
    """
    if perm is None:
        perm = block_token_order(g)
    if kperm is None:
        kperm = block_token_order(key_geometry(g))
    n, nk = g.n, g.nk
    qi = np.asarray(q, dtype=np.float64)[block_tokens(perm, i, n)]
    tok = np.concatenate([block_tokens(kperm, j, nk) for j in key_blocks])
    ks = np.asarray(k, dtype=np.float64)[tok]
    vs = np.asarray(v, dtype=np.float64)[tok]
    logits = (qi @ ks.T) * scale
    logits -= logits.max(axis=1, keepdims=True)
    w = np.exp(logits)
    w /= w.sum(axis=1, keepdims=True)
    return w @ vs


def bsa_head(
    q: np.ndarray,
    k: np.ndarray,
    v: np.ndarray,
    g: Geometry,
    params: SelectParams,
    scale: float,
):
    """Full BSA forward for one (batch, head): returns (out [S, d] float64 in
    latent order, idx, cnt, scores)."""
    idx, cnt, scores = select_head(q, k, g, params, scale)
    perm = block_token_order(g)
    kperm = block_token_order(key_geometry(g))
    out = np.zeros((g.seq_len, np.asarray(v).shape[-1]), dtype=np.float64)
    n = g.n
    for i in range(g.num_blocks):
        sel = idx[i, : cnt[i]]
        out[block_tokens(perm, i, n)] = attend_query_block(q, k, v, g, i, sel, scale, perm, kperm)
    return out, idx, cnt, scores


def dense_head(q: np.ndarray, k: np.ndarray, v: np.ndarray, g: Geometry, scale: float):
    """Dense softmax attention over every allowed key block (block-causal when
    cond_frames > 0), one (batch, head); [S, d] float64 in latent order."""
    perm = block_token_order(g)
    kperm = block_token_order(key_geometry(g))
    out = np.zeros((g.seq_len, np.asarray(v).shape[-1]), dtype=np.float64)
    n = g.n
    for i in range(g.num_blocks):
        na = allowed_key_blocks(g, i)
        out[block_tokens(perm, i, n)] = attend_query_block(
            q, k, v, g, i, range(na), scale, perm, kperm
        )
    return out


def _gathered(q, k, v, g, i, key_blocks, perm, kperm):
    n, nk = g.n, g.nk
    qt = block_tokens(perm, i, n)
    kt = np.concatenate([block_tokens(kperm, j, nk) for j in key_blocks])
    return qt, kt


def forward_lse_head(q, k, v, g: Geometry, idx, cnt, scale: float, query_blocks=None):
    """Forward over given selections, also returning each query's softmax
    log-normaliser lse = log(sum_j exp(s_j)) (natural log, over its gathered
    keys; -inf for a query block with no key block). Returns (out [S, d],
    lse [S]) in latent order, float64. With `query_blocks` given, only those
    query blocks are computed (the others stay 0 / -inf)."""
    perm = block_token_order(g)
    kperm = block_token_order(key_geometry(g))
    q = np.asarray(q, np.float64)
    k = np.asarray(k, np.float64)
    v = np.asarray(v, np.float64)
    out = np.zeros((g.seq_len, v.shape[-1]))
    lse = np.full(g.seq_len, -np.inf)
    for i in range(g.num_blocks) if query_blocks is None else sorted(set(query_blocks)):
        blocks = [int(j) for j in idx[i, : cnt[i]]]
        if not blocks:
            continue
        qt, kt = _gathered(q, k, v, g, i, blocks, perm, kperm)
        logits = (q[qt] @ k[kt].T) * scale
        m = logits.max(axis=1, keepdims=True)
        e = np.exp(logits - m)
        l = e.sum(axis=1, keepdims=True)
        out[qt] = (e / l) @ v[kt]
        lse[qt] = (m + np.log(l))[:, 0]
    return out, lse


def backward_head(q, k, v, do, g: Geometry, idx, cnt, scale: float, query_blocks=None):
    """Gradients of L = sum(dO * O) with respect to q, k and v, where O is the
    forward over the given selections (held fixed). For query block i with
    gathered keys K_J, values V_J and probabilities P = softmax(Q_i K_J^T s):

        dV_J += P^T dO_i
        dP    = dO_i V_J^T
        dS    = P * (dP - rowsum(dO_i * O_i))     (softmax Jacobian)
        dQ_i += s * dS K_J
        dK_J += s * dS^T Q_i

    Returns (dq, dk, dv), each [S, d] in latent order, float64.

    With `query_blocks` given, only those query blocks are visited: dq is
    then exact on their tokens, and dk, dv are exact on the tokens of any key
    block that only those query blocks keep (the sums above run over the
    query blocks that kept each key block)."""
    perm = block_token_order(g)
    kperm = block_token_order(key_geometry(g))
    q = np.asarray(q, np.float64)
    k = np.asarray(k, np.float64)
    v = np.asarray(v, np.float64)
    do = np.asarray(do, np.float64)
    dq = np.zeros_like(q)
    dk = np.zeros_like(k)
    dv = np.zeros_like(v)
    for i in range(g.num_blocks) if query_blocks is None else sorted(set(query_blocks)):
        blocks = [int(j) for j in idx[i, : cnt[i]]]
        if not blocks:
            continue
        qt, kt = _gathered(q, k, v, g, i, blocks, perm, kperm)
        logits = (q[qt] @ k[kt].T) * scale
        logits -= logits.max(axis=1, keepdims=True)
        p = np.exp(logits)
        p /= p.sum(axis=1, keepdims=True)
        o = p @ v[kt]
        delta = (do[qt] * o).sum(axis=1, keepdims=True)
        dp = do[qt] @ v[kt].T
        ds = p * (dp - delta)
        dq[qt] += scale * (ds @ k[kt])
        np.add.at(dk, kt, scale * (ds.T @ q[qt]))
        np.add.at(dv, kt, p.T @ do[qt])
    return dq, dk, dv
