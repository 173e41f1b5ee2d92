"""Pins for the CPU oracle: checks against what the definitions and plain
mathematics fix, independent of the oracle's own code paths.

Each ``pin_*`` function raises AssertionError when the oracle disagrees.
``test_oracle_pins.py`` runs them; ``test_oracle_mutations.py`` plants
mistakes in the oracle and checks that some pin catches each one.
"""

from __future__ import annotations

import json
import math
import os
from fractions import Fraction

import numpy as np

import oracle.bsa_oracle as O

GOLDEN = os.path.join(os.path.dirname(os.path.abspath(__file__)), "golden")


# ---------------------------------------------------------------- helpers ---
def _coords(g, tokens):
    """(t, h, w) of latent-order token ids."""
    tokens = np.asarray(tokens)
    return tokens // (g.H * g.W), (tokens // g.W) % g.H, tokens % g.W


def _block_of_token(g):
    """Block id of every latent-order token, from its grid coordinates."""
    t, h, w = _coords(g, np.arange(g.seq_len))
    return ((t // g.ct) * g.nH + (h // g.ch)) * g.nW + (w // g.cw)


def _textbook_attention(q, k, v, scale, allowed=None):
    """softmax(q k^T * scale [+ log allowed]) v over whole sequences, fp64."""
    logits = (np.asarray(q, np.float64) @ np.asarray(k, np.float64).T) * scale
    if allowed is not None:
        logits = np.where(allowed, logits, -np.inf)
    logits -= logits.max(axis=1, keepdims=True)
    w = np.exp(logits)
    w /= w.sum(axis=1, keepdims=True)
    return w @ np.asarray(v, np.float64)


def _rand(rng, g, d=16):
    S = g.seq_len
    return (rng.standard_normal((S, d)), rng.standard_normal((S, d)), rng.standard_normal((S, d)))


# ------------------------------------------------------------------- pins ---
def pin_block_order_geometry():
    """Each block is a ct x ch x cw box at its origin, blocks run in
    [N_T, N_H, N_W] order and slots in [t, h, w] order; perm is a bijection."""
    for g in (O.Geometry(8, 8, 16), O.Geometry(4, 8, 8, 2, 4, 4), O.Geometry(6, 4, 9, 3, 2, 3)):
        perm = O.block_token_order(g)
        assert np.array_equal(np.sort(perm), np.arange(g.seq_len)), "not a permutation"
        n = g.n
        for i in range(g.num_blocks):
            bt, rem = divmod(i, g.nH * g.nW)
            bh, bw = divmod(rem, g.nW)
            t, h, w = _coords(g, perm[i * n : (i + 1) * n])
            lt, lh, lw = t - bt * g.ct, h - bh * g.ch, w - bw * g.cw
            for name, loc, ext in (("t", lt, g.ct), ("h", lh, g.ch), ("w", lw, g.cw)):
                assert loc.min() == 0 and loc.max() == ext - 1, f"block {i} {name} extent"
            slot = (lt * g.ch + lh) * g.cw + lw
            assert np.array_equal(slot, np.arange(n)), f"block {i} slot order"


def _load_golden():
    with open(os.path.join(GOLDEN, "handworked_blocks.json")) as f:
        return json.load(f)


def pin_handworked_golden():
    """Hand-derived selections and outputs (tests/golden/handworked_blocks.json)."""
    gold = _load_golden()
    st = gold["setup"]
    a = st["q_first_channel_per_block"]
    b = [x * np.log(2.0) for x in st["k_first_channel_per_block_in_units_of_ln2"]]
    for case in gold["cases"]:
        g = O.Geometry(st["grid"]["T"], st["grid"]["H"], st["grid"]["W"], *st["chunk"],
                       cond_frames=case["cond_frames"])
        d = st["head_dim"]
        blk = _block_of_token(g)
        q = np.zeros((g.seq_len, d))
        k = np.zeros((g.seq_len, d))
        v = np.zeros((g.seq_len, d))
        q[:, 0] = np.asarray(a)[blk]
        k[:, 0] = np.asarray(b)[blk]
        v[np.arange(g.seq_len), blk] = 1.0
        if case["mode"] == "topk":
            p = O.SelectParams("topk", k=case["k"])
        else:
            p = O.SelectParams("cdf", p=case["p"], k_min=case["k_min"], k_max=case["k_max"])
        out, idx, cnt, _ = O.bsa_head(q, k, v, g, p, st["scale"])
        for i, exp_ids in enumerate(case["idx"]):
            got = idx[i, : cnt[i]].tolist()
            assert got == exp_ids, f"{case['name']} row {i}: {got} != {exp_ids}"
            assert np.all(idx[i, cnt[i]:] == -1)
            want = np.array([float(Fraction(x)) for x in case["out"][i]])
            rows = out[blk == i]
            assert np.abs(rows - want).max() < 1e-12, f"{case['name']} output row {i}"


def pin_dense_equals_textbook():
    """Selecting every block reduces BSA to plain softmax attention."""
    rng = np.random.default_rng(11)
    g = O.Geometry(4, 8, 16)
    q, k, v = _rand(rng, g)
    scale = 1 / np.sqrt(q.shape[1])
    ref = _textbook_attention(q, k, v, scale)
    out, idx, cnt, _ = O.bsa_head(q, k, v, g, O.SelectParams("topk", k=g.num_blocks), scale)
    assert np.all(cnt == g.num_blocks)
    assert np.abs(out - ref).max() < 1e-12, "BSA with all blocks != dense attention"
    assert np.abs(O.dense_head(q, k, v, g, scale) - ref).max() < 1e-12
    big_k = O.bsa_head(q, k, v, g, O.SelectParams("topk", k=99), scale)[0]
    assert np.abs(big_k - ref).max() < 1e-12, "k above the block count must clamp"


def pin_mask_formula():
    """Gathered attention equals the mask formulation over the whole sequence:
    keys outside the selected blocks get -inf before the softmax."""
    rng = np.random.default_rng(12)
    for g, p in (
        (O.Geometry(8, 8, 16), O.SelectParams("topk", k=3)),
        (O.Geometry(8, 8, 16, cond_frames=4), O.SelectParams("cdf", p=0.6, k_min=1, k_max=5)),
    ):
        q, k, v = _rand(rng, g)
        scale = 1 / np.sqrt(q.shape[1])
        out, idx, cnt, _ = O.bsa_head(q, k, v, g, p, scale)
        blk = _block_of_token(g)
        sel = np.zeros((g.num_blocks, g.num_blocks), dtype=bool)
        for i in range(g.num_blocks):
            sel[i, idx[i, : cnt[i]]] = True
        allowed = sel[blk[:, None], blk[None, :]]
        ref = _textbook_attention(q, k, v, scale, allowed)
        assert np.abs(out - ref).max() < 1e-12, "gathered attention != masked attention"


def pin_pooled_scores_bruteforce():
    """Pooled scores recomputed from grid coordinates (block means by
    accumulation, then dot products) match the oracle's."""
    rng = np.random.default_rng(13)
    for g in (O.Geometry(8, 8, 16), O.Geometry(4, 8, 8, 2, 4, 4, cond_frames=2)):
        q, k, _ = _rand(rng, g)
        scale = 0.37
        blk = _block_of_token(g)
        qs = np.zeros((g.num_blocks, q.shape[1]))
        ks = np.zeros_like(qs)
        np.add.at(qs, blk, q)
        np.add.at(ks, blk, k)
        counts = np.bincount(blk, minlength=g.num_blocks)[:, None]
        s_ref = (qs / counts) @ (ks / counts).T * scale
        _, _, scores = O.select_head(q, k, g, O.SelectParams("topk", k=1), scale)
        for i in range(g.num_blocks):
            na = O.allowed_key_blocks(g, i)
            assert np.abs(scores[i, :na] - s_ref[i, :na]).max() < 1e-12, "pooled score"
            assert np.all(np.isneginf(scores[i, na:]))


def pin_topk_property():
    """Top-k sets: right size, every kept score >= every dropped score, and
    equal scores at the cut go to the lower ids."""
    rng = np.random.default_rng(14)
    for trial in range(300):
        n = int(rng.integers(1, 40))
        s = np.round(rng.standard_normal(n), 1)  # rounding makes ties common
        na = int(rng.integers(1, n + 1))
        k = int(rng.integers(1, n + 3))
        sel = O.select_topk(s, na, k)
        assert sel.size == min(k, na)
        assert np.all(np.diff(sel) > 0) and (sel.size == 0 or sel.max() < na)
        rest = np.setdiff1d(np.arange(na), sel)
        if rest.size and sel.size:
            cut = s[sel].min()
            assert cut >= s[rest].max()
            tied_in = sel[s[sel] == cut]
            tied_out = rest[s[rest] == cut]
            if tied_out.size:
                assert tied_in.max() < tied_out.min(), "ties must go to lower ids"


def pin_cdf_property():
    """CDF sets: a top set by probability; its mass reaches p and dropping its
    least likely member falls below p, unless a clamp decided the count."""
    rng = np.random.default_rng(15)
    for trial in range(300):
        n = int(rng.integers(1, 30))
        s = rng.standard_normal(n) * rng.uniform(0.1, 4)
        na = int(rng.integers(1, n + 1))
        p = float(rng.uniform(0.05, 1.0))
        kmin = int(rng.integers(1, 6))
        kmax = int(rng.integers(kmin, 12))
        sel = O.select_cdf(s, na, p, kmin, kmax)
        e = np.exp(s[:na] - s[:na].max())
        prob = e / e.sum()
        assert np.all(np.diff(sel) > 0) and sel.max() < na
        rest = np.setdiff1d(np.arange(na), sel)
        if rest.size:
            assert prob[sel].min() >= prob[rest].max() - 1e-15
        m = sel.size
        mass = prob[sel].sum()
        hi = min(kmax, na)
        if kmin < m < hi:
            assert mass >= p - 1e-12, "mass must reach p"
            assert mass - prob[sel].min() < p + 1e-12, "prefix must be minimal"
        if m == hi and hi > kmin:
            assert mass - prob[sel].min() < p + 1e-12
        if m == kmin and kmin < hi:
            assert mass >= p - 1e-12, "k_min clamp only raises the count"
        assert kmin <= m or m == na
        assert m <= hi


def pin_rows_sum_to_one():
    """With V = block indicators, each output row is the attention mass per
    key block: non-negative, zero outside the selection, summing to 1."""
    rng = np.random.default_rng(16)
    g = O.Geometry(8, 8, 16, cond_frames=4)
    q, k, _ = _rand(rng, g)
    blk = _block_of_token(g)
    v = np.zeros((g.seq_len, g.num_blocks))
    v[np.arange(g.seq_len), blk] = 1.0
    for p in (O.SelectParams("topk", k=3), O.SelectParams("cdf", p=0.8, k_min=2, k_max=6)):
        out, idx, cnt, _ = O.bsa_head(q, k, v, g, p, 0.25)
        assert np.abs(out.sum(axis=1) - 1).max() < 1e-12, "rows must sum to 1"
        assert out.min() > -1e-15
        for i in range(g.num_blocks):
            off = np.setdiff1d(np.arange(g.num_blocks), idx[i, : cnt[i]])
            assert np.abs(out[blk == i][:, off]).max() == 0.0


def pin_constant_v():
    """V constant => O equals that constant for every query."""
    rng = np.random.default_rng(17)
    g = O.Geometry(8, 8, 16)
    q, k, _ = _rand(rng, g)
    v = np.tile(np.linspace(-2, 3, q.shape[1]), (g.seq_len, 1))
    out = O.bsa_head(q, k, v, g, O.SelectParams("topk", k=2), 0.3)[0]
    assert np.abs(out - v).max() < 1e-12


def pin_q_zero():
    """Q = 0: all pooled scores tie, so top-k keeps blocks 0..k-1 and every
    query averages V over those blocks' tokens; CDF keeps ceil(p * allowed)."""
    rng = np.random.default_rng(18)
    g = O.Geometry(8, 8, 16, cond_frames=4)
    _, k, v = _rand(rng, g)
    q = np.zeros_like(k)
    blk = _block_of_token(g)
    out, idx, cnt, _ = O.bsa_head(q, k, v, g, O.SelectParams("topk", k=3), 0.2)
    for i in range(g.num_blocks):
        na = O.allowed_key_blocks(g, i)
        want = list(range(min(3, na)))
        assert idx[i, : cnt[i]].tolist() == want
        mean_v = v[np.isin(blk, want)].mean(axis=0)
        assert np.abs(out[blk == i] - mean_v).max() < 1e-12
    _, idx, cnt, _ = O.bsa_head(q, k, v, g, O.SelectParams("cdf", p=0.3, k_min=1, k_max=8), 0.2)
    for i in range(g.num_blocks):
        na = O.allowed_key_blocks(g, i)
        want = min(int(np.ceil(0.3 * na)), 8)
        assert cnt[i] == want and idx[i, : cnt[i]].tolist() == list(range(want))


def pin_intra_block_shuffle():
    """Shuffling tokens inside every block (same shuffle for Q, K, V) keeps
    pooled scores and selections and moves the outputs with the tokens."""
    rng = np.random.default_rng(19)
    g = O.Geometry(8, 8, 16)
    q, k, v = _rand(rng, g)
    perm = O.block_token_order(g)
    shuffled = perm.copy()
    for i in range(g.num_blocks):
        seg = shuffled[i * g.n : (i + 1) * g.n]
        shuffled[i * g.n : (i + 1) * g.n] = seg[rng.permutation(g.n)]
    remap = np.empty(g.seq_len, dtype=np.int64)
    remap[perm] = shuffled  # token perm[x] now holds the data of token shuffled[x]
    p = O.SelectParams("topk", k=3)
    out, idx, cnt, sc = O.bsa_head(q, k, v, g, p, 0.25)
    out2, idx2, cnt2, sc2 = O.bsa_head(q[remap], k[remap], v[remap], g, p, 0.25)
    assert np.abs(sc - sc2)[np.isfinite(sc)].max() < 1e-12
    assert np.array_equal(idx, idx2) and np.array_equal(cnt, cnt2)
    assert np.abs(out2 - out[remap]).max() < 1e-12


def pin_block_causal_independence():
    """Condition rows never see noisy tokens: replacing every noisy token's
    Q, K, V leaves their selections and outputs bitwise unchanged."""
    rng = np.random.default_rng(20)
    g = O.Geometry(12, 8, 16, cond_frames=4)
    q, k, v = _rand(rng, g)
    t = _coords(g, np.arange(g.seq_len))[0]
    noisy = t >= g.cond_frames
    q2, k2, v2 = q.copy(), k.copy(), v.copy()
    for a in (q2, k2, v2):
        a[noisy] = rng.standard_normal((int(noisy.sum()), a.shape[1]))
    for p in (O.SelectParams("topk", k=2), O.SelectParams("cdf", p=0.7, k_min=1, k_max=4)):
        out, idx, cnt, _ = O.bsa_head(q, k, v, g, p, 0.25)
        out2, idx2, cnt2, _ = O.bsa_head(q2, k2, v2, g, p, 0.25)
        c = g.cond_blocks
        assert np.array_equal(idx[:c], idx2[:c]) and np.array_equal(cnt[:c], cnt2[:c])
        assert np.array_equal(out[~noisy], out2[~noisy])
        assert idx[:c].max() < c


def pin_block_causal_dense_definition():
    """Dense block-causal attention equals X_cond = Attn(Q_c, K_c, V_c) and
    X_noisy = Attn(Q_n, [K_c, K_n], [V_c, V_n]) over the token sets."""
    rng = np.random.default_rng(21)
    g = O.Geometry(8, 8, 16, cond_frames=4)
    q, k, v = _rand(rng, g)
    cond = _coords(g, np.arange(g.seq_len))[0] < g.cond_frames
    scale = 0.21
    ref = np.zeros_like(q)
    ref[cond] = _textbook_attention(q[cond], k[cond], v[cond], scale)
    ref[~cond] = _textbook_attention(q[~cond], k, v, scale)
    assert np.abs(O.dense_head(q, k, v, g, scale) - ref).max() < 1e-12


def pin_monotonic():
    """Selections grow with k and with p."""
    rng = np.random.default_rng(22)
    g = O.Geometry(8, 16, 16)
    q, k, _ = _rand(rng, g)
    prev = None
    for kk in range(1, g.num_blocks + 1):
        idx, cnt, _ = O.select_head(q, k, g, O.SelectParams("topk", k=kk), 0.25)
        sets = [set(idx[i, : cnt[i]].tolist()) for i in range(g.num_blocks)]
        if prev is not None:
            assert all(a <= b for a, b in zip(prev, sets))
        prev = sets
    prev = None
    for pp in (0.1, 0.3, 0.5, 0.7, 0.9, 1.0):
        idx, cnt, _ = O.select_head(
            q, k, g, O.SelectParams("cdf", p=pp, k_min=1, k_max=g.num_blocks), 0.25)
        sets = [set(idx[i, : cnt[i]].tolist()) for i in range(g.num_blocks)]
        if prev is not None:
            assert all(a <= b for a, b in zip(prev, sets))
        prev = sets


# ------------------------------------------------------------ backward pins ---
def _bwd_case(seed=11, d=8):
    """A 4-block geometry, random float64 tensors and fixed selections that
    include a one-block row and overlapping key sets."""
    g = O.Geometry(4, 8, 16)
    rng = np.random.default_rng(seed)
    q, k, v, do = (rng.standard_normal((g.seq_len, d)) for _ in range(4))
    idx = np.array([[0, 2, -1], [1, 3, 0], [3, -1, -1], [0, 1, 2]])
    cnt = np.array([2, 3, 1, 3])
    return g, q, k, v, do, idx, cnt


def _loss(q, k, v, do, g, idx, cnt, scale):
    """L = sum(dO * O) with O from the forward definition (attention over the
    gathered keys of each query block)."""
    perm = O.block_token_order(g)
    total = 0.0
    n = g.n
    for i in range(g.num_blocks):
        blocks = [int(j) for j in idx[i, : cnt[i]]]
        if blocks:
            o = O.attend_query_block(q, k, v, g, i, blocks, scale, perm)
            total += float((do[perm[i * n : (i + 1) * n]] * o).sum())
    return total


def pin_backward_finite_differences():
    """Analytic gradients equal central differences of L = sum(dO * O) taken
    through the forward definition, on 24 random coordinates of each input."""
    g, q, k, v, do, idx, cnt = _bwd_case()
    scale = 0.35
    dq, dk, dv = O.backward_head(q, k, v, do, g, idx, cnt, scale)
    rng = np.random.default_rng(5)
    h = 1e-5
    for name, x, grad in (("q", q, dq), ("k", k, dk), ("v", v, dv)):
        for _ in range(24):
            r = int(rng.integers(x.shape[0]))
            c = int(rng.integers(x.shape[1]))
            xp = x.copy()
            xm = x.copy()
            xp[r, c] += h
            xm[r, c] -= h
            args = {"q": q, "k": k, "v": v}
            args[name] = xp
            lp = _loss(args["q"], args["k"], args["v"], do, g, idx, cnt, scale)
            args[name] = xm
            lm = _loss(args["q"], args["k"], args["v"], do, g, idx, cnt, scale)
            fd = (lp - lm) / (2 * h)
            assert abs(fd - grad[r, c]) <= 1e-6 * max(1.0, abs(fd)), (name, r, c, fd, grad[r, c])


def pin_backward_dense_autograd():
    """With every block selected, the gradients are those of textbook softmax
    attention over the whole sequence, here from torch autograd in float64."""
    import torch

    g = O.Geometry(4, 8, 16)
    rng = np.random.default_rng(8)
    q, k, v, do = (rng.standard_normal((g.seq_len, 8)) for _ in range(4))
    nb = g.num_blocks
    idx = np.tile(np.arange(nb), (nb, 1))
    cnt = np.full(nb, nb)
    scale = 0.3
    dq, dk, dv = O.backward_head(q, k, v, do, g, idx, cnt, scale)
    tq, tk, tv = (torch.tensor(a, dtype=torch.float64, requires_grad=True) for a in (q, k, v))
    out = torch.softmax((tq @ tk.T) * scale, dim=1) @ tv
    (out * torch.tensor(do)).sum().backward()
    for mine, ref in ((dq, tq.grad), (dk, tk.grad), (dv, tv.grad)):
        assert np.abs(mine - ref.numpy()).max() < 1e-10


def pin_backward_constant_v():
    """V constant: O does not depend on q or k, so dQ = dK = 0."""
    g, q, k, _, do, idx, cnt = _bwd_case(seed=12)
    v = np.full_like(q, -1.25)
    dq, dk, _ = O.backward_head(q, k, v, do, g, idx, cnt, 0.4)
    assert np.abs(dq).max() < 1e-12 and np.abs(dk).max() < 1e-12


def pin_backward_dv_total():
    """Rows of P sum to one, so the sum of dV over all keys equals the sum of
    dO over the queries that attend to anything."""
    g, q, k, v, do, idx, cnt = _bwd_case(seed=13)
    _, _, dv = O.backward_head(q, k, v, do, g, idx, cnt, 0.4)
    perm = O.block_token_order(g)
    n = g.n
    rows = np.concatenate([perm[i * n : (i + 1) * n] for i in range(g.num_blocks) if cnt[i] > 0])
    assert np.abs(dv.sum(axis=0) - do[rows].sum(axis=0)).max() < 1e-10


def pin_forward_lse():
    """forward_lse_head reproduces the pinned forward, and exp(s - lse) over a
    query's gathered keys sums to one."""
    g, q, k, v, _, idx, cnt = _bwd_case(seed=14)
    scale = 0.4
    out, lse = O.forward_lse_head(q, k, v, g, idx, cnt, scale)
    perm = O.block_token_order(g)
    n = g.n
    for i in range(g.num_blocks):
        blocks = [int(j) for j in idx[i, : cnt[i]]]
        qt = perm[i * n : (i + 1) * n]
        ref = O.attend_query_block(q, k, v, g, i, blocks, scale, perm)
        assert np.abs(out[qt] - ref).max() < 1e-12
        kt = np.concatenate([perm[j * n : (j + 1) * n] for j in blocks])
        s = (q[qt] @ k[kt].T) * scale
        assert np.abs(np.exp(s - lse[qt][:, None]).sum(axis=1) - 1).max() < 1e-12


def pin_backward_query_block_subset():
    """Visiting a subset of query blocks: dq exact on those blocks, dk and dv
    exact on a key block kept only by the subset (key block 3 is kept by rows
    1 and 2 only), and the forward's lse exact on the visited blocks."""
    g, q, k, v, do, idx, cnt = _bwd_case(seed=5)
    s = 0.37
    full = O.backward_head(q, k, v, do, g, idx, cnt, s)
    sub = O.backward_head(q, k, v, do, g, idx, cnt, s, query_blocks=[2, 1, 1])
    perm = O.block_token_order(g)
    blk = lambda b: perm[b * g.n:(b + 1) * g.n]
    for b in (1, 2):
        assert np.allclose(sub[0][blk(b)], full[0][blk(b)], rtol=0, atol=1e-12)
    for b in (0, 3):
        assert np.all(sub[0][blk(b)] == 0)
    for t in (1, 2):
        assert np.allclose(sub[t][blk(3)], full[t][blk(3)], rtol=0, atol=1e-12)
    o_full, l_full = O.forward_lse_head(q, k, v, g, idx, cnt, s)
    o_sub, l_sub = O.forward_lse_head(q, k, v, g, idx, cnt, s, query_blocks=[3, 0])
    for b in (0, 3):
        assert np.allclose(l_sub[blk(b)], l_full[blk(b)], rtol=0, atol=1e-12)
        assert np.allclose(o_sub[blk(b)], o_full[blk(b)], rtol=0, atol=1e-12)
    assert np.all(l_sub[blk(1)] == -np.inf) and np.all(o_sub[blk(2)] == 0)


# ---------------------------------------------- decoupled key chunk pins ---
def _key_block_of_token(g):
    """Key-block id of every latent-order token, from its grid coordinates
    and the key chunk."""
    a, b, c = g.key_chunk
    t, h, w = _coords(g, np.arange(g.seq_len))
    return ((t // a) * -(-g.H // b) + (h // b)) * -(-g.W // c) + (w // c)


# Query chunk [4, 4, 8] (128 tokens) with key chunks of 64, 256 and 1024
# tokens on a 8 x 16 x 32 grid, with and without condition frames.
_KEY_CASES = (
    (O.Geometry(8, 16, 32, ctk=2, chk=4, cwk=8), O.SelectParams("topk", k=5)),
    (O.Geometry(8, 16, 32, ctk=4, chk=8, cwk=8, cond_frames=4),
     O.SelectParams("cdf", p=0.7, k_min=1, k_max=6)),
    (O.Geometry(8, 16, 32, ctk=8, chk=8, cwk=16), O.SelectParams("topk", k=2)),
    (O.Geometry(8, 16, 32, ctk=2, chk=4, cwk=8, cond_frames=4), O.SelectParams("topk", k=7)),
    # 64-token query blocks with 64-, 128- and 256-token key blocks.
    (O.Geometry(8, 16, 32, 2, 4, 8, ctk=2, chk=4, cwk=8), O.SelectParams("topk", k=5)),
    (O.Geometry(8, 16, 32, 2, 4, 8, cond_frames=4, ctk=4, chk=4, cwk=8),
     O.SelectParams("cdf", p=0.7, k_min=1, k_max=6)),
    (O.Geometry(8, 16, 32, 4, 2, 8, ctk=4, chk=8, cwk=8), O.SelectParams("topk", k=3)),
)


def pin_key_chunk_mask_formula():
    """Decoupled key blocks: gathered attention equals the mask formula over
    the whole sequence, with each token's query block and key block computed
    from its coordinates with the two chunk shapes."""
    rng = np.random.default_rng(31)
    for g, p in _KEY_CASES:
        q, k, v = _rand(rng, g)
        scale = 1 / np.sqrt(q.shape[1])
        out, idx, cnt, _ = O.bsa_head(q, k, v, g, p, scale)
        qb, kb = _block_of_token(g), _key_block_of_token(g)
        sel = np.zeros((g.num_blocks, g.num_key_blocks), dtype=bool)
        for i in range(g.num_blocks):
            ids = idx[i, : cnt[i]]
            assert np.all(ids < O.allowed_key_blocks(g, i))
            sel[i, ids] = True
        ref = _textbook_attention(q, k, v, scale, sel[qb[:, None], kb[None, :]])
        assert np.abs(out - ref).max() < 1e-12, "gathered attention != masked attention"


def pin_key_chunk_pooled_bruteforce():
    """Decoupled key blocks: pooled scores from coordinate accumulation, query
    blocks with the query chunk and key blocks with the key chunk; condition
    rows see exactly the key blocks made of condition frames."""
    rng = np.random.default_rng(32)
    for g, _ in _KEY_CASES:
        q, k, _ = _rand(rng, g)
        scale = 0.29
        qb, kb = _block_of_token(g), _key_block_of_token(g)
        qs = np.zeros((g.num_blocks, q.shape[1]))
        ks = np.zeros((g.num_key_blocks, k.shape[1]))
        np.add.at(qs, qb, q)
        np.add.at(ks, kb, k)
        qs /= np.bincount(qb)[:, None]
        ks /= np.bincount(kb)[:, None]
        s_ref = qs @ ks.T * scale
        _, _, scores = O.select_head(q, k, g, O.SelectParams("topk", k=1), scale)
        assert scores.shape == (g.num_blocks, g.num_key_blocks)
        t = _coords(g, np.arange(g.seq_len))[0]
        cond_kb = np.unique(kb[t < g.cond_frames]) if g.cond_frames else np.array([], int)
        for i in range(g.num_blocks):
            na = O.allowed_key_blocks(g, i)
            if g.cond_frames and i < g.cond_blocks:
                assert np.array_equal(np.arange(na), cond_kb)
            else:
                assert na == g.num_key_blocks
            assert np.abs(scores[i, :na] - s_ref[i, :na]).max() < 1e-12
            assert np.all(np.isneginf(scores[i, na:]))


def pin_key_chunk_dense():
    """Decoupled key blocks: keeping every allowed key block gives textbook
    attention (block-causal over the token sets when there are condition
    frames), whatever the key chunk."""
    rng = np.random.default_rng(33)
    for g, _ in _KEY_CASES:
        q, k, v = _rand(rng, g)
        scale = 0.23
        out, idx, cnt, _ = O.bsa_head(q, k, v, g, O.SelectParams("topk", k=g.num_key_blocks), scale)
        cond = _coords(g, np.arange(g.seq_len))[0] < g.cond_frames
        ref = np.zeros_like(q)
        if cond.any():
            ref[cond] = _textbook_attention(q[cond], k[cond], v[cond], scale)
        ref[~cond] = _textbook_attention(q[~cond], k, v, scale)
        assert np.abs(out - ref).max() < 1e-12
        assert np.abs(O.dense_head(q, k, v, g, scale) - ref).max() < 1e-12


def pin_key_chunk_backward_autograd():
    """Decoupled key blocks: backward_head equals torch float64 autograd of
    the mask formula (token-level mask from both chunk shapes)."""
    import torch

    rng = np.random.default_rng(34)
    g = O.Geometry(4, 8, 16, ctk=4, chk=4, cwk=4)  # 128-token queries, 64-token keys
    q, k, v, do = (rng.standard_normal((g.seq_len, 8)) for _ in range(4))
    nk = g.num_key_blocks
    idx = np.array([[0, 3, 6, -1], [1, 2, 5, 7], [4, -1, -1, -1], [0, 1, 6, 7]])
    cnt = np.array([3, 4, 1, 4])
    scale = 0.31
    dq, dk, dv = O.backward_head(q, k, v, do, g, idx, cnt, scale)
    sel = np.zeros((g.num_blocks, nk), dtype=bool)
    for i in range(g.num_blocks):
        sel[i, idx[i, : cnt[i]]] = True
    allowed = torch.tensor(sel[_block_of_token(g)[:, None], _key_block_of_token(g)[None, :]])
    tq, tk, tv = (torch.tensor(a, dtype=torch.float64, requires_grad=True) for a in (q, k, v))
    logits = ((tq @ tk.T) * scale).masked_fill(~allowed, float("-inf"))
    out = torch.softmax(logits, dim=1) @ tv
    (out * torch.tensor(do)).sum().backward()
    for mine, ref in ((dq, tq.grad), (dk, tk.grad), (dv, tv.grad)):
        assert np.abs(mine - ref.numpy()).max() < 1e-10


# ------------------------------------------------------ partial block pins ---
# Grids that a chunk does not divide: [DeepDive] "3D block partitioning"
# counts blocks with ceilings, so the last block along such an axis is cut
# at the grid's edge and holds fewer tokens.
_PARTIAL_CASES = (
    # 2 x 2 x 2 blocks of [4, 4, 8], every axis cut.
    (O.Geometry(6, 6, 12), O.SelectParams("topk", k=3)),
    # t and h cut, condition frames.
    (O.Geometry(10, 7, 16, cond_frames=4), O.SelectParams("cdf", p=0.7, k_min=1, k_max=5)),
    # 64-token query blocks and 256-token key blocks, both cut along t and w.
    (O.Geometry(5, 8, 13, 2, 4, 8, ctk=4, chk=4, cwk=16), O.SelectParams("topk", k=4)),
    # 64-token key blocks cut along h and w.
    (O.Geometry(6, 9, 20, ctk=2, chk=4, cwk=8), O.SelectParams("topk", k=6)),
)


def pin_partial_block_order():
    """Partial grids: the slots inside the grid hold every token once; each
    token sits in the block and slot that its coordinates give, and the
    remaining slots (outside the grid) are marked -1."""
    for g, _ in _PARTIAL_CASES:
        for gg in (g, O.key_geometry(g)):
            perm = O.block_token_order(gg)
            assert perm.shape == (gg.num_blocks * gg.n,)
            valid = perm >= 0
            assert np.array_equal(np.sort(perm[valid]), np.arange(gg.seq_len)), "not a bijection"
            pos = np.nonzero(valid)[0]
            tok = perm[valid]
            t, h, w = _coords(gg, tok)
            assert np.array_equal(pos // gg.n, _block_of_token(gg)[tok]), "token in the wrong block"
            slot = ((t % gg.ct) * gg.ch + (h % gg.ch)) * gg.cw + (w % gg.cw)
            assert np.array_equal(pos % gg.n, slot), "token in the wrong slot"
            assert int((~valid).sum()) == gg.num_blocks * gg.n - gg.seq_len


def pin_partial_mask_formula():
    """Partial grids: gathered attention equals the token-level mask formula,
    with every token's query and key block from its coordinates."""
    rng = np.random.default_rng(41)
    for g, p in _PARTIAL_CASES:
        q, k, v = _rand(rng, g)
        scale = 1 / np.sqrt(q.shape[1])
        out, idx, cnt, _ = O.bsa_head(q, k, v, g, p, scale)
        qb, kb = _block_of_token(g), _key_block_of_token(g)
        sel = np.zeros((g.num_blocks, g.num_key_blocks), dtype=bool)
        for i in range(g.num_blocks):
            sel[i, idx[i, : cnt[i]]] = True
        ref = _textbook_attention(q, k, v, scale, sel[qb[:, None], kb[None, :]])
        assert np.abs(out - ref).max() < 1e-12, "gathered attention != masked attention"
        dense_ref = np.zeros_like(q)
        cond = _coords(g, np.arange(g.seq_len))[0] < g.cond_frames
        if cond.any():
            dense_ref[cond] = _textbook_attention(q[cond], k[cond], v[cond], scale)
        dense_ref[~cond] = _textbook_attention(q[~cond], k, v, scale)
        assert np.abs(O.dense_head(q, k, v, g, scale) - dense_ref).max() < 1e-12


def pin_partial_pooled_bruteforce():
    """Partial grids: pooled scores from coordinate accumulation divided by
    each block's own token count."""
    rng = np.random.default_rng(42)
    for g, _ in _PARTIAL_CASES:
        q, k, _ = _rand(rng, g)
        scale = 0.31
        qb, kb = _block_of_token(g), _key_block_of_token(g)
        qs = np.zeros((g.num_blocks, q.shape[1]))
        ks = np.zeros((g.num_key_blocks, k.shape[1]))
        np.add.at(qs, qb, q)
        np.add.at(ks, kb, k)
        qs /= np.bincount(qb, minlength=g.num_blocks)[:, None]
        ks /= np.bincount(kb, minlength=g.num_key_blocks)[:, None]
        s_ref = qs @ ks.T * scale
        _, _, scores = O.select_head(q, k, g, O.SelectParams("topk", k=1), scale)
        for i in range(g.num_blocks):
            na = O.allowed_key_blocks(g, i)
            assert np.abs(scores[i, :na] - s_ref[i, :na]).max() < 1e-12, "pooled score"


def pin_partial_closed_forms():
    """Partial grids, closed forms. (1) A channel holding each token's frame
    index pools to bt*t + (r - 1)/2 for a block whose box keeps r frames of
    the grid (the mean of r consecutive integers), whatever its h and w cut.
    (2) Q = 0 ties every pooled score, so top-k keeps key blocks 0..k-1 and
    every query's output is the mean of V over exactly the tokens of those
    blocks."""
    rng = np.random.default_rng(43)
    for g, _ in _PARTIAL_CASES:
        t = _coords(g, np.arange(g.seq_len))[0].astype(np.float64)
        x = np.zeros((g.seq_len, 2))
        x[:, 0] = t
        x[:, 1] = 1.0
        pooled = O.pool_blocks(x, O.block_token_order(g), g.n)
        for i in range(g.num_blocks):
            bt = i // (g.nH * g.nW)
            r = min(g.ct, g.T - bt * g.ct)
            assert abs(pooled[i, 0] - (bt * g.ct + (r - 1) / 2)) < 1e-12
            assert abs(pooled[i, 1] - 1.0) < 1e-12
        _, k, v = _rand(rng, g)
        q = np.zeros_like(k)
        kk = 3
        out, idx, cnt, _ = O.bsa_head(q, k, v, g, O.SelectParams("topk", k=kk), 0.2)
        kb = _key_block_of_token(g)
        for i in range(g.num_blocks):
            na = O.allowed_key_blocks(g, i)
            want = list(range(min(kk, na)))
            assert idx[i, : cnt[i]].tolist() == want
            mean_v = v[np.isin(kb, want)].mean(axis=0)
            assert np.abs(out[_block_of_token(g) == i] - mean_v).max() < 1e-12


def pin_partial_backward_autograd():
    """Partial grids: backward_head equals torch float64 autograd of the
    token-level mask formula, for random selections."""
    import torch

    rng = np.random.default_rng(44)
    for g, _ in _PARTIAL_CASES:
        q, k, v, do = (rng.standard_normal((g.seq_len, 8)) for _ in range(4))
        nb, nk = g.num_blocks, g.num_key_blocks
        stride = min(3, nk)
        idx = np.full((nb, stride), -1)
        cnt = np.zeros(nb, dtype=np.int64)
        for i in range(nb):
            c = int(rng.integers(1, stride + 1))
            idx[i, :c] = np.sort(rng.choice(nk, size=c, replace=False))
            cnt[i] = c
        scale = 0.33
        dq, dk, dv = O.backward_head(q, k, v, do, g, idx, cnt, scale)
        sel = np.zeros((nb, nk), dtype=bool)
        for i in range(nb):
            sel[i, idx[i, : cnt[i]]] = True
        allowed = torch.tensor(sel[_block_of_token(g)[:, None], _key_block_of_token(g)[None, :]])
        tq, tk, tv = (torch.tensor(a, dtype=torch.float64, requires_grad=True) for a in (q, k, v))
        logits = ((tq @ tk.T) * scale).masked_fill(~allowed, float("-inf"))
        out = torch.softmax(logits, dim=1) @ tv
        (out * torch.tensor(do)).sum().backward()
        for mine, ref in ((dq, tq.grad), (dk, tk.grad), (dv, tv.grad)):
            assert np.abs(mine - ref.numpy()).max() < 1e-10


# ------------------------------------------------------ bf16 widening ---
def _bf16_by_format(bits: int) -> float:
    """Value of a bfloat16 bit pattern from the format's definition: 1 sign
    bit, 8 exponent bits with bias 127 and 7 fraction bits (the upper half of
    an IEEE-754 binary32). Written from the field layout, not by shifting into
    a float32."""
    sign = -1.0 if bits >> 15 else 1.0
    e = (bits >> 7) & 0xFF
    f = bits & 0x7F
    if e == 0xFF:
        return sign * float("inf") if f == 0 else float("nan")
    if e == 0:  # subnormal: 2^-126 * f/128
        return sign * math.ldexp(f, -126 - 7)
    return sign * math.ldexp(128 + f, e - 127 - 7)


def pin_bf16_widening():
    """bf16_bits_to_f64 against values the bfloat16 format fixes: hand-worked
    patterns, then all 65,536 patterns against the field-by-field definition
    (NaN patterns must widen to NaN, -0 must keep its sign)."""
    known = {
        0x3F80: 1.0, 0xBF80: -1.0, 0x4000: 2.0, 0xC000: -2.0, 0x3F00: 0.5,
        0xC049: -3.140625,            # -(1 + 73/128) * 2
        0x0001: 2.0 ** -133,          # smallest subnormal
        0x807F: -(127 / 128) * 2.0 ** -126,  # largest negative subnormal
        0x0080: 2.0 ** -126,          # smallest normal
        0x7F7F: (2 - 2.0 ** -7) * 2.0 ** 127,  # largest finite
        0x7F80: math.inf, 0xFF80: -math.inf,
    }
    got = O.bf16_bits_to_f64(np.array(list(known), dtype=np.uint16))
    for (bits, want), val in zip(known.items(), got):
        assert val == want, f"0x{bits:04X}: {val!r} != {want!r}"
    nz = O.bf16_bits_to_f64(np.array([0x8000, 0x0000], dtype=np.uint16))
    assert nz[0] == 0.0 and math.copysign(1.0, nz[0]) == -1.0, "0x8000 must widen to -0.0"
    assert math.copysign(1.0, nz[1]) == 1.0, "0x0000 must widen to +0.0"
    for bits in (0x7FC0, 0xFFC1, 0x7F81):
        assert math.isnan(O.bf16_bits_to_f64(np.array([bits], dtype=np.uint16))[0])
    allbits = np.arange(1 << 16, dtype=np.uint32).astype(np.uint16)
    wide = O.bf16_bits_to_f64(allbits)
    assert wide.dtype == np.float64 and wide.shape == (1 << 16,)
    ref = np.array([_bf16_by_format(int(b)) for b in allbits], dtype=np.float64)
    nan = np.isnan(ref)
    assert np.array_equal(np.isnan(wide), nan)
    assert np.array_equal(wide[~nan], ref[~nan])
    assert np.array_equal(np.signbit(wide[~nan]), np.signbit(ref[~nan]))
    # A 2-D array keeps its shape (the oracle widens [S, d] tensors).
    assert O.bf16_bits_to_f64(np.full((3, 5), 0x3F80, dtype=np.uint16)).shape == (3, 5)


ALL_PINS = [
    pin_bf16_widening,
    pin_block_order_geometry,
    pin_handworked_golden,
    pin_dense_equals_textbook,
    pin_mask_formula,
    pin_pooled_scores_bruteforce,
    pin_topk_property,
    pin_cdf_property,
    pin_rows_sum_to_one,
    pin_constant_v,
    pin_q_zero,
    pin_intra_block_shuffle,
    pin_block_causal_independence,
    pin_block_causal_dense_definition,
    pin_monotonic,
    pin_backward_finite_differences,
    pin_backward_dense_autograd,
    pin_backward_constant_v,
    pin_backward_dv_total,
    pin_forward_lse,
    pin_backward_query_block_subset,
    pin_key_chunk_mask_formula,
    pin_key_chunk_pooled_bruteforce,
    pin_key_chunk_dense,
    pin_key_chunk_backward_autograd,
    pin_partial_block_order,
    pin_partial_mask_formula,
    pin_partial_pooled_bruteforce,
    pin_partial_closed_forms,
    pin_partial_backward_autograd,
]
