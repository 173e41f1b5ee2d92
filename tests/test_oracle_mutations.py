"""Plant plausible mistakes in the oracle (on the CPU) and check that at
least one pin catches each of them. Shows the pins are strong enough to
notice a dropped term, a wrong index, a transposed operand or a wrong rule."""

import numpy as np
import pytest

import oracle.bsa_oracle as O
import oracle_pins as P

_orig_attend = O.attend_query_block
_orig_order = O.block_token_order
_orig_pool = O.pool_blocks
_orig_cdf = O.select_cdf
_orig_lse = O.forward_lse_head
_orig_bf16 = O.bf16_bits_to_f64


def _bf16_shift15(bits):
    u32 = np.asarray(bits, dtype=np.uint16).astype(np.uint32) << np.uint32(15)
    return u32.view(np.float32).astype(np.float64)


def _bf16_as_float16(bits):
    return np.asarray(bits, dtype=np.uint16).view(np.float16).astype(np.float64)


def _bf16_sign_dropped(bits):
    return np.abs(_orig_bf16(bits))


def _bf16_low_half(bits):
    return np.asarray(bits, dtype=np.uint16).astype(np.uint32).view(np.float32).astype(np.float64)


def _attend_no_scale(q, k, v, g, i, key_blocks, scale, perm=None, kperm=None):
    return _orig_attend(q, k, v, g, i, key_blocks, 1.0, perm, kperm)


def _attend_keys_as_values(q, k, v, g, i, key_blocks, scale, perm=None, kperm=None):
    return _orig_attend(q, k, k, g, i, key_blocks, scale, perm, kperm)


def _order_hw_swapped(g):
    perm = np.empty(g.seq_len, dtype=np.int64)
    pos = 0
    for bt in range(g.nT):
        for bh in range(g.nH):
            for bw in range(g.nW):
                for it in range(g.ct):
                    for iw in range(g.cw):
                        for ih in range(g.ch):
                            perm[pos] = ((bt * g.ct + it) * g.H + bh * g.ch + ih) * g.W + bw * g.cw + iw
                            pos += 1
    return perm


def _order_blocks_w_major(g):
    perm = _orig_order(g)
    n = g.n
    blocks = perm.reshape(g.nT, g.nH, g.nW, n).transpose(0, 2, 1, 3)
    return blocks.reshape(-1).copy()


def _pool_sum(x, perm, n):
    return _orig_pool(x, perm, n) * n


def _pool_first_token(x, perm, n):
    xb = np.asarray(x, dtype=np.float64)[perm]
    return xb.reshape(-1, n, xb.shape[-1])[:, 0, :].copy()


def _pool_zero_padded(x, perm, n):
    """Partial blocks padded with zeros and divided by n."""
    x = np.asarray(x, dtype=np.float64)
    xb = np.where((perm >= 0)[:, None], x[np.maximum(perm, 0)], 0.0)
    return xb.reshape(-1, n, x.shape[-1]).sum(axis=1) / n


def _tokens_keep_outside(perm, i, n):
    """Slots outside the grid not dropped (-1 then indexes the last token)."""
    return perm[i * n : (i + 1) * n]


def _attend_zero_padded_keys(q, k, v, g, i, key_blocks, scale, perm=None, kperm=None):
    """Slots of a partial key block outside the grid attended as zero keys
    and values."""
    perm = O.block_token_order(g) if perm is None else perm
    kperm = O.block_token_order(O.key_geometry(g)) if kperm is None else kperm
    n, nk = g.n, g.nk
    qi = np.asarray(q, np.float64)[O.block_tokens(perm, i, n)]
    tok = np.concatenate([kperm[j * nk : (j + 1) * nk] for j in key_blocks])
    pad = (tok < 0)[:, None]
    ks = np.where(pad, 0.0, np.asarray(k, np.float64)[np.maximum(tok, 0)])
    vs = np.where(pad, 0.0, np.asarray(v, np.float64)[np.maximum(tok, 0)])
    logits = (qi @ ks.T) * scale
    logits -= logits.max(axis=1, keepdims=True)
    w = np.exp(logits)
    w /= w.sum(axis=1, keepdims=True)
    return w @ vs


def _rank_ties_high(values):
    ids = np.arange(values.shape[0])
    return np.lexsort((-ids, -values))


def _cdf_drop_crossing(scores_row, n_allowed, p, k_min, k_max):
    probs = O.softmax_allowed(scores_row, n_allowed)
    order = O._rank_order(probs)
    cum = np.cumsum(probs[order])
    reached = np.nonzero(cum >= p)[0]
    count = int(reached[0]) if reached.size else n_allowed
    count = min(max(count, k_min), min(k_max, n_allowed))
    return np.sort(order[:count])


def _cdf_no_clamp(scores_row, n_allowed, p, k_min, k_max):
    return _orig_cdf(scores_row, n_allowed, p, 1, n_allowed)


def _topk_lowest(scores_row, n_allowed, k):
    order = np.lexsort((np.arange(n_allowed), np.asarray(scores_row[:n_allowed])))
    return np.sort(order[: min(k, n_allowed)])


def _scores_unscaled(q_pool, k_pool, scale):
    return q_pool @ k_pool.T


def _scores_transposed(q_pool, k_pool, scale):
    return (k_pool @ q_pool.T) * scale


def _backward_variant(mistake):
    """backward_head with one planted mistake."""

    def fn(q, k, v, do, g, idx, cnt, scale, query_blocks=None):
        perm = O.block_token_order(g)
        q, k, v, do = (np.asarray(a, np.float64) for a in (q, k, v, do))
        dq, dk, dv = np.zeros_like(q), np.zeros_like(k), np.zeros_like(v)
        n = g.n
        for i in range(g.num_blocks) if query_blocks is None else sorted(set(query_blocks)):
            blocks = [int(j) for j in idx[i, : cnt[i]]]
            if not blocks:
                continue
            qt = perm[i * n : (i + 1) * n]
            kt = np.concatenate([perm[j * n : (j + 1) * n] for j in blocks])
            logits = (q[qt] @ k[kt].T) * scale
            logits -= logits.max(axis=1, keepdims=True)
            p = np.exp(logits)
            p /= p.sum(axis=1, keepdims=True)
            o = p @ v[kt]
            delta = (do[qt] * o).sum(axis=1, keepdims=True)
            dp = do[qt] @ v[kt].T
            ds = p * dp if mistake == "no delta" else p * (dp - delta)
            kk = v[kt] if mistake == "dq from v" else k[kt]
            dq[qt] += scale * (ds @ kk)
            sk = 1.0 if mistake == "dk unscaled" else scale
            np.add.at(dk, kt, sk * (ds.T @ q[qt]))
            pv = p if mistake == "dv from p" else p.T
            np.add.at(dv, kt, pv @ do[qt])
        return dq, dk, dv

    return fn


def _lse_without_max(q, k, v, g, idx, cnt, scale, query_blocks=None):
    out, lse = _orig_lse(q, k, v, g, idx, cnt, scale, query_blocks=query_blocks)
    perm = O.block_token_order(g)
    n = g.n
    for i in range(g.num_blocks) if query_blocks is None else sorted(set(query_blocks)):
        blocks = [int(j) for j in idx[i, : cnt[i]]]
        if blocks:
            qt = perm[i * n : (i + 1) * n]
            kt = np.concatenate([perm[j * n : (j + 1) * n] for j in blocks])
            s = (np.asarray(q)[qt] @ np.asarray(k)[kt].T) * scale
            lse[qt] -= s.max(axis=1)
    return out, lse


MUTANTS = {
    "bf16 widened with a 15-bit shift": ("bf16_bits_to_f64", _bf16_shift15),
    "bf16 read as float16": ("bf16_bits_to_f64", _bf16_as_float16),
    "bf16 sign dropped": ("bf16_bits_to_f64", _bf16_sign_dropped),
    "bf16 placed in the low half of a float32": ("bf16_bits_to_f64", _bf16_low_half),
    "attention scale dropped": ("attend_query_block", _attend_no_scale),
    "keys used as values": ("attend_query_block", _attend_keys_as_values),
    "intra-block order h/w swapped": ("block_token_order", _order_hw_swapped),
    "block order w before h": ("block_token_order", _order_blocks_w_major),
    "pool sums instead of means": ("pool_blocks", _pool_sum),
    "pool takes first token only": ("pool_blocks", _pool_first_token),
    "partial blocks pooled as zero-padded means": ("pool_blocks", _pool_zero_padded),
    "slots outside the grid kept": ("block_tokens", _tokens_keep_outside),
    "partial key blocks padded with zero keys": ("attend_query_block", _attend_zero_padded_keys),
    "ties go to higher ids": ("_rank_order", _rank_ties_high),
    "CDF drops the crossing block": ("select_cdf", _cdf_drop_crossing),
    "CDF ignores k_min/k_max": ("select_cdf", _cdf_no_clamp),
    "top-k keeps the lowest scores": ("select_topk", _topk_lowest),
    "pooled score scale dropped": ("pooled_scores", _scores_unscaled),
    "pooled scores transposed": ("pooled_scores", _scores_transposed),
    "block-causal ignored": ("allowed_key_blocks", lambda g, i: g.num_blocks),
    "noisy rows restricted too": ("allowed_key_blocks",
                                  lambda g, i: g.cond_blocks if g.cond_frames else g.num_blocks),
    "backward drops the softmax Jacobian's row term": ("backward_head", _backward_variant("no delta")),
    "backward dQ uses V": ("backward_head", _backward_variant("dq from v")),
    "backward dK unscaled": ("backward_head", _backward_variant("dk unscaled")),
    "backward dV from P instead of P^T": ("backward_head", _backward_variant("dv from p")),
    "lse without the max": ("forward_lse_head", _lse_without_max),
    "keys cut with the query chunk": (
        "key_geometry", lambda g: O.Geometry(g.T, g.H, g.W, g.ct, g.ch, g.cw, g.cond_frames)),
    "condition key blocks counted in query blocks": (
        "allowed_key_blocks",
        lambda g, i: g.cond_blocks if (g.cond_frames and i < g.cond_blocks) else g.num_key_blocks),
}


@pytest.mark.parametrize("name", list(MUTANTS))
def test_mutant_is_caught(name, monkeypatch):
    attr, fn = MUTANTS[name]
    monkeypatch.setattr(O, attr, fn)
    caught = []
    for pin in P.ALL_PINS:
        try:
            pin()
        except (AssertionError, ValueError, IndexError):
            caught.append(pin.__name__)
    assert caught, f"no pin noticed the planted mistake: {name}"
