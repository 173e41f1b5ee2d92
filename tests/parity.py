"""Helpers for the GPU-vs-oracle parity tests: device marshalling through the
C ABI binding, the oracle run per head, and the comparison rules.

Acceptance rules
* Index sets must equal the oracle's. A difference is accepted only as a
  near-tie: every id that differs scores within 1e-5 of the oracle's last
  kept score, and the GPU set is itself a valid top set (nothing left out
  scores more than 1e-5 above anything kept). In CDF mode a different count
  is accepted only if some raw count whose prefix mass is within 1e-5 of p
  clamps to it.
* Outputs: max-abs <= 2e-2 and mean-abs <= 1e-3 against the oracle's output
  for the GPU's own (validated) key-block set.
"""

from __future__ import annotations

from concurrent.futures import ThreadPoolExecutor

import numpy as np

import oracle.bsa_oracle as O

TIE_TOL = 1e-5
MAX_ABS = 2e-2
MEAN_ABS = 1e-3


# ------------------------------------------------------------ device side ---
def to_device(bits):
    import torch

    return torch.from_numpy(np.ascontiguousarray(bits)).view(torch.bfloat16).cuda()


def from_device(t):
    import torch

    return t.view(torch.int16).cpu().numpy().view(np.uint16)


def run_select(problem, params, q_d, k_d):
    import torch

    from video_dit_block_bsa_amd import binding as B

    stride = B.index_stride(problem, params)
    rows = problem.batch * problem.heads * problem.num_blocks
    idx = torch.full((max(rows, 1), stride), -7, dtype=torch.int32, device="cuda")
    cnt = torch.full((max(rows, 1),), -7, dtype=torch.int32, device="cuda")
    ws = torch.empty(max(B.select_workspace_bytes(problem, params), 1), dtype=torch.uint8,
                     device="cuda")
    B.bsa_select(problem, params, q_d, k_d, idx, cnt, ws)
    torch.cuda.synchronize()
    return idx, cnt


def run_attention(problem, q_d, k_d, v_d, idx, cnt, stride):
    import torch

    from video_dit_block_bsa_amd import binding as B

    o = torch.full_like(q_d, float("nan"))
    ws = torch.empty(max(B.attention_workspace_bytes(problem), 1), dtype=torch.uint8,
                     device="cuda")
    B.bsa_attention(problem, q_d, k_d, v_d, idx, cnt, stride, o, ws)
    torch.cuda.synchronize()
    return o


def run_dense(problem, q_d, k_d, v_d):
    import torch

    from video_dit_block_bsa_amd import binding as B

    o = torch.full_like(q_d, float("nan"))
    ws = torch.empty(max(B.attention_workspace_bytes(problem), 1), dtype=torch.uint8,
                     device="cuda")
    B.dense_attention(problem, q_d, k_d, v_d, o, ws)
    torch.cuda.synchronize()
    return o


# ------------------------------------------------------------ oracle side ---
def geometry(problem) -> O.Geometry:
    return O.Geometry(problem.T, problem.H, problem.W, problem.ct, problem.ch, problem.cw,
                      problem.cond_frames, problem.ctk, problem.chk, problem.cwk)


def oracle_params(params) -> O.SelectParams:
    if params.mode == 0:
        return O.SelectParams("topk", k=params.k)
    return O.SelectParams("cdf", p=float(params.cdf_p), k_min=params.k_min, k_max=params.k_max)


def oracle_select_all(q_bits, k_bits, g, sp, scale, threads=8):
    """Oracle selection for every (batch, head): lists of (idx, cnt, scores)."""
    B, Hh = q_bits.shape[:2]
    pairs = [(b, h) for b in range(B) for h in range(Hh)]

    def one(bh):
        b, h = bh
        return O.select_head(O.bf16_bits_to_f64(q_bits[b, h]), O.bf16_bits_to_f64(k_bits[b, h]),
                             g, sp, scale)

    with ThreadPoolExecutor(threads) as ex:
        return list(ex.map(one, pairs))


# ------------------------------------------------------------- comparison ---
def _valid_top(row_scores, sel, na):
    if sel.size == 0:
        return True
    rest = np.setdiff1d(np.arange(na), sel)
    if rest.size == 0:
        return True
    return row_scores[sel].min() >= row_scores[rest].max() - TIE_TOL


def check_row(gpu_ids, oracle_ids, row_scores, na, sp):
    """Returns None if the GPU row is acceptable, else a reason string."""
    g_ids = np.asarray(gpu_ids)
    if g_ids.size and (np.any(np.diff(g_ids) <= 0) or g_ids.min() < 0 or g_ids.max() >= na):
        return f"ids not ascending/in range: {g_ids.tolist()}"
    if np.array_equal(g_ids, oracle_ids):
        return None
    if not _valid_top(row_scores, g_ids, na):
        return "GPU set is not a top set"
    if sp.mode == "topk":
        if g_ids.size != oracle_ids.size:
            return f"count {g_ids.size} != {oracle_ids.size}"
        boundary = row_scores[oracle_ids].min()
        diff = np.setxor1d(g_ids, oracle_ids)
        if np.all(np.abs(row_scores[diff] - boundary) < TIE_TOL):
            return None
        return f"differs beyond near-ties: {diff.tolist()}"
    # CDF: the count must come from a raw count decided within TIE_TOL of p.
    s = row_scores[:na]
    e = np.exp(s - s.max())
    prob = e / e.sum()
    order = np.lexsort((np.arange(na), -prob))
    cum = np.concatenate([[0.0], np.cumsum(prob[order])])
    hi = min(sp.k_max, na)
    ok_counts = set()
    for c in range(1, na + 1):
        if cum[c] >= sp.p - TIE_TOL and cum[c - 1] < sp.p + TIE_TOL:
            ok_counts.add(min(max(c, sp.k_min), hi))
    if cum[na] < sp.p + TIE_TOL:
        ok_counts.add(min(max(na, sp.k_min), hi))
    if g_ids.size not in ok_counts:
        return f"CDF count {g_ids.size} not within tolerance (oracle {oracle_ids.size})"
    if g_ids.size == oracle_ids.size:
        boundary = row_scores[oracle_ids].min()
        diff = np.setxor1d(g_ids, oracle_ids)
        if not np.all(np.abs(row_scores[diff] - boundary) < TIE_TOL):
            return f"differs beyond near-ties: {diff.tolist()}"
    return None


def check_selection(idx, cnt, oracle_rows, g, sp, stride):
    """Compare GPU idx/cnt (numpy, rows ordered (batch, head, block)) with the
    oracle. Returns (exact_rows, tie_rows, failures)."""
    nb = g.num_blocks
    exact = ties = 0
    failures = []
    for pair, (oi, oc, sc) in enumerate(oracle_rows):
        for i in range(nb):
            row = pair * nb + i
            c = int(cnt[row])
            if c < 0 or c > stride:
                failures.append((pair, i, f"cnt {c} out of range"))
                continue
            if np.any(idx[row, c:] != -1):
                failures.append((pair, i, "padding is not -1"))
                continue
            na = O.allowed_key_blocks(g, i)
            why = check_row(idx[row, :c], oi[i, : oc[i]], sc[i], na, sp)
            if why is not None:
                failures.append((pair, i, why))
            elif np.array_equal(idx[row, :c], oi[i, : oc[i]]):
                exact += 1
            else:
                ties += 1
    return exact, ties, failures


def compare_outputs(out_bits, q_bits, k_bits, v_bits, g, blocks_of_pair, scale, pairs_blocks,
                    threads=8):
    """Oracle attention (float64) for the listed (pair, query block) items,
    using the key-block lists given by blocks_of_pair(pair, i). Items are
    grouped per (batch, head) so each head is widened to float64 once.
    Returns (max_abs, mean_abs, n_values)."""
    perm = O.block_token_order(g)
    kperm = O.block_token_order(O.key_geometry(g))
    n = g.n
    Hh = q_bits.shape[1]
    by_pair = {}
    for pair, i in pairs_blocks:
        by_pair.setdefault(pair, []).append(i)

    def one(pair):
        b, h = divmod(pair, Hh)
        q = O.bf16_bits_to_f64(q_bits[b, h])
        k = O.bf16_bits_to_f64(k_bits[b, h])
        v = O.bf16_bits_to_f64(v_bits[b, h])
        out = []
        for i in by_pair[pair]:
            ref = O.attend_query_block(q, k, v, g, i, blocks_of_pair(pair, i), scale, perm, kperm)
            got = O.bf16_bits_to_f64(out_bits[b, h][O.block_tokens(perm, i, n)])
            err = np.abs(got - ref)
            out.append((err.max(), err.sum(), err.size, bool(np.isfinite(got).all())))
        return out

    with ThreadPoolExecutor(threads) as ex:
        res = [r for lst in ex.map(one, list(by_pair)) for r in lst]
    assert all(r[3] for r in res), "non-finite GPU outputs"
    mx = max(r[0] for r in res)
    total = sum(r[1] for r in res)
    nvals = sum(r[2] for r in res)
    return mx, total / nvals, nvals
