"""Host-side checks of the C ABI (no GPU needed): every symbol that
include/bsa.h declares is exported, and invalid calls return the documented
status before anything is launched."""

from __future__ import annotations

import ctypes
import os
import re

import pytest

from video_dit_block_bsa_amd import binding as B

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "bsa.h")

OK, INVALID, UNSUPPORTED, WORKSPACE = 0, -1, -2, -3
FAKE = 0x10000  # never dereferenced: every call below fails validation first


def declared_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"^[A-Za-z_][\w\s\*]*?\b(\w+)\s*\(", text, flags=re.M)))


def test_header_declares_the_boundary():
    names = declared_functions()
    for must in ("bsa_select", "bsa_attention", "dense_attention"):
        assert must in names


def test_every_declared_symbol_is_exported():
    lib = B.lib()
    missing = [n for n in declared_functions() if not hasattr(lib, n)]
    assert not missing, missing


def test_status_strings():
    lib = B.lib()
    for code in (0, -1, -2, -3, -4, 7):
        assert lib.bsa_status_string(code)


def _problem(**kw):
    args = dict(T=56, H=48, W=80, heads=32)
    args.update({k: kw.pop(k) for k in list(kw) if k in args})
    return B.Problem.make(**args, **kw)


def test_workspace_sizes():
    p = _problem()
    nb = 1680
    sel = B.select_workspace_bytes(p, B.SelectParams.topk(105))
    assert sel == 2 * 32 * nb * 128 * 4  # pooled Q and K; the scores stay on chip
    assert B.attention_workspace_bytes(p) == 0
    assert B.select_workspace_bytes(_problem(head_dim=64), B.SelectParams.topk(1)) == 0
    assert B.attention_workspace_bytes(_problem(T=57)) == 0


def test_index_stride():
    p = _problem()
    assert B.index_stride(p, B.SelectParams.topk(45)) == 45
    assert B.index_stride(p, B.SelectParams.cdf(0.9, 4, 64)) == 64
    assert B.index_stride(None, B.SelectParams.cdf(0.9, 4, 64)) == 64
    assert B.index_stride(p, B.SelectParams.topk(0)) == -1
    assert B.index_stride(_problem(head_dim=64), B.SelectParams.topk(4)) == -1


def test_boundary_names_of_the_contract():
    """The hot-path contract's entry points and helpers, by name: bsa_select,
    bsa_attention, dense_attention, bsa_workspace_bytes(problem, params),
    bsa_index_stride(problem, params) and bsa_status_string. The split
    workspace helpers come on top."""
    names = declared_functions()
    for must in ("bsa_select", "bsa_attention", "dense_attention", "bsa_workspace_bytes",
                 "bsa_index_stride", "bsa_status_string", "bsa_select_workspace_bytes",
                 "bsa_attention_workspace_bytes"):
        assert must in names, must
    text = open(HEADER).read()
    assert re.search(r"int32_t bsa_index_stride\(const bsa_problem\* problem,\s*"
                     r"const bsa_select_params\* params\)", text)
    assert re.search(r"size_t bsa_workspace_bytes\(const bsa_problem\* problem,\s*"
                     r"const bsa_select_params\* params\)", text)
    p, sp = _problem(), B.SelectParams.topk(105)
    assert B.workspace_bytes(p, sp) == max(B.select_workspace_bytes(p, sp),
                                           B.attention_workspace_bytes(p))
    assert B.workspace_bytes(_problem(head_dim=64), sp) == 0


def _select(problem, params, q=FAKE, k=FAKE, idx=FAKE, cnt=FAKE, ws=FAKE, ws_bytes=1 << 40):
    lib = B.lib()
    return lib.bsa_select(ctypes.byref(problem), ctypes.byref(params), q, k, idx, cnt, ws,
                          ws_bytes, None)


def _attn(problem, q=FAKE, k=FAKE, v=FAKE, idx=FAKE, cnt=FAKE, stride=4, o=FAKE + 4096,
          ws=FAKE, ws_bytes=1 << 40):
    lib = B.lib()
    return lib.bsa_attention(ctypes.byref(problem), q, k, v, idx, cnt, stride, o, ws, ws_bytes,
                             None)


@pytest.mark.parametrize(
    "problem,code",
    [
        (dict(head_dim=64), UNSUPPORTED),
        (dict(head_dim=0), INVALID),
        (dict(chunk=(2, 4, 4)), UNSUPPORTED),   # 32-token query blocks
        (dict(chunk=(4, 8, 8)), UNSUPPORTED),   # 256-token query blocks
        (dict(cond_frames=3), INVALID),
        (dict(cond_frames=56), INVALID),
        (dict(cond_frames=-4), INVALID),
        (dict(heads=-1), INVALID),
        (dict(T=0), INVALID),
        (dict(chunk=(0, 4, 8)), INVALID),
    ],
)
def test_invalid_problem(problem, code):
    p = _problem(**problem)
    assert _select(p, B.SelectParams.topk(4)) == code
    assert _attn(p) == code
    assert B.lib().bsa_last_error()


@pytest.mark.parametrize(
    "params,code",
    [
        (B.SelectParams.topk(0), INVALID),
        (B.SelectParams.cdf(0.0, 1, 4), INVALID),
        (B.SelectParams.cdf(1.5, 1, 4), INVALID),
        (B.SelectParams.cdf(0.9, 5, 4), INVALID),
        (B.SelectParams.cdf(0.9, 0, 4), INVALID),
        (B.SelectParams(7, 1, 0.5, 1, 1), INVALID),
    ],
)
def test_invalid_params(params, code):
    assert _select(_problem(), params) == code


def test_null_and_misaligned_pointers():
    p = _problem()
    sp = B.SelectParams.topk(4)
    assert _select(p, sp, q=None) == INVALID
    assert _select(p, sp, idx=None) == INVALID
    assert _select(p, sp, k=FAKE + 2) == INVALID
    assert _attn(p, v=None) == INVALID
    assert _attn(p, o=FAKE + 8) == INVALID
    assert _attn(p, o=FAKE) == INVALID  # aliases q
    assert _attn(p, stride=0) == INVALID


def test_workspace_too_small():
    p = _problem()
    assert _select(p, B.SelectParams.topk(4), ws_bytes=1024) == WORKSPACE
    assert _select(p, B.SelectParams.topk(4), ws=None) == WORKSPACE



def test_too_many_blocks_for_selection():
    """Selection takes up to 32,768 key blocks per head (a tile's score rows
    live in 128 KB of LDS)."""
    p = _problem(T=4 * 300, H=48, W=80)  # 36,000 blocks
    assert _select(p, B.SelectParams.topk(4)) == UNSUPPORTED


def test_empty_problem_is_a_no_op():
    lib = B.lib()
    p = _problem(heads=0)
    sp = B.SelectParams.topk(4)
    assert lib.bsa_select(ctypes.byref(p), ctypes.byref(sp), None, None, None, None, None, 0, None) == OK
    assert lib.bsa_attention(ctypes.byref(p), None, None, None, None, None, 4, None, None, 0, None) == OK
    assert lib.dense_attention(ctypes.byref(p), None, None, None, None, None, 0, None) == OK


def test_binding_raises_with_message():
    p = _problem(head_dim=64)
    with pytest.raises(B.BSAError, match="head_dim"):
        B.bsa_select(p, B.SelectParams.topk(4), FAKE, FAKE, FAKE, FAKE, (FAKE, 1 << 40), stream=0)


def test_sequence_limit():
    # T*H*W must stay below 2^24 tokens (K/V of one head are addressed with
    # 32-bit byte offsets); the check happens on the host, before any launch.
    lib = B.lib()
    ok = B.Problem.make(256, 256, 248, 1)          # 16,252,928 tokens
    bad = B.Problem.make(256, 256, 256, 1)         # 2^24 tokens
    assert lib.bsa_attention_workspace_bytes(ctypes.byref(ok)) == 0
    r = lib.bsa_attention(ctypes.byref(bad), None, None, None, None, None, 1, None, None, 0, None)
    assert r == -2 and b"too long" in lib.bsa_last_error()


GiB4 = 1 << 32  # spacing of the fake tensors below: the 215K x 32-head tensors are 1.76 GB


def _bwd(p, **kw):
    """bsa_attention_bwd with fake, well-separated pointers; every call in
    the tests below is rejected by the host checks before any launch."""
    lib = B.lib()
    names = ["q", "k", "v", "o", "dout", "lse", "idx", "cnt", "dq", "dk", "dv", "ws"]
    a = {n: GiB4 * (i + 1) for i, n in enumerate(names)}
    a.update(stride=4, ws_bytes=1 << 40)
    a.update(kw)
    return lib.bsa_attention_bwd(ctypes.byref(p), a["q"], a["k"], a["v"], a["o"], a["dout"],
                                 a["lse"], a["idx"], a["cnt"], a["stride"], a["dq"], a["dk"],
                                 a["dv"], a["ws"], a["ws_bytes"], None)


def test_backward_workspace_size():
    p = _problem()
    nb, nbw = 1680, 53
    stats = 32 * nb * 256 * 4
    mask = 32 * nb * nbw * 4
    got = B.attention_bwd_workspace_bytes(p)
    assert stats + mask <= got < stats + mask + 2 * 256
    assert B.attention_bwd_workspace_bytes(_problem(head_dim=64)) == 0


def test_backward_rejects_bad_arguments():
    p = _problem()
    for name in ("q", "o", "dout", "lse", "idx", "cnt", "dq", "dk", "dv"):
        assert _bwd(p, **{name: None}) == INVALID, name
    assert _bwd(p, stride=0) == INVALID
    assert _bwd(p, dq=GiB4 * 9 + 8) == INVALID        # misaligned
    assert _bwd(p, dout=GiB4 * 5 + 4) == INVALID
    assert _bwd(p, lse=GiB4 * 6 + 2) == INVALID
    assert _bwd(p, dk=GiB4 * 9 + 4096) == INVALID     # overlaps dq
    assert _bwd(p, dv=GiB4 * 1) == INVALID            # is q
    assert _bwd(p, dq=GiB4 * 6 + 256) == INVALID      # overlaps lse
    assert _bwd(p, ws_bytes=1024) == WORKSPACE
    assert _bwd(p, ws=None) == WORKSPACE
    assert _bwd(p, ws=GiB4 * 12 + 8) == INVALID
    assert _bwd(_problem(T=4 * 100)) == UNSUPPORTED   # 12,000 blocks
    assert _bwd(_problem(head_dim=64)) == UNSUPPORTED


def test_backward_and_lse_forward_empty_problem():
    lib = B.lib()
    p = _problem(heads=0)
    assert lib.bsa_attention_bwd(ctypes.byref(p), *([None] * 8), 4, None, None, None, None, 0,
                                 None) == OK
    assert lib.bsa_attention_lse(ctypes.byref(p), None, None, None, None, None, 4, None, None,
                                 None, 0, None) == OK


def test_lse_forward_rejects_bad_lse():
    lib = B.lib()
    p = _problem()

    def call(lse, o=GiB4 * 4):
        return lib.bsa_attention_lse(ctypes.byref(p), GiB4, GiB4 * 2, GiB4 * 3, GiB4 * 5,
                                     GiB4 * 6, 4, o, lse, None, 0, None)

    assert call(None) == INVALID
    assert call(GiB4 * 7 + 2) == INVALID
    assert call(GiB4 * 4) == INVALID  # is o


def test_key_chunk_checks():
    """Key chunk: all 0 or all positive, 64..1024 tokens (powers of two),
    condition frames a multiple of ctk; selection limited to 32768 key blocks;
    the backward needs key blocks of 128 tokens or more."""
    sp = B.SelectParams.topk(4)
    ok = _problem(key_chunk=(4, 8, 8))
    nb, nbk = 1680, 840
    sel = B.select_workspace_bytes(ok, sp)
    want = 32 * nb * 512 + 32 * nbk * 512
    assert want <= sel < want + 2 * 256
    p = _problem()
    p.ctk, p.chk, p.cwk = 4, 0, 8
    assert _select(p, sp) == INVALID
    assert _select(_problem(key_chunk=(2, 2, 8)), sp) == UNSUPPORTED     # 32 tokens
    assert _select(_problem(key_chunk=(8, 16, 16)), sp) == UNSUPPORTED   # 2048 tokens
    assert _select(_problem(key_chunk=(4, 4, 12)), sp) == UNSUPPORTED    # 192 tokens
    assert _select(_problem(key_chunk=(8, 4, 8), cond_frames=4), sp) == INVALID
    assert _select(_problem(T=4 * 300, key_chunk=(2, 4, 8)), sp) == UNSUPPORTED  # 72,000 key blocks
    assert B.attention_bwd_workspace_bytes(_problem(key_chunk=(2, 4, 8))) > 0  # 64-token keys
    assert B.attention_bwd_workspace_bytes(_problem(key_chunk=(4, 8, 8))) > 0


def test_cond_cache_checks():
    p = _problem(T=16, cond_frames=4)   # 16 x 48 x 80: 480 blocks, 120 condition blocks
    assert B.cond_cache_bytes(p) == 32 * 120 * 128 * 4
    assert B.cond_cache_bytes(_problem(T=16)) == 0
    assert B.cond_cache_bytes(_problem(T=16, cond_frames=4, key_chunk=(4, 8, 8))) == 32 * 60 * 512
    lib = B.lib()
    sp = B.SelectParams.topk(4)

    def sel(cache, cache_bytes, ws_bytes=1 << 40):
        return lib.bsa_select_noisy(ctypes.byref(p), ctypes.byref(sp), GiB4, GiB4 * 2, cache,
                                    cache_bytes, GiB4 * 3, GiB4 * 4, GiB4 * 5, ws_bytes, None)

    assert sel(None, 0) == INVALID                         # condition rows need the cache
    assert sel(GiB4 * 6, 1024) == WORKSPACE                # cache too small
    assert sel(GiB4 * 6 + 8, 1 << 30) == INVALID           # misaligned
    assert sel(GiB4 * 6, 1 << 30, ws_bytes=16) == WORKSPACE
    assert lib.bsa_pool_cond_keys(ctypes.byref(p), GiB4, None, 0, None) == INVALID
    assert lib.bsa_pool_cond_keys(ctypes.byref(p), GiB4, GiB4 * 2, 64, None) == WORKSPACE
    q0 = _problem(heads=0, cond_frames=4)
    assert lib.bsa_attention_noisy(ctypes.byref(q0), None, None, None, None, None, 4, None, None,
                                   0, None) == OK


def test_query_chunk_of_64():
    """64-token query blocks are accepted by selection, attention and the
    backward (up to 4,096 query blocks per head)."""
    p = _problem(chunk=(2, 4, 8))          # 3,360 query blocks
    sp = B.SelectParams.topk(4)
    assert B.select_workspace_bytes(p, sp) > 0
    assert B.attention_bwd_workspace_bytes(p) > 0
    assert _bwd(_problem(T=4 * 40, chunk=(2, 4, 8))) == UNSUPPORTED  # 9,600 query blocks
    assert _select(_problem(T=4 * 300, chunk=(2, 4, 8)), sp) == UNSUPPORTED  # 36,000 key blocks


def test_partial_grids():
    """Grids a chunk does not divide have ceil(T/t) x ceil(H/h) x ceil(W/w)
    blocks, the last ones cut at the edge: the selection workspace is sized
    for them and for the backward's workspace."""
    sp = B.SelectParams.topk(4)
    p = _problem(T=57)                       # 15 x 12 x 10 blocks, the last t-row cut
    nb = 15 * 12 * 10
    assert p.num_blocks == nb
    sel = B.select_workspace_bytes(p, sp)
    want = 32 * nb * 512 * 2
    assert want <= sel < want + 2 * 256
    q = _problem(T=56, key_chunk=(4, 4, 64))   # W = 80: key blocks 4 x 4 x 64, the last w cut
    assert q.num_key_blocks == 14 * 12 * 2
    assert B.select_workspace_bytes(q, sp) > 0
    assert B.attention_bwd_workspace_bytes(p) == B.attention_bwd_workspace_bytes(_problem(T=60))


def test_binding_checks_tensors_before_the_library():
    """The binding rejects a wrong dtype, a non-contiguous view, too few
    elements and a host tensor before any pointer reaches the library (which
    cannot see sizes or strides). Runs on the CPU: every call fails in the
    binding's own checks."""
    import torch

    p = B.Problem.make(8, 8, 16, 2)  # 1024 tokens, 8 blocks, 2 heads
    n = 2 * 1024 * 128
    good = torch.empty(n, dtype=torch.bfloat16)
    sp = B.SelectParams.topk(2)
    idx = torch.empty(16 * 2, dtype=torch.int32)
    cnt = torch.empty(16, dtype=torch.int32)
    cases = [
        ("q must be torch.bfloat16", dict(q=torch.empty(n, dtype=torch.float16))),
        ("q must be contiguous", dict(q=torch.empty(2 * n, dtype=torch.bfloat16)[::2])),
        ("needs at least", dict(q=torch.empty(n - 1, dtype=torch.bfloat16))),
        ("must be on a GPU", dict(q=good)),
    ]
    for msg, kw in cases:
        args = dict(q=good, k=good, v=good, o=good)
        args.update(kw)
        with pytest.raises(B.BSAError, match=msg):
            B.bsa_attention(p, args["q"], args["k"], args["v"], idx, cnt, 2, args["o"],
                            (0, 0), stream=0)
    with pytest.raises(B.BSAError, match="idx must be torch.int32"):
        B.bsa_select(p, sp, FAKE, FAKE, idx.to(torch.int64), cnt, (0, 0), stream=0)
    with pytest.raises(B.BSAError, match="idx holds 31 elements"):
        B.bsa_select(p, sp, FAKE, FAKE, idx[:31], cnt, (0, 0), stream=0)
    with pytest.raises(B.BSAError, match="cnt holds"):
        B.bsa_attention(p, FAKE, FAKE, FAKE, FAKE, cnt[:15], 2, FAKE, (0, 0), stream=0)
    with pytest.raises(B.BSAError, match="lse must be torch.float32"):
        B.bsa_attention_lse(p, FAKE, FAKE, FAKE, FAKE, FAKE, 2, FAKE,
                            torch.empty(2048, dtype=torch.float64), (0, 0), stream=0)


def test_noalloc_select_checks_on_the_host():
    """bsa_select_noalloc validates like bsa_select and rejects a problem
    whose workspace exceeds its static scratch before touching a device."""
    lib = B.lib()
    sp = B.SelectParams.topk(105)
    cap = B.select_noalloc_max_workspace_bytes()
    assert cap == 64 << 20
    big = _problem(batch=4)
    assert B.select_workspace_bytes(big, sp) > cap
    call = lambda p, s=sp: lib.bsa_select_noalloc(ctypes.byref(p), ctypes.byref(s), FAKE, FAKE,
                                                  FAKE, FAKE, None)
    assert call(big) == WORKSPACE
    assert b"static scratch" in lib.bsa_last_error()
    assert call(_problem(head_dim=64)) == UNSUPPORTED
    assert call(_problem(), B.SelectParams.topk(0)) == INVALID
    assert call(_problem(heads=0)) == OK
