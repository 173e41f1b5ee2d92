"""ctypes binding over libbsa.so (C ABI in include/bsa.h).

Argument marshalling only: every function here turns Python objects into
the pointers and sizes of the C entry point of the same name and raises
``BSAError`` on a non-OK status. Torch tensors are checked first (dtype,
contiguous layout, GPU device, enough elements for the problem), because
the library receives bare pointers and cannot see sizes or strides. Device buffers may be torch tensors (their
``data_ptr()`` is passed) or raw integer device addresses. ``stream`` is a
``torch.cuda.Stream``, a raw hipStream_t integer, or None for torch's current
stream. The library must have been built (``python -m
video_dit_block_bsa_amd.build``); nothing here falls back to other code.
"""

from __future__ import annotations

import ctypes
import os

_LIB_PATH = os.path.join(os.path.dirname(os.path.abspath(__file__)), "libbsa.so")

BSA_TOPK = 0
BSA_CDF = 1


def _cdiv(a, b):
    return -(-a // b)


class Problem(ctypes.Structure):
    """Mirror of ``bsa_problem``."""

    _fields_ = [
        ("batch", ctypes.c_int32),
        ("heads", ctypes.c_int32),
        ("head_dim", ctypes.c_int32),
        ("T", ctypes.c_int32),
        ("H", ctypes.c_int32),
        ("W", ctypes.c_int32),
        ("ct", ctypes.c_int32),
        ("ch", ctypes.c_int32),
        ("cw", ctypes.c_int32),
        ("cond_frames", ctypes.c_int32),
        ("scale", ctypes.c_float),
        ("ctk", ctypes.c_int32),
        ("chk", ctypes.c_int32),
        ("cwk", ctypes.c_int32),
    ]

    @classmethod
    def make(cls, T, H, W, heads, batch=1, head_dim=128, chunk=(4, 4, 8), cond_frames=0,
             scale=0.0, key_chunk=None):
        kc = tuple(key_chunk) if key_chunk else (0, 0, 0)
        return cls(batch, heads, head_dim, T, H, W, chunk[0], chunk[1], chunk[2], cond_frames,
                   scale, kc[0], kc[1], kc[2])

    @classmethod
    def from_workload(cls, w):
        return cls.make(w.T, w.H, w.W, w.heads, w.batch, w.head_dim, w.chunk, w.cond_frames,
                        key_chunk=w.key_chunk or None)

    @property
    def key_chunk(self):
        if (self.ctk, self.chk, self.cwk) == (0, 0, 0):
            return (self.ct, self.ch, self.cw)
        return (self.ctk, self.chk, self.cwk)

    @property
    def num_key_blocks(self):
        a, b, c = self.key_chunk
        return _cdiv(self.T, a) * _cdiv(self.H, b) * _cdiv(self.W, c)

    @property
    def seq_len(self):
        return self.T * self.H * self.W

    @property
    def num_blocks(self):
        """Query blocks per (batch, head); a chunk that does not divide the
        grid leaves partial blocks at its far edge, counted here."""
        return _cdiv(self.T, self.ct) * _cdiv(self.H, self.ch) * _cdiv(self.W, self.cw)


class SelectParams(ctypes.Structure):
    """Mirror of ``bsa_select_params``."""

    _fields_ = [
        ("mode", ctypes.c_int32),
        ("k", ctypes.c_int32),
        ("cdf_p", ctypes.c_float),
        ("k_min", ctypes.c_int32),
        ("k_max", ctypes.c_int32),
    ]

    @classmethod
    def topk(cls, k):
        return cls(BSA_TOPK, k, 0.0, 0, 0)

    @classmethod
    def cdf(cls, p, k_min, k_max):
        return cls(BSA_CDF, 0, p, k_min, k_max)

    @classmethod
    def from_workload(cls, w):
        return cls.topk(w.k) if w.mode == "topk" else cls.cdf(w.p, w.k_min, w.k_max)


class BSAError(RuntimeError):
    def __init__(self, status, message):
        super().__init__(f"{message} (status {status})")
        self.status = status


_lib = None


def lib():
    """Load libbsa.so once; raise if it has not been built."""
    global _lib
    if _lib is None:
        if not os.path.exists(_LIB_PATH):
            raise RuntimeError(
                f"{_LIB_PATH} is missing: build it with `python -m video_dit_block_bsa_amd.build`"
            )
        # torch brings its own HIP runtime and asks for it by its unversioned
        # file name. Loaded first, libbsa.so would pull in the system copy
        # (soname libamdhip64.so.7), torch would then load a second one, and
        # kernels launched through the first would find no device. With torch
        # imported first, libbsa.so binds to torch's copy by soname.
        import torch  # noqa: F401

        L = ctypes.CDLL(_LIB_PATH)
        P, SP = ctypes.POINTER(Problem), ctypes.POINTER(SelectParams)
        vp, i32p = ctypes.c_void_p, ctypes.c_void_p
        L.bsa_index_stride.argtypes = [P, SP]
        L.bsa_index_stride.restype = ctypes.c_int32
        L.bsa_workspace_bytes.argtypes = [P, SP]
        L.bsa_workspace_bytes.restype = ctypes.c_size_t
        L.bsa_select_workspace_bytes.argtypes = [P, SP]
        L.bsa_select_workspace_bytes.restype = ctypes.c_size_t
        L.bsa_attention_workspace_bytes.argtypes = [P]
        L.bsa_attention_workspace_bytes.restype = ctypes.c_size_t
        L.bsa_select.argtypes = [P, SP, vp, vp, i32p, i32p, vp, ctypes.c_size_t, vp]
        L.bsa_select.restype = ctypes.c_int32
        L.bsa_attention.argtypes = [P, vp, vp, vp, i32p, i32p, ctypes.c_int32, vp, vp,
                                    ctypes.c_size_t, vp]
        L.bsa_attention.restype = ctypes.c_int32
        L.dense_attention.argtypes = [P, vp, vp, vp, vp, vp, ctypes.c_size_t, vp]
        L.dense_attention.restype = ctypes.c_int32
        L.bsa_attention_lse.argtypes = [P, vp, vp, vp, i32p, i32p, ctypes.c_int32, vp, vp, vp,
                                        ctypes.c_size_t, vp]
        L.bsa_attention_lse.restype = ctypes.c_int32
        L.bsa_attention_bwd_workspace_bytes.argtypes = [P]
        L.bsa_attention_bwd_workspace_bytes.restype = ctypes.c_size_t
        L.bsa_attention_bwd.argtypes = [P, vp, vp, vp, vp, vp, vp, i32p, i32p, ctypes.c_int32,
                                        vp, vp, vp, vp, ctypes.c_size_t, vp]
        L.bsa_attention_bwd.restype = ctypes.c_int32
        L.bsa_cond_cache_bytes.argtypes = [P]
        L.bsa_cond_cache_bytes.restype = ctypes.c_size_t
        L.bsa_pool_cond_keys.argtypes = [P, vp, vp, ctypes.c_size_t, vp]
        L.bsa_pool_cond_keys.restype = ctypes.c_int32
        L.bsa_select_noisy.argtypes = [P, SP, vp, vp, vp, ctypes.c_size_t, i32p, i32p, vp,
                                       ctypes.c_size_t, vp]
        L.bsa_select_noisy.restype = ctypes.c_int32
        L.bsa_attention_noisy.argtypes = [P, vp, vp, vp, i32p, i32p, ctypes.c_int32, vp, vp,
                                          ctypes.c_size_t, vp]
        L.bsa_attention_noisy.restype = ctypes.c_int32
        L.bsa_select_noalloc.argtypes = [P, SP, vp, vp, i32p, i32p, vp]
        L.bsa_select_noalloc.restype = ctypes.c_int32
        L.bsa_select_noalloc_max_workspace_bytes.argtypes = []
        L.bsa_select_noalloc_max_workspace_bytes.restype = ctypes.c_size_t
        L.bsa_status_string.argtypes = [ctypes.c_int32]
        L.bsa_status_string.restype = ctypes.c_char_p
        L.bsa_last_error.argtypes = []
        L.bsa_last_error.restype = ctypes.c_char_p
        _lib = L
    return _lib


def _ptr(x):
    if x is None:
        return None
    if isinstance(x, int):
        return x
    return x.data_ptr()


def _require(x, name, dtype, numel):
    """Checks a torch tensor argument before its pointer reaches the library,
    which cannot see sizes or strides: the dtype, a contiguous layout, a GPU
    device and at least `numel` elements. Raw integer addresses and None are
    passed through unchecked (the library rejects NULL itself)."""
    if x is None or isinstance(x, int):
        return
    import torch

    if dtype is not None and x.dtype != getattr(torch, dtype):
        raise BSAError(-1, f"{name} must be torch.{dtype} (got {x.dtype})")
    if not x.is_contiguous():
        raise BSAError(-1, f"{name} must be contiguous")
    if x.numel() < numel:
        raise BSAError(-1, f"{name} holds {x.numel()} elements, needs at least {numel}")
    if x.device.type != "cuda":
        raise BSAError(-1, f"{name} must be on a GPU (got {x.device})")


def _check_qkv(problem, **tensors):
    n = problem.batch * problem.heads * problem.seq_len * problem.head_dim
    for name, t in tensors.items():
        _require(t, name, "bfloat16", n)


def _check_lists(problem, idx, cnt, stride):
    rows = problem.batch * problem.heads * problem.num_blocks
    _require(idx, "idx", "int32", rows * max(int(stride), 0))
    _require(cnt, "cnt", "int32", rows)


def _check_workspace(ws):
    if isinstance(ws, tuple) or ws is None:
        return
    _require(ws, "workspace", None, 0)


def _nbytes(x):
    if x is None:
        return 0
    if isinstance(x, tuple):
        return x[1]
    return x.numel() * x.element_size()


def _stream(stream):
    if stream is None:
        import torch

        return torch.cuda.current_stream().cuda_stream
    if isinstance(stream, int):
        return stream
    return stream.cuda_stream


def _check(status):
    if status != 0:
        L = lib()
        msg = L.bsa_last_error().decode() or L.bsa_status_string(status).decode()
        raise BSAError(status, msg)


def index_stride(problem, params: SelectParams) -> int:
    """bsa_index_stride; ``problem`` may be None."""
    return lib().bsa_index_stride(None if problem is None else ctypes.byref(problem),
                                  ctypes.byref(params))


def workspace_bytes(problem: Problem, params: SelectParams) -> int:
    """bsa_workspace_bytes: one buffer for bsa_select followed by bsa_attention."""
    return lib().bsa_workspace_bytes(ctypes.byref(problem), ctypes.byref(params))


def select_workspace_bytes(problem: Problem, params: SelectParams) -> int:
    return lib().bsa_select_workspace_bytes(ctypes.byref(problem), ctypes.byref(params))


def attention_workspace_bytes(problem: Problem) -> int:
    return lib().bsa_attention_workspace_bytes(ctypes.byref(problem))


def bsa_select(problem, params, q, k, idx, cnt, workspace, stream=None):
    """bsa_select: pooled scores and key-block selection -> idx, cnt.
    ``workspace`` is a tensor or a (pointer, nbytes) tuple."""
    _check_qkv(problem, q=q, k=k)
    _check_lists(problem, idx, cnt, index_stride(problem, params))
    _check_workspace(workspace)
    ws_ptr = workspace[0] if isinstance(workspace, tuple) else _ptr(workspace)
    _check(lib().bsa_select(ctypes.byref(problem), ctypes.byref(params), _ptr(q), _ptr(k),
                            _ptr(idx), _ptr(cnt), ws_ptr, _nbytes(workspace), _stream(stream)))


def bsa_attention(problem, q, k, v, idx, cnt, idx_stride, o, workspace, stream=None):
    """bsa_attention: attention restricted to the listed key blocks -> o."""
    _check_qkv(problem, q=q, k=k, v=v, o=o)
    _check_lists(problem, idx, cnt, idx_stride)
    _check_workspace(workspace)
    ws_ptr = workspace[0] if isinstance(workspace, tuple) else _ptr(workspace)
    _check(lib().bsa_attention(ctypes.byref(problem), _ptr(q), _ptr(k), _ptr(v), _ptr(idx),
                               _ptr(cnt), int(idx_stride), _ptr(o), ws_ptr, _nbytes(workspace),
                               _stream(stream)))


def dense_attention(problem, q, k, v, o, workspace, stream=None):
    """dense_attention: softmax attention over every allowed key -> o."""
    _check_qkv(problem, q=q, k=k, v=v, o=o)
    _check_workspace(workspace)
    ws_ptr = workspace[0] if isinstance(workspace, tuple) else _ptr(workspace)
    _check(lib().dense_attention(ctypes.byref(problem), _ptr(q), _ptr(k), _ptr(v), _ptr(o),
                                 ws_ptr, _nbytes(workspace), _stream(stream)))


def attention_bwd_workspace_bytes(problem: Problem) -> int:
    return lib().bsa_attention_bwd_workspace_bytes(ctypes.byref(problem))


def bsa_attention_lse(problem, q, k, v, idx, cnt, idx_stride, o, lse, workspace, stream=None):
    """bsa_attention_lse: bsa_attention that also writes the per-query
    log-normaliser -> o, lse."""
    _check_qkv(problem, q=q, k=k, v=v, o=o)
    _check_lists(problem, idx, cnt, idx_stride)
    _require(lse, "lse", "float32", problem.batch * problem.heads * problem.seq_len)
    _check_workspace(workspace)
    ws_ptr = workspace[0] if isinstance(workspace, tuple) else _ptr(workspace)
    _check(lib().bsa_attention_lse(ctypes.byref(problem), _ptr(q), _ptr(k), _ptr(v), _ptr(idx),
                                   _ptr(cnt), int(idx_stride), _ptr(o), _ptr(lse), ws_ptr,
                                   _nbytes(workspace), _stream(stream)))


def bsa_attention_bwd(problem, q, k, v, o, dout, lse, idx, cnt, idx_stride, dq, dk, dv,
                      workspace, stream=None):
    """bsa_attention_bwd: gradients of sum(dout * o) for fixed selections
    -> dq, dk, dv."""
    _check_qkv(problem, q=q, k=k, v=v, o=o, dout=dout, dq=dq, dk=dk, dv=dv)
    _check_lists(problem, idx, cnt, idx_stride)
    _require(lse, "lse", "float32", problem.batch * problem.heads * problem.seq_len)
    _check_workspace(workspace)
    ws_ptr = workspace[0] if isinstance(workspace, tuple) else _ptr(workspace)
    _check(lib().bsa_attention_bwd(ctypes.byref(problem), _ptr(q), _ptr(k), _ptr(v), _ptr(o),
                                   _ptr(dout), _ptr(lse), _ptr(idx), _ptr(cnt), int(idx_stride),
                                   _ptr(dq), _ptr(dk), _ptr(dv), ws_ptr, _nbytes(workspace),
                                   _stream(stream)))


def cond_cache_bytes(problem: Problem) -> int:
    return lib().bsa_cond_cache_bytes(ctypes.byref(problem))


def bsa_pool_cond_keys(problem, k, cache, stream=None):
    """bsa_pool_cond_keys: pooled condition keys -> cache (tensor or (ptr, nbytes))."""
    _check_qkv(problem, k=k)
    if not isinstance(cache, tuple):
        _require(cache, "cache", "float32", cond_cache_bytes(problem) // 4)
    cache_ptr = cache[0] if isinstance(cache, tuple) else _ptr(cache)
    _check(lib().bsa_pool_cond_keys(ctypes.byref(problem), _ptr(k), cache_ptr, _nbytes(cache),
                                    _stream(stream)))


def bsa_select_noisy(problem, params, q, k, cache, idx, cnt, workspace, stream=None):
    """bsa_select_noisy: selection for the noisy query blocks, condition
    pooled keys from the cache."""
    _check_qkv(problem, q=q, k=k)
    _check_lists(problem, idx, cnt, index_stride(problem, params))
    if not isinstance(cache, tuple):
        _require(cache, "cache", "float32", cond_cache_bytes(problem) // 4)
    _check_workspace(workspace)
    ws_ptr = workspace[0] if isinstance(workspace, tuple) else _ptr(workspace)
    cache_ptr = cache[0] if isinstance(cache, tuple) else _ptr(cache)
    _check(lib().bsa_select_noisy(ctypes.byref(problem), ctypes.byref(params), _ptr(q), _ptr(k),
                                  cache_ptr, _nbytes(cache), _ptr(idx), _ptr(cnt), ws_ptr,
                                  _nbytes(workspace), _stream(stream)))


def bsa_attention_noisy(problem, q, k, v, idx, cnt, idx_stride, o, workspace, stream=None):
    """bsa_attention_noisy: attention for the noisy query blocks -> o."""
    _check_qkv(problem, q=q, k=k, v=v, o=o)
    _check_lists(problem, idx, cnt, idx_stride)
    _check_workspace(workspace)
    ws_ptr = workspace[0] if isinstance(workspace, tuple) else _ptr(workspace)
    _check(lib().bsa_attention_noisy(ctypes.byref(problem), _ptr(q), _ptr(k), _ptr(v), _ptr(idx),
                                     _ptr(cnt), int(idx_stride), _ptr(o), ws_ptr,
                                     _nbytes(workspace), _stream(stream)))


def select_noalloc_max_workspace_bytes() -> int:
    return lib().bsa_select_noalloc_max_workspace_bytes()


def bsa_select_noalloc(problem, params, q, k, idx, cnt, stream=None):
    """bsa_select_noalloc: bsa_select with the library's static device
    scratch as workspace (no allocation) -> idx, cnt."""
    _check_qkv(problem, q=q, k=k)
    _check_lists(problem, idx, cnt, index_stride(problem, params))
    _check(lib().bsa_select_noalloc(ctypes.byref(problem), ctypes.byref(params), _ptr(q), _ptr(k),
                                    _ptr(idx), _ptr(cnt), _stream(stream)))
