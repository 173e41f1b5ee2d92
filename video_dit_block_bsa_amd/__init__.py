"""MI355X-native 3D Block Sparse Attention (BSA).

The compute lives in ``libbsa.so`` (hand-written HIP kernels for gfx950
behind a C ABI, declared in ``include/bsa.h``). This package is a thin
ctypes binding over it plus the synthetic-input generators and workload
table. Importing the package does not load the library; the first call
does, and it raises if the library has not been built.
"""

from .workloads import WORKLOADS, Workload, effective_flops  # noqa: F401


def __getattr__(name):
    # The binding is loaded lazily so that CPU-only tooling (input generation,
    # workload tables) works on machines without a built library.
    if name in {
        "bsa_select",
        "bsa_attention",
        "dense_attention",
        "Problem",
        "SelectParams",
        "BSAError",
        "lib",
        "select_workspace_bytes",
        "attention_workspace_bytes",
        "index_stride",
        "bsa_attention_lse",
        "bsa_attention_bwd",
        "attention_bwd_workspace_bytes",
        "cond_cache_bytes",
        "bsa_pool_cond_keys",
        "bsa_select_noisy",
        "bsa_attention_noisy",
    }:
        from . import binding

        return getattr(binding, name)
    raise AttributeError(name)
