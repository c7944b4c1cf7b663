"""Masked group-mask layer execution (WIDE) for AMD Instinct MI355X.

The compute lives in libwide.so (hand-written HIP kernels for gfx950 behind
the C ABI of include/wide.h); this package holds that library, its ctypes
binding and the seeded synthetic workload generators.
"""
from ._lib import (  # noqa: F401
    WideError, attn, attn_workspace_bytes, gemm_k, gemm_k_grouped, gemm_k_workspace_bytes, gemm_mn,
    gemm_mn_swiglu, gemm_mn_workspace_bytes, load, mfma_probe, order_by_pattern, reorder, router,
    status_string,
)

__all__ = ["WideError", "attn", "attn_workspace_bytes", "gemm_k", "gemm_k_grouped", "gemm_k_workspace_bytes",
           "gemm_mn", "gemm_mn_swiglu", "gemm_mn_workspace_bytes", "load", "mfma_probe", "order_by_pattern",
           "reorder", "router", "status_string"]
