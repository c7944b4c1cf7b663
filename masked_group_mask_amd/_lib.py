"""ctypes binding of libwide.so.

Argument marshalling only: tensors are checked for device, dtype, shape and
layout, and their device pointers and the current HIP stream are handed to the
C ABI declared in include/wide.h. Every computation runs in the library's HIP
kernels; there is no fallback. If the library is missing, loading raises.
"""
from __future__ import annotations

import ctypes
import os
from typing import Optional, Tuple

import torch

_PKG = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_PKG, "libwide.so")

WIDE_DTYPE_BF16 = 0
WIDE_DTYPE_F32 = 1

_i64 = ctypes.c_int64
_int = ctypes.c_int
_ptr = ctypes.c_void_p
_size = ctypes.c_size_t
_f32 = ctypes.c_float

_SIGS = {
    "wide_reorder": [_ptr, _i64, _i64, _i64, _ptr, _ptr, _ptr],
    "wide_gemm_mn": [_ptr, _i64, _ptr, _i64, _ptr, _i64, _int, _i64, _i64, _i64, _i64,
                     _ptr, _ptr, _ptr, _ptr],
    "wide_gemm_mn_swiglu": [_ptr, _i64, _ptr, _ptr, _i64, _ptr, _i64, _int, _i64, _i64, _i64,
                            _i64, _ptr, _ptr, _ptr, _ptr],
    "wide_gemm_mn_ws": [_ptr, _i64, _ptr, _i64, _ptr, _i64, _int, _i64, _i64, _i64, _i64,
                        _ptr, _ptr, _ptr, _ptr, _size, _ptr],
    "wide_gemm_mn_swiglu_ws": [_ptr, _i64, _ptr, _ptr, _i64, _ptr, _i64, _int, _i64, _i64, _i64,
                               _i64, _ptr, _ptr, _ptr, _ptr, _size, _ptr],
    "wide_gemm_mn_workspace_bytes": [_i64, _i64, _i64, _i64, _int],
    "wide_order_by_pattern": [_ptr, _i64, _i64, _ptr, _ptr],
    "wide_gemm_k": [_ptr, _i64, _ptr, _i64, _ptr, _i64, _int, _i64, _i64, _i64, _i64, _ptr, _ptr, _ptr],
    "wide_gemm_k_ws": [_ptr, _i64, _ptr, _i64, _ptr, _i64, _int, _i64, _i64, _i64, _i64, _ptr, _ptr, _ptr,
                       _size, _ptr],
    "wide_gemm_k_workspace_bytes": [_i64] * 3,
    "wide_gemm_k_grouped": [_ptr, _i64, _ptr, _i64, _ptr, _i64, _int, _i64, _i64, _i64, _i64, _ptr, _ptr,
                            _ptr],
    "wide_attn": [_ptr, _ptr, _ptr, _ptr, _int, _i64, _i64, _i64, _i64, _i64, _i64, _int, _f32,
                  _ptr, _ptr, _ptr, _ptr, _ptr, _size, _ptr],
    "wide_router": [_ptr, _i64, _ptr, _ptr, _i64, _i64, _i64, _i64, _i64, _ptr, _ptr, _ptr, _ptr,
                    _ptr],
    "wide_attn_grouped": [_ptr, _ptr, _ptr, _ptr, _int, _i64, _i64, _i64, _i64, _i64, _i64, _i64, _int,
                          _f32, _ptr, _ptr, _ptr, _ptr, _ptr, _size, _ptr],
    "wide_attn_noalloc": [_ptr, _ptr, _ptr, _ptr, _int, _i64, _i64, _i64, _i64, _i64, _i64, _int, _f32,
                          _ptr, _ptr, _ptr, _ptr, _ptr],
    "wide_attn_workspace_bytes": [_i64] * 6,
    "wide_mfma_probe": [_i64, _i64, _ptr, _ptr],
    "wide_status_string": [_int],
    "wide_abi_version": [],
}
_RESTYPES = {"wide_attn_workspace_bytes": _size, "wide_gemm_k_workspace_bytes": _size,
             "wide_gemm_mn_workspace_bytes": _size,
             "wide_status_string": ctypes.c_char_p}

EXPORTED = tuple(_SIGS)

_lib = None


class WideError(RuntimeError):
    def __init__(self, fn: str, status: int):
        self.status = status
        super().__init__(f"{fn} failed: {status_string(status)} ({status})")


def load(path: str = LIB_PATH) -> ctypes.CDLL:
    """Load libwide.so (once). Raises if it has not been built."""
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(path):
        raise ImportError(f"{path} is missing: build it with masked_group_mask_amd.build.build()")
    lib = ctypes.CDLL(path)
    for name, args in _SIGS.items():
        fn = getattr(lib, name)
        fn.argtypes = args
        fn.restype = _RESTYPES.get(name, _int)
    _lib = lib
    return lib


def status_string(status: int) -> str:
    return load().wide_status_string(status).decode()


def _call(name: str, *args) -> None:
    st = getattr(load(), name)(*args)
    if st != 0:
        raise WideError(name, st)


def _p(t: Optional[torch.Tensor]):
    return None if t is None else ctypes.c_void_p(t.data_ptr())


def _stream() -> ctypes.c_void_p:
    return ctypes.c_void_p(torch.cuda.current_stream().cuda_stream)


def _need(t: torch.Tensor, name: str, dtype, ndim: Optional[int] = None):
    """Type, element type and rank; the device is checked by _on_device once
    every size has been checked."""
    if not isinstance(t, torch.Tensor):
        raise TypeError(f"{name} must be a torch.Tensor")
    if t.dtype != dtype:
        raise TypeError(f"{name} must be {dtype}, got {t.dtype}")
    if ndim is not None and t.dim() != ndim:
        raise ValueError(f"{name} must have {ndim} dimensions, got {t.dim()}")


def _on_device(first: torch.Tensor, **others) -> None:
    """Every tensor is a device tensor on `first`'s device (last check before
    pointers are handed to the library)."""
    for name, t in (("first operand", first),) + tuple(others.items()):
        if t is None:
            continue
        if not t.is_cuda:
            raise ValueError(f"{name} must be a device tensor")
        if t.device != first.device:
            raise ValueError(f"{name} is on {t.device}, expected {first.device}")


def _sized(t: Optional[torch.Tensor], name: str, dtype, numel: int, last: int):
    """A contiguous routing tensor of exactly `numel` elements whose last
    dimension is `last` (the kernels index it with these sizes)."""
    if t is None:
        return
    _need(t, name, dtype)
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")
    if t.numel() != numel or t.dim() == 0 or t.shape[-1] != last:
        raise ValueError(f"{name} has shape {tuple(t.shape)}: expected {numel} elements, last dimension {last}")


def _rowmajor(t: torch.Tensor, name: str) -> int:
    """Leading dimension of a 2-D tensor whose rows are contiguous."""
    if t.stride(1) != 1:
        raise ValueError(f"{name} rows must be contiguous")
    return t.stride(0)


def _dt(dtype) -> int:
    if dtype == torch.bfloat16:
        return WIDE_DTYPE_BF16
    if dtype == torch.float32:
        return WIDE_DTYPE_F32
    raise TypeError(f"unsupported output dtype {dtype}")


# ---------------------------------------------------------------------------


def reorder(mask: torch.Tensor, perm: Optional[torch.Tensor] = None,
            counts: Optional[torch.Tensor] = None) -> Tuple[torch.Tensor, torch.Tensor]:
    """mask [B][T][NG] uint8 -> (perm [B][NG][T] int32, counts [B][NG] int32)."""
    _need(mask, "mask", torch.uint8, 3)
    mask = mask.contiguous()
    B, T, NG = mask.shape
    if perm is None:
        perm = torch.empty((B, NG, T), dtype=torch.int32, device=mask.device)
    if counts is None:
        counts = torch.empty((B, NG), dtype=torch.int32, device=mask.device)
    _need(perm, "perm", torch.int32, 3)
    _need(counts, "counts", torch.int32, 2)
    if tuple(perm.shape) != (B, NG, T) or tuple(counts.shape) != (B, NG):
        raise ValueError("perm/counts shape mismatch")
    if not (perm.is_contiguous() and counts.is_contiguous()):
        raise ValueError("perm/counts must be contiguous")
    _on_device(mask, perm=perm, counts=counts)
    _call("wide_reorder", _p(mask), B, T, NG, _p(perm), _p(counts), _stream())
    return perm, counts


def order_by_pattern(mask: torch.Tensor, order: Optional[torch.Tensor] = None) -> torch.Tensor:
    """mask [M][NG] uint8 (or [1][M][NG]) -> order [M] int32: the token rows
    stably sorted by the Gray-code rank of their pattern over the first
    min(NG, 8) groups; GEMM-K's row order."""
    _need(mask, "mask", torch.uint8)
    if mask.dim() not in (2, 3) or (mask.dim() == 3 and mask.shape[0] != 1):
        raise ValueError("mask must be [M][NG] or [1][M][NG]")
    if not mask.is_contiguous():
        raise ValueError("mask must be contiguous")
    M, NG = mask.shape[-2], mask.shape[-1]
    if order is None:
        order = torch.empty(M, dtype=torch.int32, device=mask.device)
    _sized(order, "order", torch.int32, M, M)
    _on_device(mask, order=order)
    _call("wide_order_by_pattern", _p(mask), M, NG, _p(order), _stream())
    return order


def router(X: torch.Tensor, W1: torch.Tensor, W2: torch.Tensor, B: int = 1,
           with_logits: bool = False, with_reorder: bool = True):
    """Bottleneck router and routing decision, then (optionally) the reorder.

    X [B*T][D] bf16; W1 [r][D] and W2 [2*NG][r] bf16, contiguous. Returns
    (mask [B][T][NG] uint8, perm, counts, logits) with perm/counts None unless
    with_reorder and logits ([B*T][2*NG] fp32) None unless with_logits."""
    _need(X, "X", torch.bfloat16, 2)
    _need(W1, "W1", torch.bfloat16, 2)
    _need(W2, "W2", torch.bfloat16, 2)
    if not (W1.is_contiguous() and W2.is_contiguous()):
        raise ValueError("W1 and W2 must be contiguous")
    M, D = X.shape
    r = W1.shape[0]
    if W1.shape[1] != D or W2.shape[1] != r or W2.shape[0] % 2:
        raise ValueError("router shapes disagree")
    if M % B:
        raise ValueError("rows of X must be a multiple of B")
    T, NG = M // B, W2.shape[0] // 2
    dev = X.device
    mask = torch.empty((B, T, NG), dtype=torch.uint8, device=dev)
    logits = torch.empty((M, 2 * NG), dtype=torch.float32, device=dev) if with_logits else None
    perm = torch.empty((B, NG, T), dtype=torch.int32, device=dev) if with_reorder else None
    counts = torch.empty((B, NG), dtype=torch.int32, device=dev) if with_reorder else None
    _on_device(X, W1=W1, W2=W2)
    _call("wide_router", _p(X), _rowmajor(X, "X"), _p(W1), _p(W2), B, T, D, r, NG, _p(mask),
          _p(logits), _p(perm), _p(counts), _stream())
    return mask, perm, counts, logits


def _routing(M: int, NG: int, perm, counts, mask):
    """perm [NG][M] int32 and counts [NG] int32 (a wide_reorder output with
    batch 1) and mask [M][NG] uint8, checked against the problem's sizes
    before any pointer reaches a kernel."""
    if (perm is None) != (counts is None):
        raise ValueError("perm and counts go together")
    _sized(perm, "perm", torch.int32, NG * M, M)
    _sized(counts, "counts", torch.int32, NG, NG)
    _sized(mask, "mask", torch.uint8, M * NG, NG)


def _mn_common(A, N, G, perm, counts, mask):
    _need(A, "A", torch.bfloat16, 2)
    lda = _rowmajor(A, "A")
    if G < 1 or N % G:
        raise ValueError(f"N = {N} is not a multiple of the group size {G}")
    _routing(A.shape[0], N // G, perm, counts, mask)
    return lda


def gemm_mn_workspace_bytes(M: int, N: int, K: int, G: int, swiglu: bool = False) -> int:
    return int(load().wide_gemm_mn_workspace_bytes(M, N, K, G, int(bool(swiglu))))


def _ws(workspace: Optional[torch.Tensor], A: torch.Tensor):
    if workspace is None:
        return None, 0
    if workspace.device != A.device or not workspace.is_contiguous():
        raise ValueError("workspace must be a contiguous tensor on A's device")
    return _p(workspace), workspace.numel() * workspace.element_size()


def gemm_mn(A: torch.Tensor, B: torch.Tensor, G: int, perm: Optional[torch.Tensor] = None,
            counts: Optional[torch.Tensor] = None, mask: Optional[torch.Tensor] = None,
            out: Optional[torch.Tensor] = None, out_dtype=torch.bfloat16,
            workspace: Optional[torch.Tensor] = None) -> torch.Tensor:
    """C = A B^T on the active (token, group) entries; others keep `out`'s values
    (zeros if `out` is allocated here). workspace: optional device buffer of
    gemm_mn_workspace_bytes(M, N, K, G) bytes; with it the active tiles are
    scheduled on the device and a partly filled last round is split along K."""
    _need(B, "B", torch.bfloat16, 2)
    lda = _mn_common(A, B.shape[0], G, perm, counts, mask)
    ldb = _rowmajor(B, "B")
    M, K = A.shape
    N = B.shape[0]
    if B.shape[1] != K:
        raise ValueError("A and B disagree on K")
    if out is None:
        out = torch.zeros((M, N), dtype=out_dtype, device=A.device)
    _need(out, "out", out.dtype, 2)
    if tuple(out.shape) != (M, N):
        raise ValueError("out shape mismatch")
    _on_device(A, B=B, out=out, perm=perm, counts=counts, mask=mask, workspace=workspace)
    ws, wsb = _ws(workspace, A)
    _call("wide_gemm_mn_ws", _p(A), lda, _p(B), ldb, _p(out), _rowmajor(out, "out"), _dt(out.dtype),
          M, N, K, G, _p(perm), _p(counts), _p(mask), ws, wsb, _stream())
    return out


def gemm_mn_swiglu(A: torch.Tensor, Wg: torch.Tensor, Wu: torch.Tensor, G: int,
                   perm: Optional[torch.Tensor] = None, counts: Optional[torch.Tensor] = None,
                   mask: Optional[torch.Tensor] = None, out: Optional[torch.Tensor] = None,
                   out_dtype=torch.bfloat16, workspace: Optional[torch.Tensor] = None) -> torch.Tensor:
    """H = SiLU(A Wg^T) * (A Wu^T) on the active entries. workspace: as gemm_mn
    (gemm_mn_workspace_bytes(M, N, K, G, swiglu=True) bytes)."""
    _need(Wg, "Wg", torch.bfloat16, 2)
    _need(Wu, "Wu", torch.bfloat16, 2)
    lda = _mn_common(A, Wg.shape[0], G, perm, counts, mask)
    ldb = _rowmajor(Wg, "Wg")
    if Wu.shape != Wg.shape or _rowmajor(Wu, "Wu") != ldb:
        raise ValueError("Wg and Wu must have the same shape and leading dimension")
    M, K = A.shape
    N = Wg.shape[0]
    if Wg.shape[1] != K:
        raise ValueError("A and Wg disagree on K")
    if out is None:
        out = torch.zeros((M, N), dtype=out_dtype, device=A.device)
    _need(out, "out", out.dtype, 2)
    if tuple(out.shape) != (M, N):
        raise ValueError("out shape mismatch")
    _on_device(A, Wg=Wg, Wu=Wu, out=out, perm=perm, counts=counts, mask=mask, workspace=workspace)
    ws, wsb = _ws(workspace, A)
    _call("wide_gemm_mn_swiglu_ws", _p(A), lda, _p(Wg), _p(Wu), ldb, _p(out),
          _rowmajor(out, "out"), _dt(out.dtype), M, N, K, G, _p(perm), _p(counts), _p(mask),
          ws, wsb, _stream())
    return out


def gemm_k_workspace_bytes(M: int, N: int, K: int) -> int:
    return int(load().wide_gemm_k_workspace_bytes(M, N, K))


def gemm_k(A: torch.Tensor, B: torch.Tensor, G: int, mask: torch.Tensor,
           out: Optional[torch.Tensor] = None, beta: int = 0,
           workspace: Optional[torch.Tensor] = None, order: Optional[torch.Tensor] = None) -> torch.Tensor:
    """C = beta*C + sum over active K-groups of A B^T (fp32 output).
    workspace: optional device buffer of gemm_k_workspace_bytes(M, N, K)
    bytes; with it the last, partly filled round of tiles is split along K.
    order: optional [M] int32 row permutation (order_by_pattern(mask)); with
    it tiles skip the work of groups their rows do not keep."""
    _need(A, "A", torch.bfloat16, 2)
    _need(B, "B", torch.bfloat16, 2)
    M, K = A.shape
    N = B.shape[0]
    if B.shape[1] != K:
        raise ValueError("A and B disagree on K")
    if G < 1 or K % G:
        raise ValueError(f"K = {K} is not a multiple of the group size {G}")
    if mask is None:
        raise ValueError("gemm_k needs the mask")
    _sized(mask, "mask", torch.uint8, M * (K // G), K // G)
    _sized(order, "order", torch.int32, M, M)
    if out is None:
        out = torch.empty((M, N), dtype=torch.float32, device=A.device)
        beta = 0
    _need(out, "out", torch.float32, 2)
    if tuple(out.shape) != (M, N):
        raise ValueError("out shape mismatch")
    _on_device(A, B=B, out=out, mask=mask, workspace=workspace, order=order)
    ws, wsb = _ws(workspace, A)
    _call("wide_gemm_k_ws", _p(A), _rowmajor(A, "A"), _p(B), _rowmajor(B, "B"), _p(out),
          _rowmajor(out, "out"), int(beta), M, N, K, G, _p(order), _p(mask), ws, wsb, _stream())
    return out


def gemm_k_grouped(A: torch.Tensor, B: torch.Tensor, G: int, perm: torch.Tensor, counts: torch.Tensor,
                   out: Optional[torch.Tensor] = None, beta: int = 0) -> torch.Tensor:
    """GEMM-K group by group from the reorder of the [M][K/G] mask: every
    active (group, row tile) multiplies over the group's columns and adds its
    partial into C (fp32) with atomics. perm [K/G][M] (or [1][K/G][M]) and
    counts [K/G] (or [1][K/G]) from reorder."""
    _need(A, "A", torch.bfloat16, 2)
    _need(B, "B", torch.bfloat16, 2)
    M, K = A.shape
    N = B.shape[0]
    if B.shape[1] != K:
        raise ValueError("A and B disagree on K")
    if G < 1 or K % G:
        raise ValueError(f"K = {K} is not a multiple of the group size {G}")
    if perm is None or counts is None:
        raise ValueError("gemm_k_grouped needs perm and counts")
    _routing(M, K // G, perm, counts, None)
    if out is None:
        out = torch.empty((M, N), dtype=torch.float32, device=A.device)
        beta = 0
    _need(out, "out", torch.float32, 2)
    if tuple(out.shape) != (M, N):
        raise ValueError("out shape mismatch")
    _on_device(A, B=B, out=out, perm=perm, counts=counts)
    _call("wide_gemm_k_grouped", _p(A), _rowmajor(A, "A"), _p(B), _rowmajor(B, "B"), _p(out),
          _rowmajor(out, "out"), int(beta), M, N, K, G, _p(perm), _p(counts), _stream())
    return out


def attn_workspace_bytes(B: int, Tq: int, Tk: int, Hq: int, Hk: int, d: int) -> int:
    return int(load().wide_attn_workspace_bytes(B, Tq, Tk, Hq, Hk, d))


def attn(Q: torch.Tensor, K: torch.Tensor, V: torch.Tensor, perm: Optional[torch.Tensor] = None,
         counts: Optional[torch.Tensor] = None, mask: Optional[torch.Tensor] = None,
         causal: bool = True, scale: float = 0.0, leftpad: Optional[torch.Tensor] = None,
         out: Optional[torch.Tensor] = None, out_dtype=torch.bfloat16,
         workspace: Optional[torch.Tensor] = None, groups: Optional[int] = None,
         noalloc: bool = False) -> torch.Tensor:
    """Head-group-masked GQA attention; Q [B][Tq][Hq][d], K/V [B][Tk][Hk][d].
    groups: routing groups (default Hk); finer groups gate fewer query heads
    each (mask [B][Tq][groups], perm/counts from reorder of that mask).
    noalloc: call wide_attn_noalloc (the library's built-in decode scratch;
    no workspace is allocated here; `out` must then be given)."""
    for t, n in ((Q, "Q"), (K, "K"), (V, "V")):
        _need(t, n, torch.bfloat16, 4)
        if not t.is_contiguous():
            raise ValueError(f"{n} must be contiguous")
    B, Tq, Hq, d = Q.shape
    Bk, Tk, Hk, dk = K.shape
    if Bk != B or dk != d or tuple(V.shape) != tuple(K.shape):
        raise ValueError("Q/K/V shapes disagree")
    NG = Hk if groups is None else int(groups)
    if NG < 1:
        raise ValueError("groups must be positive")
    if (perm is None) != (counts is None):
        raise ValueError("perm and counts go together")
    _sized(perm, "perm", torch.int32, B * NG * Tq, Tq)
    _sized(counts, "counts", torch.int32, B * NG, NG)
    _sized(mask, "mask", torch.uint8, B * Tq * NG, NG)
    _sized(leftpad, "leftpad", torch.int32, B, B)
    if noalloc and out is None:
        raise ValueError("noalloc needs the output tensor: the call allocates nothing")
    if out is None:
        out = torch.zeros((B, Tq, Hq, d), dtype=out_dtype, device=Q.device)
    _need(out, "out", out.dtype, 4)
    if tuple(out.shape) != (B, Tq, Hq, d) or not out.is_contiguous():
        raise ValueError("out must be a contiguous [B][Tq][Hq][d] tensor")
    _on_device(Q, K=K, V=V, out=out, perm=perm, counts=counts, mask=mask, leftpad=leftpad,
               workspace=workspace)
    if noalloc:
        if workspace is not None or (groups is not None and groups != Hk):
            raise ValueError("noalloc takes no workspace and only one routing group per KV head")
        _call("wide_attn_noalloc", _p(Q), _p(K), _p(V), _p(out), _dt(out.dtype), B, Tq, Tk, Hq, Hk, d,
              int(bool(causal)), float(scale), _p(leftpad), _p(perm), _p(counts), _p(mask), _stream())
        return out
    need = attn_workspace_bytes(B, Tq, Tk, Hq, Hk, d)
    if need and workspace is None:
        workspace = torch.empty(need, dtype=torch.uint8, device=Q.device)
    if workspace is not None and not workspace.is_contiguous():
        raise ValueError("workspace must be contiguous")
    ws_bytes = 0 if workspace is None else workspace.numel() * workspace.element_size()
    if groups is None or groups == Hk:
        _call("wide_attn", _p(Q), _p(K), _p(V), _p(out), _dt(out.dtype), B, Tq, Tk, Hq, Hk, d,
              int(bool(causal)), float(scale), _p(leftpad), _p(perm), _p(counts), _p(mask),
              _p(workspace), ws_bytes, _stream())
    else:
        _call("wide_attn_grouped", _p(Q), _p(K), _p(V), _p(out), _dt(out.dtype), B, Tq, Tk, Hq, Hk,
              int(groups), d, int(bool(causal)), float(scale), _p(leftpad), _p(perm), _p(counts),
              _p(mask), _p(workspace), ws_bytes, _stream())
    return out


def mfma_probe(blocks: int, iters: int, sink: torch.Tensor) -> None:
    """Launch the MFMA rate probe (blocks * 4 * iters * 8 * 16384 bf16 FLOPs);
    sink is a device float tensor of at least blocks * 4 elements."""
    _need(sink, "sink", torch.float32)
    if sink.numel() < blocks * 4 or not sink.is_contiguous():
        raise ValueError("sink needs blocks * 4 contiguous floats")
    _on_device(sink)
    _call("wide_mfma_probe", blocks, iters, _p(sink), _stream())
