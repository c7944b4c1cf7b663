"""Algorithmic work of the routed operators, counted from the masks.

Only the work the method must do is counted (the active (token, group) pairs),
never the dense work it skips. Integer results, exact.
"""
from __future__ import annotations

import numpy as np


def active_pairs(mask) -> int:
    return int(np.count_nonzero(np.asarray(mask)))


def gemm_mn_flops(mask2d, K: int, G: int) -> int:
    """Each active (token, group) computes G outputs of length-K dot products."""
    return 2 * K * G * active_pairs(mask2d)


def gemm_k_flops(mask2d, N: int, G: int) -> int:
    """Each active (token, K-group) contributes G reduction steps to N outputs."""
    return 2 * N * G * active_pairs(mask2d)


def attention_flops(mask, Tk: int, Hq: int, d: int, causal: bool = True, leftpad=None) -> int:
    """QK^T and PV: 4*d FLOPs per valid key for every head of an active group
    (keys before a sequence's left padding are not valid)."""
    mask = np.asarray(mask) != 0
    B, Tq, Hk = mask.shape
    rep = Hq // Hk
    t = np.arange(Tq)
    end = np.minimum(t + (Tk - Tq) + 1, Tk) if causal else np.full(Tq, Tk)
    total = 0
    for b in range(B):
        start = int(leftpad[b]) if leftpad is not None else 0
        nkeys = np.maximum(end - start, 0).astype(np.int64)
        total += int(np.dot(mask[b].sum(axis=1).astype(np.int64), nkeys))
    return int(4 * d * rep * total)


def layer_flops(s, mask_attn, mask_ffn, leftpad=None) -> dict:
    """Active FLOPs of each routed operator of one masked layer."""
    out = {}
    M = s.M
    if mask_attn is not None:
        ma = np.asarray(mask_attn).reshape(M, s.Hk)
        out["q_proj"] = gemm_mn_flops(ma, s.D, s.G_attn)
        out["attention"] = attention_flops(mask_attn, s.Tkv, s.Hq, s.d, leftpad=leftpad)
        out["o_proj"] = gemm_k_flops(ma, s.D, s.G_attn)
    if mask_ffn is not None:
        mf = np.asarray(mask_ffn).reshape(M, s.NG_ffn)
        out["gate_up_swiglu"] = 2 * gemm_mn_flops(mf, s.D, s.G_ffn)
        out["down_proj"] = gemm_k_flops(mf, s.D, s.G_ffn)
    return out


def decode_bytes(s, mask_attn, mask_ffn) -> dict:
    """HBM bytes one decode step must read (bf16), for B sequences with one new
    token each (masks [B][1][Hk] and [B][1][NG_ffn], or one row for B = 1):
    a weight row or column is read once if any token keeps its group; each
    sequence reads the K and V cache of every group its token keeps."""
    ma = np.asarray(mask_attn).reshape(-1, s.Hk) != 0
    mf = np.asarray(mask_ffn).reshape(-1, s.NG_ffn) != 0
    ga = int(ma.any(axis=0).sum())    # attention groups some token keeps
    gf = int(mf.any(axis=0).sum())
    kv_pairs = int(ma.sum())          # (sequence, group) pairs
    return {
        "q_proj": ga * s.G_attn * s.D * 2,
        "attention": kv_pairs * 2 * s.Tkv * s.d * 2,
        "o_proj": ga * s.D * s.G_attn * 2,
        "gate_up_swiglu": gf * 2 * s.G_ffn * s.D * 2,
        "down_proj": gf * s.D * s.G_ffn * 2,
    }
