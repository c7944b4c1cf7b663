"""CPU oracle for the masked group-mask layer (WIDE).

TEST INFRASTRUCTURE ONLY. This module is the plain, slow, obviously correct
statement of what the masked layer computes. It is imported by the tests, by
the package's smoke check and by the bench's CPU-baseline leg, and by nothing
else: the product path (the HIP library and its binding) never calls it and
shares no code with it.

Source: "WIDE: Boosting Adaptive LLM Inference via Token-level Dynamic Width
Pruning" (arXiv 2607.28418, HTML version). Citations below name that page's
sections, equations and algorithms.

Conventions
-----------
* Floating-point inputs arrive as raw bfloat16 bits (uint16). They are widened
  exactly to float64 and every computation runs in float64.
* Masks are integer arrays; any nonzero entry means "active" (class 0 of the
  router, section 3.1 Eq. 5, executes the group).
* Outputs are float64. ``round_bf16`` gives the round-to-nearest-even bfloat16
  value of a float64 result, for comparing bf16-stored outputs.
* Entries the method never writes (inactive rows/groups) are exactly +0.0,
  the value of the zero-initialised output the kernels write into (Appendix B,
  Algorithms 2-4 take a zero-initialised C or O).

Readings of the page where it is silent (each restated where used):
* SortDesc is stable: active rows ascending, then inactive rows ascending.
* A query head h belongs to routing group g = h // (Hq/Hk), which is also its
  KV head (section 3.1 Eq. 2, G = (Hq/Hk)*d).
* Causal attention is bottom-right aligned: query row t sees keys j with
  j <= t + (Tk - Tq) (Appendix B, Algorithm 4's query-key offset).
* The activation phi of Eq. 3 is SiLU (SwiGLU FFN).
* A query row with no valid key outputs 0 (the online softmax leaves its state
  at zero, Appendix B, implementation of attention).
* The router's reshape of 2 N_G logits into N_G pairs takes consecutive
  entries (2g, 2g + 1), and an argmax tie keeps class 0, so the group runs
  (section 3.1 Eq. 4 and 5).

Every function is pinned by ``tests/test_oracle.py`` against closed forms,
library routines, the page's naive gather-scatter formulations (Appendix A),
hand-worked fixtures and invariants; none is "parity unpinned".
"""
from __future__ import annotations

import math
from typing import Optional, Sequence

import numpy as np

# ---------------------------------------------------------------------------
# bfloat16 <-> float64
# ---------------------------------------------------------------------------


def from_bf16(bits) -> np.ndarray:
    """Exact float64 value of bfloat16 bit patterns."""
    b = np.asarray(bits, dtype=np.uint16)
    return (b.astype(np.uint32) << 16).view(np.float32).astype(np.float64)


def round_bf16(x) -> np.ndarray:
    """float64 -> nearest bfloat16 value (ties to even), returned as float64.

    bfloat16 keeps 8 significant bits. Writing x = m * 2**e with 0.5 <= |m| < 1,
    the result is rint(m * 256) / 256 * 2**e; numpy's rint rounds halves to
    even. Values below the smallest normal keep the normal spacing 2**-133,
    which is exact for the magnitudes the tests use.
    """
    x = np.asarray(x, dtype=np.float64)
    m, e = np.frexp(x)
    e = np.maximum(e, -125)          # subnormal range: fixed spacing
    m = np.ldexp(x, -e)
    return np.ldexp(np.rint(m * 256.0) / 256.0, e)


def to_bf16_bits(x) -> np.ndarray:
    """float64 -> bfloat16 bits, ties to even (via the exact bf16 value)."""
    v = round_bf16(x).astype(np.float32)   # exact: v has <= 8 significant bits
    return (v.view(np.uint32) >> 16).astype(np.uint16)


# ---------------------------------------------------------------------------
# Mask reordering (section 3.3 Eq. 7; Appendix B Algorithm 1)
# ---------------------------------------------------------------------------


def reorder(mask) -> tuple:
    """Per routing column, the row order that puts active rows first.

    mask: [B][T][NG] (nonzero = active). A routing column is mask[b, :, g]
    (Algorithm 1 keeps one column per (b, g); for a GEMM the caller passes
    B=1 with the flattened token dimension).

    Returns (perm [B][NG][T] int32, counts [B][NG] int32) with
    perm[b, g, :counts[b, g]] the active rows in ascending order and
    perm[b, g, counts[b, g]:] the inactive rows in ascending order, so that the
    reordered column mask[b, perm[b, g, j], g] is 1 exactly for j < counts
    (the relation between the reordered mask and the index I in Appendix B).
    """
    mask = np.asarray(mask)
    if mask.ndim != 3:
        raise ValueError("mask must be [B][T][NG]")
    B, T, NG = mask.shape
    perm = np.empty((B, NG, T), dtype=np.int32)
    counts = np.empty((B, NG), dtype=np.int32)
    for b in range(B):
        for g in range(NG):
            active = []
            inactive = []
            for t in range(T):
                (active if mask[b, t, g] != 0 else inactive).append(t)
            perm[b, g, :] = active + inactive
            counts[b, g] = len(active)
    return perm, counts


# ---------------------------------------------------------------------------
# GEMMs (section 3.3: C = A B^T with A [M][K], B [N][K])
# ---------------------------------------------------------------------------


def expand(mask2d, G: int) -> np.ndarray:
    """Repeat every mask column G times: [M][NG] -> boolean [M][NG*G].

    This is the group gating written as a mask over features, the meaning of
    the group-wise product in section 3.1 Eq. 2 and Eq. 3.
    """
    return np.repeat(np.asarray(mask2d) != 0, G, axis=1)


def gemm_mn(A_bits, B_bits, mask2d, G: int) -> np.ndarray:
    """N-axis routed GEMM (GEMM-MN, Appendix B Algorithm 2; Figure 1).

    C[m, n] = sum_k A[m, k] * B[n, k] if token m keeps group n // G, else +0.
    A: [M][K] bf16 bits; B: [N][K] bf16 bits; mask2d: [M][N/G].
    """
    A = from_bf16(A_bits)
    B = from_bf16(B_bits)
    if B.shape[0] % G:
        raise ValueError("N must be a multiple of G")
    keep = expand(mask2d, G)
    if keep.shape != (A.shape[0], B.shape[0]):
        raise ValueError("mask shape does not match [M][N/G]")
    return np.where(keep, A @ B.T, 0.0)


def gemm_k(A_bits, B_bits, mask2d, G: int) -> np.ndarray:
    """K-axis routed GEMM (GEMM-K, Appendix B Eq. 21 and Algorithm 3).

    C[m, n] = sum_g mask[m, g] * sum_{k in group g} A[m, k] * B[n, k],
    i.e. the dense product after zeroing every inactive K-group of A's row.
    A: [M][K]; B: [N][K]; mask2d: [M][K/G]. All M x N entries are defined.
    """
    A = from_bf16(A_bits)
    B = from_bf16(B_bits)
    if A.shape[1] % G:
        raise ValueError("K must be a multiple of G")
    keep = expand(mask2d, G)
    if keep.shape != A.shape:
        raise ValueError("mask shape does not match [M][K/G]")
    return np.where(keep, A, 0.0) @ B.T


def silu(x) -> np.ndarray:
    """SiLU(x) = x / (1 + exp(-x)), the reading of phi in section 3.1 Eq. 3."""
    x = np.asarray(x, dtype=np.float64)
    with np.errstate(over="ignore"):
        return x / (1.0 + np.exp(-x))


def swiglu(gate, up) -> np.ndarray:
    """phi(gate) * up, elementwise (section 3.1 Eq. 3)."""
    return silu(gate) * np.asarray(up, dtype=np.float64)


# ---------------------------------------------------------------------------
# Attention (section 3.1 Eq. 1-2; Appendix B Algorithm 4)
# ---------------------------------------------------------------------------


def attention(Q_bits, K_bits, V_bits, mask, causal: bool = True,
              leftpad: Optional[Sequence[int]] = None,
              scale: Optional[float] = None,
              queries: Optional[Sequence[tuple]] = None,
              q_tile: int = 128) -> np.ndarray:
    """Head-group-masked GQA attention.

    Q: [B][Tq][Hq][d]; K, V: [B][Tk][Hk][d] (bf16 bits); mask: [B][Tq][NG]
    with NG routing groups, a multiple of Hk that divides Hq (NG = Hk: one
    group per KV head, section 3.1 Eq. 2; NG > Hk: the finer sub-GQA groups,
    down to one query head each). Query head h uses KV head h // (Hq/Hk) and
    is gated by mask[b, t, h // (Hq/NG)].
    For an active (b, t, h) the valid keys are j in [jmin, jmax) with
    jmin = leftpad[b] (0 without leftpad) and jmax = t + (Tk - Tq) + 1 when
    causal, Tk otherwise; o = sum_j softmax_j(scale * q.k_j) v_j over the valid
    keys, computed exactly (maximum subtracted, two passes). No valid key, or an
    inactive group, gives o = 0. scale defaults to 1/sqrt(d).

    queries: optional list of (b, t) pairs; only those rows are computed and
    the result is [len(queries)][Hq][d]. Otherwise the result is
    [B][Tq][Hq][d]. Query rows are processed in blocks of q_tile.
    """
    Q = np.asarray(Q_bits)
    K = np.asarray(K_bits)
    V = np.asarray(V_bits)
    B, Tq, Hq, d = Q.shape
    _, Tk, Hk, _ = K.shape
    if Hq % Hk:
        raise ValueError("Hq must be a multiple of Hk")
    mask = np.asarray(mask)
    NG = mask.shape[2] if mask.ndim == 3 else -1
    if mask.shape[:2] != (B, Tq) or NG < Hk or NG % Hk or Hq % NG:
        raise ValueError("mask must be [B][Tq][NG] with NG a multiple of Hk dividing Hq")
    rep = Hq // Hk
    hpg = Hq // NG  # query heads per routing group
    if scale is None:
        scale = 1.0 / math.sqrt(d)
    delta = Tk - Tq
    if queries is None:
        sel = [(b, t) for b in range(B) for t in range(Tq)]
    else:
        sel = [(int(b), int(t)) for b, t in queries]
    out = np.zeros((len(sel), Hq, d), dtype=np.float64)
    keys = np.arange(Tk)
    by_batch = {}
    for i, (b, t) in enumerate(sel):
        by_batch.setdefault(b, []).append((i, t))
    for b, items in by_batch.items():
        jmin = int(leftpad[b]) if leftpad is not None else 0
        for g in range(Hk):
            Kg = from_bf16(K[b, :, g, :])            # [Tk][d]
            Vg = from_bf16(V[b, :, g, :])
            for h in range(g * rep, (g + 1) * rep):
                act = [(i, t) for (i, t) in items if mask[b, t, h // hpg] != 0]
                for s0 in range(0, len(act), q_tile):
                    blk = act[s0:s0 + q_tile]
                    idx = np.array([i for i, _ in blk])
                    ts = np.array([t for _, t in blk])
                    valid = keys[None, :] >= jmin
                    if causal:
                        valid = valid & (keys[None, :] <= ts[:, None] + delta)
                    has_key = valid.any(axis=1)
                    q = from_bf16(Q[b, ts, h, :])          # [n][d]
                    s = (q @ Kg.T) * scale                  # [n][Tk]
                    s = np.where(valid, s, -np.inf)
                    mx = np.where(has_key, s.max(axis=1, initial=-np.inf), 0.0)
                    p = np.where(valid, np.exp(s - mx[:, None]), 0.0)
                    z = p.sum(axis=1)
                    o = (p @ Vg) / np.where(has_key, z, 1.0)[:, None]
                    out[idx, h, :] = np.where(has_key[:, None], o, 0.0)
    if queries is None:
        return out.reshape(B, Tq, Hq, d)
    return out


# ---------------------------------------------------------------------------
# Sub-layer compositions (section 3.1 Eq. 1-3)
# ---------------------------------------------------------------------------


def ffn_layer(X_bits, Wg_bits, Wu_bits, Wd_bits, mask_ffn, G: int,
              fused: bool = True):
    """Masked SwiGLU FFN: y = ((phi(X Wg^T) * (X Wu^T)) gated by M_ffn) Wd^T.

    mask_ffn: [M][D'/G]. Returns (h, y): h is the gated intermediate
    (bf16-rounded, as stored between the two GEMMs) and y the fp64 output.
    fused=True feeds the fp64 gate/up values to SwiGLU (one rounding, of h);
    fused=False first rounds gate and up to bf16, as two separate GEMM-MN
    calls that store bf16 would.
    """
    gate = gemm_mn(X_bits, Wg_bits, mask_ffn, G)
    up = gemm_mn(X_bits, Wu_bits, mask_ffn, G)
    if not fused:
        gate = round_bf16(gate)
        up = round_bf16(up)
    h = round_bf16(swiglu(gate, up))
    y = gemm_k(to_bf16_bits(h), Wd_bits, mask_ffn, G)
    return h, y


def attn_layer(X_bits, Wq_bits, K_bits, V_bits, Wo_bits, mask_attn,
               Hq: int, Hk: int, d: int, causal: bool = True):
    """Masked attention sub-layer for batch B (Eq. 1-2).

    X: [B*T][D]; K, V: [B][Tk][Hk][d] (the dense K/V projections, which the
    mask never prunes); mask_attn: [B][T][Hk]. Returns (q, o, y): q and o are
    the bf16-rounded stored intermediates, y the fp64 output.
    """
    B, T, _ = mask_attn.shape
    G = (Hq // Hk) * d
    m2 = mask_attn.reshape(B * T, Hk)
    q = round_bf16(gemm_mn(X_bits, Wq_bits, m2, G))
    o = attention(to_bf16_bits(q).reshape(B, T, Hq, d), K_bits, V_bits,
                  mask_attn, causal=causal)
    o = round_bf16(o)
    y = gemm_k(to_bf16_bits(o).reshape(B * T, Hq * d), Wo_bits, m2, G)
    return q, o, y


# ---------------------------------------------------------------------------
# Work counts (algorithmic FLOPs and bytes of the routed operators)
# ---------------------------------------------------------------------------


def router_logits(X_bits, W1_bits, W2_bits) -> np.ndarray:
    """The bottleneck router's logits, section 3.1 "Routing Components", Eq. 4:
    R = reshape(X W1 W2) to [M][N_G][2].

    X [M][D]; the page's W1 (D x r) and W2 (r x 2 N_G) arrive in this
    library's weight convention, [out][in]: W1_bits [r][D] and W2_bits
    [2 N_G][r]. The reshape of each row's 2 N_G logits to N_G pairs takes
    consecutive entries: pair g is (column 2g, column 2g + 1), classes 0 and 1.
    """
    x = from_bf16(X_bits)
    w1 = from_bf16(W1_bits)
    w2 = from_bf16(W2_bits)
    R = (x @ w1.T) @ w2.T                     # [M][2 N_G]
    return R.reshape(R.shape[0], -1, 2)


def router_mask(X_bits, W1_bits, W2_bits) -> np.ndarray:
    """Inference routing decision, section 3.1 Eq. 5: group g of token m is
    executed (mask 1) when the argmax over the two classes of R[m, g] is class
    0. A tie keeps class 0, the first maximum (numpy's argmax convention).
    Returns uint8 [M][N_G]."""
    R = router_logits(X_bits, W1_bits, W2_bits)
    return (np.argmax(R, axis=-1) == 0).astype(np.uint8)


def flops_gemm_mn(mask2d, K: int, G: int) -> int:
    """2*K per active (row, output column): 2*K*G per active (row, group)."""
    return 2 * K * G * int(np.count_nonzero(np.asarray(mask2d)))


def flops_gemm_k(mask2d, N: int, G: int) -> int:
    """2*N per active (row, reduction index): 2*N*G per active (row, group)."""
    return 2 * N * G * int(np.count_nonzero(np.asarray(mask2d)))


def flops_attention(mask, Tk: int, Hq: int, d: int, causal: bool = True,
                    leftpad=None) -> int:
    """4*d FLOPs (QK^T and PV) per valid key of every active (b, t, h)."""
    mask = np.asarray(mask)
    B, Tq, Hk = mask.shape
    rep = Hq // Hk
    total = 0
    for b in range(B):
        jmin = int(leftpad[b]) if leftpad is not None else 0
        for t in range(Tq):
            jmax = t + (Tk - Tq) + 1 if causal else Tk
            nk = max(0, min(jmax, Tk) - jmin)
            total += int(np.count_nonzero(mask[b, t, :])) * rep * 4 * d * nk
    return total


def decode_bytes(mask_attn, mask_ffn, D: int, Hq: int, Hk: int, d: int,
                 G_ffn: int, Tk: int) -> int:
    """HBM bytes a decode step must read (bf16 weights and KV), for B sequences
    with one new token each: masks [B][Hk] and [B][NG_ffn] (a single row is one
    sequence).

    The W_q rows and W_o columns of an attention group (G_attn x D each), and
    the G_ffn rows of W_gate and W_up and G_ffn columns of W_down of an FFN
    group, are read once if any of the B tokens keeps the group. Every
    sequence reads its own K and V cache (Tk x d each) for every group its
    token keeps.
    """
    ma = np.atleast_2d(np.asarray(mask_attn)) != 0
    mf = np.atleast_2d(np.asarray(mask_ffn)) != 0
    G_attn = (Hq // Hk) * d
    weights = 0
    for g in range(ma.shape[1]):
        if ma[:, g].any():
            weights += 2 * (2 * G_attn * D)
    for g in range(mf.shape[1]):
        if mf[:, g].any():
            weights += 2 * (3 * G_ffn * D)
    kv = 0
    for b in range(ma.shape[0]):
        for g in range(ma.shape[1]):
            if ma[b, g]:
                kv += 2 * (2 * Tk * d)
    return weights + kv
