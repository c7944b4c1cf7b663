"""Pins for the CPU oracle (runs without a GPU).

Each oracle function is checked against something other than itself: hand-
worked fixtures (tests/golden), a different library's routine (torch on the
CPU, float64), element-by-element brute force of the routed products (the
meaning of WIDE Appendix A's naive N- and K-axis pruning), closed forms and
invariants. Non-square shapes are used
throughout so that a transposed operand or a swapped index fails.
"""
import json
import math
import os

import numpy as np
import pytest
import torch
from hypothesis import given, settings, strategies as st

from oracle import wide_ref as ref
from masked_group_mask_amd import workloads as wl

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def load(name):
    with open(os.path.join(GOLDEN, name)) as f:
        return json.load(f)


def bits(x):
    """Exact bf16 bits of small test values (all exactly representable)."""
    x = np.asarray(x, dtype=np.float32)
    b = wl.f32_to_bf16_bits(x)
    assert np.array_equal(wl.bf16_bits_to_f32(b), x), "fixture value not bf16-exact"
    return b


# ---------------------------------------------------------------------------
# bf16 conversion
# ---------------------------------------------------------------------------

def test_bf16_known_bit_patterns():
    assert ref.to_bf16_bits(1.0) == 0x3F80
    assert ref.to_bf16_bits(-1.5) == 0xBFC0
    assert ref.to_bf16_bits(1.0 + 2.0 ** -8) == 0x3F80      # tie -> even
    assert ref.to_bf16_bits(1.0 + 3 * 2.0 ** -8) == 0x3F82  # tie -> even
    assert ref.to_bf16_bits(1.0 + 2.0 ** -8 + 2.0 ** -20) == 0x3F81
    assert ref.from_bf16(np.uint16(0x4049)) == 3.140625


def test_bf16_rounding_matches_torch():
    x = np.random.default_rng(1).standard_normal(20000) * np.float64(7.0)
    x = np.concatenate([x, x * 1e-30, x * 1e30, x * 2.0 ** -130]).astype(np.float32)
    # float32 inputs are exact in float64, so both round the same real number
    ours = ref.to_bf16_bits(x.astype(np.float64))
    theirs = torch.from_numpy(x).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    assert np.array_equal(ours, theirs)


# ---------------------------------------------------------------------------
# Reorder
# ---------------------------------------------------------------------------

def test_reorder_golden():
    fx = load("reorder_small.json")
    perm, counts = ref.reorder(np.array(fx["mask"], np.uint8))
    assert perm.tolist() == fx["perm"]
    assert counts.tolist() == fx["counts"]


def check_reorder_properties(mask):
    perm, counts = ref.reorder(mask)
    B, T, NG = mask.shape
    assert perm.shape == (B, NG, T) and counts.shape == (B, NG)
    for b in range(B):
        for g in range(NG):
            p = perm[b, g]
            c = counts[b, g]
            col = mask[b, :, g] != 0
            assert sorted(p.tolist()) == list(range(T))          # a permutation
            assert c == col.sum()                                  # counts = mask sum
            assert col[p[:c]].all() and not col[p[c:]].any()       # active prefix
            assert (np.diff(p[:c]) > 0).all() and (np.diff(p[c:]) > 0).all()  # stable
            # library routine: a stable argsort of "inactive" keys
            assert np.array_equal(p, np.argsort(~col, kind="stable"))
            # contiguous-run property: active rows in [r0, r1) sit at sorted
            # positions [a(r0), a(r1)) with a(r) = #active rows below r
            a = np.concatenate([[0], np.cumsum(col)])
            for r0, r1 in [(0, T), (T // 3, T // 2), (T // 2, T)]:
                run = p[a[r0]:a[r1]]
                assert np.array_equal(run, np.nonzero(col[r0:r1])[0] + r0)


@settings(max_examples=40, deadline=None)
@given(st.integers(1, 3), st.integers(1, 70), st.integers(1, 9), st.floats(0, 1),
       st.integers(0, 2 ** 31))
def test_reorder_properties(B, T, NG, p, seed):
    mask = (np.random.default_rng(seed).random((B, T, NG)) < p).astype(np.uint8)
    check_reorder_properties(mask)


def test_reorder_special_cases():
    # one row: perm is [0], count is the mask
    m = np.array([[[1, 0, 1]]], np.uint8)
    perm, counts = ref.reorder(m)
    assert perm.tolist() == [[[0], [0], [0]]] and counts.tolist() == [[1, 0, 1]]
    # nonzero values other than 1 count as active
    m = np.array([[[3], [0], [255]]], np.uint8)
    perm, counts = ref.reorder(m)
    assert perm.tolist() == [[[0, 2, 1]]] and counts.tolist() == [[2]]
    # all active / all inactive: identity order
    for v in (0, 1):
        perm, counts = ref.reorder(np.full((2, 5, 3), v, np.uint8))
        assert (perm == np.arange(5)).all() and (counts == 5 * v).all()


# ---------------------------------------------------------------------------
# GEMM-MN
# ---------------------------------------------------------------------------

def brute_n_axis(A, B, mask, G):
    """Element-by-element definition of N-axis routing (WIDE Appendix A, naive
    N-axis pruning): output (m, n) is the full dot product over k when token m
    keeps group n // G, and zero otherwise. Plain loops, no library routine."""
    M, K = A.shape
    N = B.shape[0]
    C = np.zeros((M, N))
    for m in range(M):
        for n in range(N):
            if mask[m][n // G] == 0:
                continue
            acc = 0.0
            for k in range(K):
                acc += A[m, k] * B[n, k]
            C[m, n] = acc
    return C


def test_gemm_mn_golden():
    fx = load("gemm_mn_small.json")
    C = ref.gemm_mn(bits(fx["A"]), bits(fx["B"]), np.array(fx["mask"]), fx["G"])
    assert C.tolist() == fx["C"]


@pytest.mark.parametrize("M,N,K,G", [(5, 48, 7, 16), (33, 64, 24, 32), (1, 32, 9, 16)])
def test_gemm_mn_pins(M, N, K, G):
    A = wl.random_bf16(1, (M, K))
    B = wl.random_bf16(2, (N, K))
    mask = wl.random_mask(3, (M, N // G))
    Af, Bf = ref.from_bf16(A), ref.from_bf16(B)
    C = ref.gemm_mn(A, B, mask, G)
    # element-by-element brute force (Appendix A, naive N-axis pruning)
    np.testing.assert_allclose(C, brute_n_axis(Af, Bf, mask, G), rtol=1e-12, atol=1e-12)
    # all-ones mask: the dense product, by another library
    dense = (torch.from_numpy(Af) @ torch.from_numpy(Bf).T).numpy()
    np.testing.assert_allclose(ref.gemm_mn(A, B, np.ones_like(mask), G), dense, rtol=1e-12, atol=1e-12)
    # inactive entries are exactly +0.0 (not -0.0)
    off = ~ref.expand(mask, G)
    assert (C[off] == 0).all() and not np.signbit(C[off]).any()
    assert (ref.gemm_mn(A, B, np.zeros_like(mask), G) == 0).all()
    # per group: a dense GEMM of the group's active rows
    for g in range(N // G):
        rows = np.nonzero(mask[:, g])[0]
        blk = Af[rows] @ Bf[g * G:(g + 1) * G].T
        np.testing.assert_allclose(C[np.ix_(rows, np.arange(g * G, (g + 1) * G))], blk, rtol=1e-12, atol=1e-12)


def test_gemm_mn_bruteforce_tiny():
    A = wl.random_bf16(4, (3, 4))
    B = wl.random_bf16(5, (4, 4))
    mask = np.array([[1, 0], [0, 1], [1, 1]])
    Af, Bf = ref.from_bf16(A), ref.from_bf16(B)
    C = ref.gemm_mn(A, B, mask, 2)
    for m in range(3):
        for n in range(4):
            want = sum(Af[m, k] * Bf[n, k] for k in range(4)) if mask[m, n // 2] else 0.0
            assert abs(C[m, n] - want) < 1e-12


# ---------------------------------------------------------------------------
# GEMM-K
# ---------------------------------------------------------------------------

def brute_k_axis(A, B, mask, G):
    """Element-by-element definition of K-axis routing (WIDE Appendix A, naive
    K-axis pruning): output (m, n) sums A[m, k] B[n, k] over the reduction
    indices k whose group k // G token m keeps. Plain loops."""
    M, K = A.shape
    N = B.shape[0]
    C = np.zeros((M, N))
    for m in range(M):
        for n in range(N):
            acc = 0.0
            for k in range(K):
                if mask[m][k // G] != 0:
                    acc += A[m, k] * B[n, k]
            C[m, n] = acc
    return C


def test_gemm_k_golden():
    fx = load("gemm_k_small.json")
    C = ref.gemm_k(bits(fx["A"]), bits(fx["B"]), np.array(fx["mask"]), fx["G"])
    assert C.tolist() == fx["C"]


@pytest.mark.parametrize("M,N,K,G", [(5, 9, 48, 16), (40, 24, 64, 32), (1, 7, 32, 16)])
def test_gemm_k_pins(M, N, K, G):
    A = wl.random_bf16(6, (M, K))
    B = wl.random_bf16(7, (N, K))
    mask = wl.random_mask(8, (M, K // G))
    Af, Bf = ref.from_bf16(A), ref.from_bf16(B)
    C = ref.gemm_k(A, B, mask, G)
    np.testing.assert_allclose(C, brute_k_axis(Af, Bf, mask, G), rtol=1e-12, atol=1e-12)
    dense = (torch.from_numpy(Af) @ torch.from_numpy(Bf).T).numpy()
    np.testing.assert_allclose(ref.gemm_k(A, B, np.ones_like(mask), G), dense, rtol=1e-12, atol=1e-12)
    assert (ref.gemm_k(A, B, np.zeros_like(mask), G) == 0).all()
    # Eq. 21 term by term: sum over groups of the gated partial products
    eq21 = np.zeros((M, N))
    for g in range(K // G):
        ks = slice(g * G, (g + 1) * G)
        eq21 += mask[:, g:g + 1] * (Af[:, ks] @ Bf[:, ks].T)
    np.testing.assert_allclose(C, eq21, rtol=1e-12, atol=1e-12)
    # additivity over disjoint masks
    m1 = mask * wl.random_mask(9, mask.shape)
    m2 = mask - m1
    np.testing.assert_allclose(ref.gemm_k(A, B, m1, G) + ref.gemm_k(A, B, m2, G), C, rtol=1e-12, atol=1e-12)


def test_gemm_k_bruteforce_tiny():
    A = wl.random_bf16(10, (2, 6))
    B = wl.random_bf16(11, (3, 6))
    mask = np.array([[1, 0, 1], [0, 1, 0]])
    Af, Bf = ref.from_bf16(A), ref.from_bf16(B)
    C = ref.gemm_k(A, B, mask, 2)
    for m in range(2):
        for n in range(3):
            want = sum(Af[m, k] * Bf[n, k] for k in range(6) if mask[m, k // 2])
            assert abs(C[m, n] - want) < 1e-12


# ---------------------------------------------------------------------------
# SwiGLU
# ---------------------------------------------------------------------------

def test_swiglu_closed_forms():
    assert ref.silu(0.0) == 0.0
    assert abs(ref.silu(1.0) - 0.7310585786300049) < 1e-15      # sigmoid(1)
    assert abs(ref.silu(-1.0) + 0.2689414213699951) < 1e-15
    assert abs(ref.silu(40.0) - 40.0) < 1e-12
    assert abs(ref.silu(-800.0)) == 0.0
    x = np.linspace(-12, 12, 101)
    np.testing.assert_allclose(ref.silu(x), torch.nn.functional.silu(torch.from_numpy(x)).numpy(), rtol=1e-14, atol=1e-300)
    u = np.linspace(3, -2, 101)
    np.testing.assert_allclose(ref.swiglu(x, u), ref.silu(x) * u)
    assert ref.swiglu(0.0, 5.0) == 0.0     # an inactive gate stays zero


# ---------------------------------------------------------------------------
# Attention
# ---------------------------------------------------------------------------

def test_attention_golden():
    fx = load("attention_small.json")
    Q, K, V = bits(fx["Q"]), bits(fx["K"]), bits(fx["V"])
    for case in fx["cases"]:
        O = ref.attention(Q, K, V, np.array(case["mask"]), causal=case["causal"],
                          leftpad=case["leftpad"], scale=fx["scale"])
        np.testing.assert_allclose(O, np.array(case["O"]), rtol=0, atol=1e-15)


def sdpa(Q, K, V, causal):
    q = torch.from_numpy(ref.from_bf16(Q)).permute(0, 2, 1, 3)
    k = torch.from_numpy(ref.from_bf16(K)).permute(0, 2, 1, 3)
    v = torch.from_numpy(ref.from_bf16(V)).permute(0, 2, 1, 3)
    o = torch.nn.functional.scaled_dot_product_attention(q, k, v, is_causal=causal, enable_gqa=True)
    return o.permute(0, 2, 1, 3).numpy()


@pytest.mark.parametrize("B,T,Hq,Hk,d", [(2, 37, 6, 2, 16), (1, 130, 4, 4, 8), (1, 20, 5, 1, 32)])
@pytest.mark.parametrize("causal", [True, False])
def test_attention_dense_matches_sdpa(B, T, Hq, Hk, d, causal):
    Q = wl.random_bf16(20, (B, T, Hq, d))
    K = wl.random_bf16(21, (B, T, Hk, d))
    V = wl.random_bf16(22, (B, T, Hk, d))
    O = ref.attention(Q, K, V, np.ones((B, T, Hk), np.uint8), causal=causal)
    np.testing.assert_allclose(O, sdpa(Q, K, V, causal), rtol=1e-10, atol=1e-12)


def test_attention_mask_gates_groups():
    B, T, Hq, Hk, d = 2, 33, 6, 3, 16
    Q = wl.random_bf16(23, (B, T, Hq, d))
    K = wl.random_bf16(24, (B, T, Hk, d))
    V = wl.random_bf16(25, (B, T, Hk, d))
    mask = wl.random_mask(26, (B, T, Hk))
    O = ref.attention(Q, K, V, mask)
    dense = sdpa(Q, K, V, True)
    rep = Hq // Hk
    keep = np.repeat(mask != 0, rep, axis=2)[..., None]      # head h -> group h // rep
    np.testing.assert_allclose(O, np.where(keep, dense, 0.0), rtol=1e-10, atol=1e-12)
    assert not np.signbit(O[~np.broadcast_to(keep, O.shape)]).any()


def test_attention_special_cases():
    d = 16
    # one key: every active row is V[0]
    Q = wl.random_bf16(27, (1, 1, 4, d))
    K = wl.random_bf16(28, (1, 1, 2, d))
    V = wl.random_bf16(29, (1, 1, 2, d))
    O = ref.attention(Q, K, V, np.ones((1, 1, 2), np.uint8))
    np.testing.assert_array_equal(O[0, 0], np.repeat(ref.from_bf16(V[0, 0]), 2, axis=0))
    # zero query: uniform weights -> mean of the valid values (causal prefix)
    T = 9
    Q = np.zeros((1, T, 2, d), np.uint16)
    K = wl.random_bf16(30, (1, T, 1, d))
    V = wl.random_bf16(31, (1, T, 1, d))
    O = ref.attention(Q, K, V, np.ones((1, T, 1), np.uint8))
    Vf = ref.from_bf16(V[0, :, 0])
    for t in range(T):
        np.testing.assert_allclose(O[0, t, 0], Vf[:t + 1].mean(axis=0), rtol=1e-13, atol=1e-14)


def test_attention_key_permutation_invariance():
    B, T, Hq, Hk, d = 1, 25, 4, 2, 16
    Q = wl.random_bf16(32, (B, T, Hq, d))
    K = wl.random_bf16(33, (B, T, Hk, d))
    V = wl.random_bf16(34, (B, T, Hk, d))
    mask = wl.random_mask(35, (B, T, Hk))
    p = np.random.default_rng(0).permutation(T)
    O1 = ref.attention(Q, K, V, mask, causal=False)
    O2 = ref.attention(Q, K[:, p], V[:, p], mask, causal=False)
    np.testing.assert_allclose(O1, O2, rtol=1e-12, atol=1e-13)


def test_attention_bottom_right_alignment_and_decode():
    """With Tq < Tk, query t sits at key position t + Tk - Tq: the result is the
    last Tq rows of the square causal problem; Tq = 1 sees every key."""
    B, Tk, Hq, Hk, d = 1, 40, 4, 2, 16
    Qfull = wl.random_bf16(36, (B, Tk, Hq, d))
    K = wl.random_bf16(37, (B, Tk, Hk, d))
    V = wl.random_bf16(38, (B, Tk, Hk, d))
    full = sdpa(Qfull, K, V, True)
    for Tq in (1, 7, Tk):
        O = ref.attention(Qfull[:, Tk - Tq:], K, V, np.ones((B, Tq, Hk), np.uint8))
        np.testing.assert_allclose(O, full[:, Tk - Tq:], rtol=1e-10, atol=1e-12)
    O1 = ref.attention(Qfull[:, -1:], K, V, np.ones((B, 1, Hk), np.uint8), causal=False)
    np.testing.assert_allclose(O1, full[:, -1:], rtol=1e-10, atol=1e-12)


def test_attention_leftpad():
    B, T, Hq, Hk, d = 2, 12, 2, 1, 16
    Q = wl.random_bf16(39, (B, T, Hq, d))
    K = wl.random_bf16(40, (B, T, Hk, d))
    V = wl.random_bf16(41, (B, T, Hk, d))
    ones = np.ones((B, T, Hk), np.uint8)
    O = ref.attention(Q, K, V, ones, leftpad=[0, 5])
    np.testing.assert_allclose(O[0], ref.attention(Q[:1], K[:1], V[:1], ones[:1])[0])
    # batch 1: keys below 5 are invalid; rows t < 5 have no valid key -> 0
    assert (O[1, :5] == 0).all()
    sub = ref.attention(Q[1:, 5:], K[1:, 5:], V[1:, 5:], ones[1:, 5:])
    np.testing.assert_allclose(O[1, 5:], sub[0], rtol=1e-12, atol=1e-13)


def test_attention_query_subset():
    B, T, Hq, Hk, d = 2, 30, 4, 2, 16
    Q = wl.random_bf16(42, (B, T, Hq, d))
    K = wl.random_bf16(43, (B, T, Hk, d))
    V = wl.random_bf16(44, (B, T, Hk, d))
    mask = wl.random_mask(45, (B, T, Hk))
    full = ref.attention(Q, K, V, mask)
    qs = [(1, 29), (0, 0), (1, 3), (0, 17)]
    part = ref.attention(Q, K, V, mask, queries=qs)
    for i, (b, t) in enumerate(qs):
        np.testing.assert_allclose(part[i], full[b, t], rtol=1e-13, atol=1e-15)


# ---------------------------------------------------------------------------
# Compositions and work counts
# ---------------------------------------------------------------------------

def test_ffn_layer_dense_and_empty():
    M, D, Dff, G = 9, 32, 64, 16
    X = wl.random_bf16(50, (M, D))
    Wg = wl.random_bf16(51, (Dff, D), 0.1)
    Wu = wl.random_bf16(52, (Dff, D), 0.1)
    Wd = wl.random_bf16(53, (D, Dff), 0.1)
    ones = np.ones((M, Dff // G), np.uint8)
    h, y = ref.ffn_layer(X, Wg, Wu, Wd, ones, G)
    x = torch.from_numpy(ref.from_bf16(X))
    hh = torch.nn.functional.silu(x @ torch.from_numpy(ref.from_bf16(Wg)).T) * (x @ torch.from_numpy(ref.from_bf16(Wu)).T)
    hh = torch.from_numpy(ref.round_bf16(hh.numpy()))
    np.testing.assert_allclose(h, hh.numpy(), rtol=0, atol=0)
    np.testing.assert_allclose(y, (hh @ torch.from_numpy(ref.from_bf16(Wd)).T).numpy(), rtol=1e-12, atol=1e-12)
    h0, y0 = ref.ffn_layer(X, Wg, Wu, Wd, np.zeros_like(ones), G)
    assert (h0 == 0).all() and (y0 == 0).all()


def test_attn_layer_empty_mask_is_zero():
    B, T, D, Hq, Hk, d = 1, 10, 32, 4, 2, 16
    X = wl.random_bf16(60, (B * T, D))
    Wq = wl.random_bf16(61, (Hq * d, D), 0.1)
    Wo = wl.random_bf16(62, (D, Hq * d), 0.1)
    K = wl.random_bf16(63, (B, T, Hk, d))
    V = wl.random_bf16(64, (B, T, Hk, d))
    q, o, y = ref.attn_layer(X, Wq, K, V, Wo, np.zeros((B, T, Hk), np.uint8), Hq, Hk, d)
    assert (q == 0).all() and (o == 0).all() and (y == 0).all()


def _attn_layer_inputs(seed, B=2, T=12, D=48, Hq=6, Hk=2, d=16):
    X = wl.random_bf16(seed, (B * T, D))
    Wq = wl.random_bf16(seed + 1, (Hq * d, D), 0.1)
    Wo = wl.random_bf16(seed + 2, (D, Hq * d), 0.1)
    K = wl.random_bf16(seed + 3, (B, T, Hk, d))
    V = wl.random_bf16(seed + 4, (B, T, Hk, d))
    return X, Wq, Wo, K, V


def _within_one_bf16_step(got, want):
    """got is a bf16 value within one rounding of the real number want."""
    return np.all(np.abs(got - want) <= 2.0 ** -8 * np.abs(want) + 1e-300)


def test_attn_layer_all_ones_is_the_dense_sublayer():
    """Section 3.1, Eq. 1-2 with every group kept: the masked attention
    sub-layer is the plain dense one. Each stage is checked against torch on
    the CPU (float64 matmul, SDPA with grouped KV heads), fed the oracle's own
    stored bf16 intermediate so a wrong group size, head mapping or reshape
    shows up as a mismatch."""
    B, T, D, Hq, Hk, d = 2, 12, 48, 6, 2, 16
    X, Wq, Wo, K, V = _attn_layer_inputs(600, B, T, D, Hq, Hk, d)
    ones = np.ones((B, T, Hk), np.uint8)
    q, o, y = ref.attn_layer(X, Wq, K, V, Wo, ones, Hq, Hk, d)
    tq = (torch.from_numpy(ref.from_bf16(X)) @ torch.from_numpy(ref.from_bf16(Wq)).T).numpy()
    assert _within_one_bf16_step(q, tq)
    q_bits = wl.f32_to_bf16_bits(q.astype(np.float32)).reshape(B, T, Hq, d)
    to = sdpa(q_bits, K, V, True)
    assert _within_one_bf16_step(o.reshape(B, T, Hq, d), to)
    o_in = torch.from_numpy(o.reshape(B * T, Hq * d))
    ty = (o_in @ torch.from_numpy(ref.from_bf16(Wo)).T).numpy()
    np.testing.assert_allclose(y, ty, rtol=1e-12, atol=1e-12)


def test_attn_layer_switched_off_group():
    """Switching one group off for some tokens zeroes exactly that group's
    heads in q and o for those tokens, leaves every other entry unchanged, and
    removes exactly that group's o_proj term from y (Eq. 2 and Eq. 21)."""
    B, T, D, Hq, Hk, d = 1, 10, 40, 6, 3, 16
    X, Wq, Wo, K, V = _attn_layer_inputs(610, B, T, D, Hq, Hk, d)
    ones = np.ones((B, T, Hk), np.uint8)
    q1, o1, y1 = ref.attn_layer(X, Wq, K, V, Wo, ones, Hq, Hk, d)
    g, toks = 1, [0, 3, 9]
    m = ones.copy()
    m[0, toks, g] = 0
    q, o, y = ref.attn_layer(X, Wq, K, V, Wo, m, Hq, Hk, d)
    G = (Hq // Hk) * d
    cols = np.zeros(Hq * d, bool)
    cols[g * G:(g + 1) * G] = True
    off = np.zeros((B * T, Hq * d), bool)
    off[np.ix_(toks, cols)] = True
    o2, o12 = o.reshape(B * T, -1), o1.reshape(B * T, -1)
    assert (q[off] == 0).all() and (o2[off] == 0).all()
    assert np.array_equal(q[~off], q1[~off]) and np.array_equal(o2[~off], o12[~off])
    wo = ref.from_bf16(Wo)
    removed = np.zeros_like(y1)
    removed[toks] = o12[toks][:, cols] @ wo[:, cols].T
    np.testing.assert_allclose(y, y1 - removed, rtol=1e-12, atol=1e-12)
    others = np.setdiff1d(np.arange(T), toks)
    assert np.array_equal(y[others], y1[others])


def test_work_counts():
    mask = wl.random_mask(70, (50, 6))
    assert ref.flops_gemm_mn(mask, 40, 16) == sum(2 * 40 for m in range(50) for n in range(96) if mask[m, n // 16])
    assert ref.flops_gemm_k(mask, 24, 16) == sum(2 * 24 for m in range(50) for k in range(96) if mask[m, k // 16])
    am = wl.random_mask(71, (2, 11, 3))
    want = 0
    for b in range(2):
        for t in range(11):
            for h in range(6):
                if am[b, t, h // 2]:
                    want += 4 * 8 * (t + (15 - 11) + 1)
    assert ref.flops_attention(am, 15, 6, 8) == want
    # one decode step of the Llama3.1-8B shape with half the groups on
    s = wl.shape("llama8b_decode")
    nb = ref.decode_bytes([1] * 4 + [0] * 4, [1] * 56 + [0] * 56, s.D, s.Hq, s.Hk, s.d, s.G_ffn, s.Tk)
    assert nb == 4 * (2 * 2 * 512 * 4096 + 2 * 2 * 16384 * 128) + 56 * 2 * 3 * 128 * 4096
    assert abs(nb / 1e6 - 243.27) < 0.01
    # two sequences: group weights are read once for the union of the tokens'
    # groups, K/V once per (sequence, kept group)
    nb2 = ref.decode_bytes([[1, 1, 0, 0], [0, 1, 1, 0]], [[1, 0, 0], [1, 1, 0]], D=64, Hq=8, Hk=4, d=16,
                           G_ffn=32, Tk=10)
    G_attn = 2 * 16
    assert nb2 == 3 * 2 * 2 * G_attn * 64 + 4 * 2 * 2 * 10 * 16 + 2 * 2 * 3 * 32 * 64


# ---------------------------------------------------------------------------
# Router (section 3.1, Eq. 4 and 5)
# ---------------------------------------------------------------------------

def _router_inputs(seed, M=7, D=40, r=4, NG=5):
    X = wl.random_bf16(seed, (M, D))
    W1 = wl.random_bf16(seed + 1, (r, D), D ** -0.5)
    W2 = wl.random_bf16(seed + 2, (2 * NG, r), r ** -0.5)
    return X, W1, W2


def test_router_logits_brute_force():
    """Element-by-element loops over the page's formula: R[m, g, c] is the
    product X W1 W2 at output column 2g + c (W1 [D][r] and W2 [r][2 N_G] in the
    page's orientation, i.e. the transposes of the stored arrays)."""
    X, W1, W2 = _router_inputs(200)
    x, w1, w2 = ref.from_bf16(X), ref.from_bf16(W1), ref.from_bf16(W2)
    M, D = x.shape
    r, NG = w1.shape[0], w2.shape[0] // 2
    R = ref.router_logits(X, W1, W2)
    assert R.shape == (M, NG, 2)
    for m in range(M):
        h = [sum(x[m, k] * w1[j, k] for k in range(D)) for j in range(r)]
        for g in range(NG):
            for c in range(2):
                want = sum(h[j] * w2[2 * g + c, j] for j in range(r))
                assert abs(R[m, g, c] - want) <= 1e-12 * (1 + abs(want))


def test_router_mask_decision_rule():
    X, W1, W2 = _router_inputs(210, M=50, NG=9)
    R = ref.router_logits(X, W1, W2)
    mask = ref.router_mask(X, W1, W2)
    assert mask.dtype == np.uint8 and mask.shape == (50, 9)
    assert np.array_equal(mask, (R[..., 0] >= R[..., 1]).astype(np.uint8))
    assert 0 < mask.mean() < 1


def test_router_ties_execute_and_swaps_flip():
    X, W1, W2 = _router_inputs(220, M=30, NG=6)
    tied = W2.copy()
    tied[1::2] = tied[0::2]                       # class 1 logits equal class 0: every pair ties
    assert ref.router_mask(X, W1, tied).all()      # a tie keeps class 0: executed
    swapped = W2.copy()
    swapped[0::2], swapped[1::2] = W2[1::2], W2[0::2]
    R = ref.router_logits(X, W1, W2)
    strict = R[..., 0] != R[..., 1]
    assert np.array_equal(ref.router_mask(X, W1, swapped)[strict], 1 - ref.router_mask(X, W1, W2)[strict])


def test_router_antisymmetric_pairs_are_a_sign_test():
    """With W2 row 2g+1 = -(row 2g), the decision is R[m, g, 0] >= 0, i.e. the
    sign of (X W1) w_g."""
    X, W1, W2 = _router_inputs(230, M=40, NG=7)
    anti = W2.copy()
    anti[1::2] = anti[0::2] ^ np.uint16(0x8000)   # negate the bf16 values exactly
    h = ref.from_bf16(X) @ ref.from_bf16(W1).T
    want = (h @ ref.from_bf16(W2[0::2]).T >= 0).astype(np.uint8)
    assert np.array_equal(ref.router_mask(X, W1, anti), want)


def test_router_mask_invariant_to_positive_scaling():
    X, W1, W2 = _router_inputs(240, M=40, NG=7)
    X2 = wl.f32_to_bf16_bits(ref.from_bf16(X).astype(np.float32) * np.float32(4.0))  # exact power of two
    assert np.array_equal(ref.router_mask(X2, W1, W2), ref.router_mask(X, W1, W2))


# ---------------------------------------------------------------------------
# Sub-GQA routing groups (section 3.1: G_attn down to one query head)
# ---------------------------------------------------------------------------

def _attn_inputs(seed, B=2, T=9, Hq=8, Hk=2, d=16):
    Q = wl.random_bf16(seed, (B, T, Hq, d))
    K = wl.random_bf16(seed + 1, (B, T, Hk, d))
    V = wl.random_bf16(seed + 2, (B, T, Hk, d))
    return Q, K, V


def test_attention_finer_groups_reduce_to_kv_groups():
    """Routing groups finer than the KV heads that all carry their KV head's
    decision give exactly the one-group-per-KV-head result."""
    Q, K, V = _attn_inputs(500)
    m = wl.random_mask(501, (2, 9, 2), 0.5)
    want = ref.attention(Q, K, V, m)
    for NG in (4, 8):
        fine = np.repeat(m, NG // 2, axis=2)
        assert np.array_equal(ref.attention(Q, K, V, fine), want)


def test_attention_per_head_mask_gates_only_its_head():
    """With one group per query head, switching a head's group off zeroes that
    head only; every other head equals the all-on result; flops count only
    the heads that run."""
    Q, K, V = _attn_inputs(510)
    on = np.ones((2, 9, 8), np.uint8)
    full = ref.attention(Q, K, V, on)
    m = on.copy()
    m[1, 4, 5] = 0
    m[0, :, 2] = 0
    got = ref.attention(Q, K, V, m)
    assert (got[1, 4, 5] == 0).all() and (got[0, :, 2] == 0).all()
    keep = np.ones_like(got, dtype=bool)
    keep[1, 4, 5] = False
    keep[0, :, 2] = False
    assert np.array_equal(got[keep], full[keep])
    assert ref.flops_attention(m, 9, 8, 16) == ref.flops_attention(on, 9, 8, 16) - 4 * 16 * (5 + sum(range(1, 10)))


def test_attention_rejects_groups_not_aligned_to_kv_heads():
    Q, K, V = _attn_inputs(520)
    with pytest.raises(ValueError):
        ref.attention(Q, K, V, np.ones((2, 9, 3), np.uint8))   # 3 groups: not a multiple of Hk = 2
    with pytest.raises(ValueError):
        ref.attention(Q, K, V, np.ones((2, 9, 1), np.uint8))   # fewer groups than KV heads
