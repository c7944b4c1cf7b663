"""GPU parity of the pattern order and of GEMM-K over pattern-sorted rows.

The order (wide_order_by_pattern) is index work: it must equal, bit for bit,
the stable sort of the rows by the Gray-code rank of their pattern over the
first min(NG, 8) groups. GEMM-K with an order is the same product as
without one (WIDE Appendix B, Eq. 21): it is checked against the oracle at
the GEMM bar and, without a K split, bitwise against the token-order kernel,
since the skipped work only ever added exact zeros.
"""
import numpy as np
import pytest

from oracle import wide_ref as ref
from masked_group_mask_amd import workloads as wl

from helpers import check_gemm, f32_of, say, to_dev

pytestmark = pytest.mark.gpu
torch = pytest.importorskip("torch")


@pytest.fixture(scope="module", autouse=True)
def gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import masked_group_mask_amd as mg
    mg.load()


def W():
    import masked_group_mask_amd as mg
    return mg


def gray_rank(pattern):
    """Position of a pattern in the reflected Gray code sequence: the
    inverse of g(i) = i ^ (i >> 1), i.e. the prefix XOR of the bits."""
    r = np.array(pattern, dtype=np.int64)
    shift = 1
    while shift < 64:
        r ^= r >> shift
        shift *= 2
    return r


def expected_order(mask):
    M, NG = mask.shape
    nb = min(NG, 8)
    bits = (mask[:, :nb] != 0).astype(np.int64)
    pattern = (bits << np.arange(nb - 1, -1, -1)).sum(axis=1) if nb else np.zeros(M, np.int64)
    return np.argsort(gray_rank(pattern), kind="stable").astype(np.int32)


def test_gray_rank_hand_worked():
    # Gray sequence of two bits: 00, 01, 11, 10
    assert gray_rank([0b00, 0b01, 0b11, 0b10]).tolist() == [0, 1, 2, 3]
    # three bits: g(5) = 5 ^ 2 = 7, g(6) = 6 ^ 3 = 5
    assert gray_rank([7, 5]).tolist() == [5, 6]
    m = np.array([[1, 0], [0, 0], [1, 1], [0, 1], [0, 0]], np.uint8)
    # patterns 10, 00, 11, 01, 00 -> ranks 3, 0, 2, 1, 0
    assert expected_order(m).tolist() == [1, 4, 3, 2, 0]


ORDER_CASES = [(1, 8, 0.5), (64, 8, 0.5), (1000, 3, 0.5), (1025, 8, 0.34), (8192, 8, 0.5),
               (5000, 136, 0.5), (3000, 1, 0.5), (700, 12, 0.9), (300, 8, 0.0), (300, 8, 1.0),
               (16384, 8, 0.5), (20000, 8, 0.5), (17000, 5, 0.5)]  # more rounds than keys kept in registers


@pytest.mark.parametrize("M,NG,p", ORDER_CASES)
def test_order_by_pattern_bit_exact(M, NG, p):
    mask = wl.random_mask(M + NG, (M, NG), p)
    mask[mask != 0] = np.random.default_rng(M).integers(1, 256, np.count_nonzero(mask), dtype=np.uint8)
    say("order_by_pattern", M, NG, p)
    got = W().order_by_pattern(to_dev(mask, torch))
    torch.cuda.synchronize()
    assert np.array_equal(got.cpu().numpy(), expected_order(mask))


ORDERED_CASES = [  # M, N, K, G
    (1000, 256, 1280, 640),     # 2 groups, ragged last row tile
    (300, 512, 2560, 640),      # 4 groups
    (2304, 512, 5120, 640),     # 8 groups (the Qwen3-14B attention group size)
    (777, 768, 1024, 128),      # 8 groups of 128
    (600, 256, 8704, 64),       # 136 groups: the order sees the first 8
    (513, 256, 4096, 256),      # 16 groups
]


@pytest.mark.parametrize("p", [0.5, 0.25])
@pytest.mark.parametrize("M,N,K,G", ORDERED_CASES)
def test_gemm_k_ordered(M, N, K, G, p):
    A = wl.random_bf16(M + 1, (M, K))
    B = wl.random_bf16(N + 2, (N, K), 0.05)
    mask = wl.random_mask(M + K + 3, (M, K // G), p)
    mask[:2] = 0
    say("gemm_k ordered", M, N, K, G, p)
    Ad, Bd, md = to_dev(A, torch), to_dev(B, torch), to_dev(mask, torch)
    order = W().order_by_pattern(md)
    got = W().gemm_k(Ad, Bd, G, md, out=torch.full((M, N), float("nan"), device="cuda"), order=order)
    plain = W().gemm_k(Ad, Bd, G, md)
    torch.cuda.synchronize()
    check_gemm(f32_of(got), ref.gemm_k(A, B, mask, G), f"gemm_k ordered {M}x{N}x{K} G{G}")
    assert torch.equal(got, plain), "ordered GEMM-K differs from the token-order kernel"
    assert (got.cpu().numpy()[:2] == 0).all()


def test_gemm_k_any_permutation():
    """Any permutation is a valid order (only the speed depends on it)."""
    M, N, K, G = 900, 256, 2560, 640
    A = wl.random_bf16(31, (M, K))
    B = wl.random_bf16(32, (N, K), 0.05)
    mask = wl.random_mask(33, (M, K // G), 0.5)
    Ad, Bd, md = to_dev(A, torch), to_dev(B, torch), to_dev(mask, torch)
    say("gemm_k random permutation and identity orders")
    plain = W().gemm_k(Ad, Bd, G, md)
    for order in (np.random.default_rng(5).permutation(M), np.arange(M)):
        got = W().gemm_k(Ad, Bd, G, md, order=to_dev(order.astype(np.int32), torch))
        torch.cuda.synchronize()
        assert torch.equal(got, plain)


@pytest.mark.parametrize("p", [0.0, 1.0])
def test_gemm_k_ordered_all_or_nothing(p):
    M, N, K, G = 400, 256, 2560, 640
    A = wl.random_bf16(41, (M, K))
    B = wl.random_bf16(42, (N, K), 0.05)
    mask = np.full((M, K // G), int(p), np.uint8)
    md = to_dev(mask, torch)
    say("gemm_k ordered all/none", p)
    got = W().gemm_k(to_dev(A, torch), to_dev(B, torch), G, md, order=W().order_by_pattern(md))
    torch.cuda.synchronize()
    if p == 0:
        assert (f32_of(got) == 0).all()
    else:
        check_gemm(f32_of(got), ref.from_bf16(A) @ ref.from_bf16(B).T, "ordered all-ones = dense")


KSPLIT_CASES = [(256, 256, 5120, 640), (1000, 512, 2560, 640), (4352, 4096, 1280, 640),
                (512, 768, 2048, 128)]


@pytest.mark.parametrize("beta", [0, 1])
@pytest.mark.parametrize("M,N,K,G", KSPLIT_CASES)
def test_gemm_k_ordered_ksplit(M, N, K, G, beta):
    """Ordered tiles with the K-split plan (the slices cover the tile's live
    steps); NaN-filled workspace, bitwise reproducible."""
    A = wl.random_bf16(M + 50, (M, K))
    B = wl.random_bf16(N + 51, (N, K), 0.05)
    mask = wl.random_mask(M + 52, (M, K // G), 0.5)
    mask[:3] = 0
    C0 = ref.from_bf16(wl.random_bf16(53, (M, N)).view(np.uint16)).astype(np.float32)
    need = W().gemm_k_workspace_bytes(M, N, K)
    assert need > 0
    say("gemm_k ordered ksplit", M, N, K, G, beta)
    Ad, Bd, md = to_dev(A, torch), to_dev(B, torch), to_dev(mask, torch)
    order = W().order_by_pattern(md)
    res = []
    for _ in range(2):
        ws = torch.full((need // 4,), float("nan"), dtype=torch.float32, device="cuda")
        out = to_dev(C0, torch) if beta else torch.full((M, N), float("nan"), device="cuda")
        W().gemm_k(Ad, Bd, G, md, out=out, beta=beta, workspace=ws, order=order)
        res.append(out)
    torch.cuda.synchronize()
    want = ref.gemm_k(A, B, mask, G) + (C0 if beta else 0)
    check_gemm(f32_of(res[0]), want, f"gemm_k ordered ksplit {M}x{N}x{K} beta={beta}")
    assert torch.equal(res[0], res[1])
    if not beta:
        assert (res[0].cpu().numpy()[:3] == 0).all()


def test_gemm_k_order_entry_out_of_range_is_dropped():
    """An order entry outside [0, M) is skipped, never dereferenced: the row
    it displaced stays as it was, every other row is right."""
    M, N, K, G = 600, 256, 1280, 640
    A = wl.random_bf16(61, (M, K))
    B = wl.random_bf16(62, (N, K), 0.05)
    mask = wl.random_mask(63, (M, K // G), 0.5)
    order = np.arange(M, dtype=np.int32)
    lost = 321
    order[lost] = M + 7
    say("gemm_k ordered, one order entry out of range")
    out = torch.full((M, N), -5.0, device="cuda")
    W().gemm_k(to_dev(A, torch), to_dev(B, torch), G, to_dev(mask, torch), out=out,
               order=to_dev(order, torch))
    torch.cuda.synchronize()
    got = f32_of(out)
    assert (got[lost] == -5.0).all()
    keep = np.arange(M) != lost
    check_gemm(got[keep], ref.gemm_k(A, B, mask, G)[keep], "rows with valid order entries")


def test_prefill_layer_ordered_o_proj_matches_token_order():
    """The layer with o_proj over pattern-sorted rows: every output but
    y_attn is bitwise that of the token-order layer,
    y_attn agrees at the GEMM bar (a K-split tile groups different rows), and
    the all-ones reference step still runs in token order."""
    from masked_group_mask_amd import workloads as wl2
    from masked_group_mask_amd.layer import PrefillLayer
    s = wl2.shape("qwen14b_prefill", T=2048, p_attn=0.5, p_ffn=0.5, G_ffn=128)
    host = wl2.make_layer(s, seed=9)
    say("layer, ordered o_proj vs token order", s.T)
    outs = {}
    for ordered in ((), ("o_proj",)):
        layer = PrefillLayer(s, host, with_dense=True, ordered_k=ordered)
        for t in (layer.q, layer.o, layer.h):
            t.zero_()  # inactive entries are never written
        layer.step("masked")
        torch.cuda.synchronize()
        outs[ordered] = {k: getattr(layer, k).detach().clone() for k in ("q", "o", "h", "y_attn", "y_ffn")}
        assert not layer._ordered("o_proj", "dense")
        del layer
    a, b = outs[()], outs[("o_proj",)]
    for k in ("q", "o", "h", "y_ffn"):
        assert torch.equal(a[k], b[k]), k
    check_gemm(f32_of(b["y_attn"]), f32_of(a["y_attn"]), "ordered o_proj in the layer")
