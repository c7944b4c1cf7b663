"""GPU parity of GEMM-K computed group by group from the reorder (WIDE
Appendix B, Eq. 21 and Algorithm 3): the same product as the mask-driven
GEMM-K, checked against the oracle at the GEMM bar. The partial tiles are
added with atomics, so results are compared at the bar, never bitwise; rows
that keep no group must be exact zeros (beta 0) or untouched (beta 1)."""
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


def routed(mask_dev):
    perm, counts = W().reorder(mask_dev[None])
    return perm[0], counts[0]


CASES = [  # M, N, K, G
    (1000, 256, 1280, 640),     # 2 groups, ragged last row tile
    (300, 512, 2560, 640),      # 4 groups, one row tile
    (2304, 512, 5120, 640),     # 8 groups (the Qwen3-14B attention group size)
    (777, 768, 1024, 128),      # 8 groups of 128
    (513, 256, 4096, 256),      # 16 groups
    (600, 384, 8704, 64),       # 136 groups; N % 256 != 0: 128-wide tiles
    (257, 128, 512, 64),        # 8 groups, 128-wide tiles, one row past a tile
]


@pytest.mark.parametrize("p", [0.5, 0.25])
@pytest.mark.parametrize("M,N,K,G", CASES)
def test_gemm_k_grouped(M, N, K, G, p):
    A = wl.random_bf16(M + 1, (M, K))
    B = wl.random_bf16(N + 2, (N, K), 0.05)
    mask = wl.random_mask(M + K + 3, (M, K // G), p)
    mask[:2] = 0
    say("gemm_k grouped", M, N, K, G, p)
    Ad, Bd, md = to_dev(A, torch), to_dev(B, torch), to_dev(mask, torch)
    perm, counts = routed(md)
    got = W().gemm_k_grouped(Ad, Bd, G, perm, counts, out=torch.full((M, N), float("nan"), device="cuda"))
    plain = W().gemm_k(Ad, Bd, G, md)
    torch.cuda.synchronize()
    want = ref.gemm_k(A, B, mask, G)
    check_gemm(f32_of(got), want, f"gemm_k grouped {M}x{N}x{K} G{G}")
    check_gemm(f32_of(got), f32_of(plain), "grouped vs token-order kernel")
    assert (got.cpu().numpy()[:2] == 0).all()


@pytest.mark.parametrize("M,N,K,G", [(1000, 256, 1280, 640), (600, 384, 8704, 64)])
def test_gemm_k_grouped_beta1(M, N, K, G):
    A = wl.random_bf16(M + 11, (M, K))
    B = wl.random_bf16(N + 12, (N, K), 0.05)
    mask = wl.random_mask(M + 13, (M, K // G), 0.5)
    mask[:3] = 0
    C0 = ref.from_bf16(wl.random_bf16(14, (M, N)).view(np.uint16)).astype(np.float32)
    say("gemm_k grouped beta 1", M, N, K, G)
    md = to_dev(mask, torch)
    perm, counts = routed(md)
    out = to_dev(C0, torch)
    W().gemm_k_grouped(to_dev(A, torch), to_dev(B, torch), G, perm, counts, out=out, beta=1)
    torch.cuda.synchronize()
    got = f32_of(out)
    check_gemm(got, ref.gemm_k(A, B, mask, G) + C0, "grouped, beta 1")
    assert np.array_equal(out.cpu().numpy()[:3], C0[:3]), "rows in no group must be left as they were"


@pytest.mark.parametrize("p", [0.0, 1.0])
def test_gemm_k_grouped_all_or_nothing(p):
    M, N, K, G = 400, 256, 2560, 640
    A = wl.random_bf16(41, (M, K))
    B = wl.random_bf16(42, (N, K), 0.05)
    mask = np.full((M, K // G), int(p), np.uint8)
    md = to_dev(mask, torch)
    perm, counts = routed(md)
    say("gemm_k grouped all/none", p)
    got = W().gemm_k_grouped(to_dev(A, torch), to_dev(B, torch), G, perm, counts,
                             out=torch.full((M, N), float("nan"), device="cuda"))
    torch.cuda.synchronize()
    if p == 0:
        assert (f32_of(got) == 0).all()
    else:
        check_gemm(f32_of(got), ref.from_bf16(A) @ ref.from_bf16(B).T, "grouped all-ones = dense")


def test_gemm_k_grouped_one_group_switched_off():
    """Group 2 kept by no row: its tiles all exit at level 0 and its columns
    of A (filled with NaN here) are never read."""
    M, N, K, G = 700, 256, 2560, 640
    A = wl.random_bf16(71, (M, K))
    A[:, 2 * G:3 * G] = 0x7FC0  # bf16 NaN
    B = wl.random_bf16(72, (N, K), 0.05)
    mask = wl.random_mask(73, (M, K // G), 0.5)
    mask[:, 2] = 0
    md = to_dev(mask, torch)
    perm, counts = routed(md)
    say("gemm_k grouped, group 2 off, its A columns NaN")
    got = W().gemm_k_grouped(to_dev(A, torch), to_dev(B, torch), G, perm, counts)
    torch.cuda.synchronize()
    A_clean = A.copy()
    A_clean[:, 2 * G:3 * G] = 0
    check_gemm(f32_of(got), ref.gemm_k(A_clean, B, mask, G), "group 2 off")


def test_gemm_k_grouped_perm_entry_out_of_range_is_dropped():
    """A perm entry outside [0, M) is skipped, never dereferenced: its row
    misses that one group's partial, every other (row, group) is summed."""
    M, N, K, G = 600, 256, 1280, 640
    A = wl.random_bf16(81, (M, K))
    B = wl.random_bf16(82, (N, K), 0.05)
    mask = wl.random_mask(83, (M, K // G), 0.5)
    md = to_dev(mask, torch)
    perm, counts = routed(md)
    g0 = 1
    row = int(perm[g0, 0].item())
    perm[g0, 0] = M + 7
    say("gemm_k grouped, one perm entry out of range")
    got = W().gemm_k_grouped(to_dev(A, torch), to_dev(B, torch), G, perm, counts)
    torch.cuda.synchronize()
    m2 = mask.copy()
    m2[row, g0] = 0
    check_gemm(f32_of(got), ref.gemm_k(A, B, m2, G), "perm entry dropped")


FULL = [  # the Qwen3-14B prefill projections at T = 8192, 50% of the groups kept
    ("o_proj", 8192, 5120, 5120, 640),
    ("down_proj_g256", 8192, 5120, 17408, 256),
]


@pytest.mark.parametrize("name,M,N,K,G", FULL)
def test_gemm_k_grouped_full_size_sampled(name, M, N, K, G):
    """Full-size launch; the oracle computes 40 sampled rows, and the whole
    output is compared with the mask-driven kernel at the GEMM bar."""
    A = wl.random_bf16(91, (M, K))
    B = wl.random_bf16(92, (N, K), 0.05)
    mask = wl.random_mask(93, (M, K // G), 0.5)
    say("gemm_k grouped full size", name, M, N, K, G)
    Ad, Bd, md = to_dev(A, torch), to_dev(B, torch), to_dev(mask, torch)
    perm, counts = routed(md)
    got = W().gemm_k_grouped(Ad, Bd, G, perm, counts)
    plain = W().gemm_k(Ad, Bd, G, md)
    torch.cuda.synchronize()
    rows = np.sort(np.random.default_rng(94).choice(M, 40, replace=False))
    check_gemm(f32_of(got[torch.from_numpy(rows).cuda()]), ref.gemm_k(A[rows], B, mask[rows], G),
               f"{name} sampled rows")
    g, pl = got.cpu().numpy().astype(np.float64), plain.cpu().numpy().astype(np.float64)
    check_gemm(g, pl, f"{name} vs token-order kernel")
    del Ad, Bd, got, plain


def _random_k_cases(n=16, seed=2025):
    """Seeded random shapes for the three GEMM-K forms: group sizes 64 to 640
    (multiples of 64, so every form applies), N a multiple of 256 or only of
    128, M from 5 to 2500, activity from none to all, beta 0 or 1."""
    rng = np.random.default_rng(seed)
    cases = []
    while len(cases) < n:
        G = int(rng.choice([64, 128, 192, 256, 640]))
        NG = int(rng.integers(1, 9))
        N = int(rng.choice([128, 256, 384, 512, 768]))
        M = int(rng.choice([5, 77, 256, 300, 1000, 2500]))
        if M * N * NG * G > 2.5e9:     # keep the fp64 oracle quick
            continue
        cases.append((M, N, NG * G, G, float(rng.choice([0.0, 0.1, 0.5, 0.9, 1.0])), int(rng.integers(0, 2))))
    return cases


@pytest.mark.parametrize("M,N,K,G,p,beta", _random_k_cases())
def test_gemm_k_three_forms_random_shapes(M, N, K, G, p, beta):
    """Token order, pattern order (where N % 256 == 0 makes it apply) and the
    per-group form agree with the oracle on the same inputs."""
    A = wl.random_bf16(M + 600, (M, K))
    B = wl.random_bf16(N + 601, (N, K), 0.05)
    mask = wl.random_mask(M + N + K + 602, (M, K // G), p)
    C0 = ref.from_bf16(wl.random_bf16(603, (M, N)).view(np.uint16)).astype(np.float32)
    say("gemm_k three forms random", M, N, K, G, p, beta)
    Ad, Bd, md = to_dev(A, torch), to_dev(B, torch), to_dev(mask, torch)
    need = W().gemm_k_workspace_bytes(M, N, K)
    ws = torch.full((max(need, 16) // 4,), float("nan"), dtype=torch.float32, device="cuda")

    def fresh():
        return to_dev(C0, torch) if beta else torch.full((M, N), float("nan"), device="cuda")

    outs = {"token": W().gemm_k(Ad, Bd, G, md, out=fresh(), beta=beta, workspace=ws if need else None)}
    torch.cuda.synchronize()
    outs["ordered"] = W().gemm_k(Ad, Bd, G, md, out=fresh(), beta=beta, workspace=ws if need else None,
                                 order=W().order_by_pattern(md))
    perm, counts = routed(md)
    outs["grouped"] = W().gemm_k_grouped(Ad, Bd, G, perm, counts, out=fresh(), beta=beta)
    torch.cuda.synchronize()
    want = ref.gemm_k(A, B, mask, G) + (C0 if beta else 0)
    for name, o in outs.items():
        check_gemm(f32_of(o), want, f"gemm_k {name} {M}x{N}x{K} G{G} p{p} beta{beta}")


def test_prefill_layer_grouped_gemm_k_matches_token_order():
    """The layer with o_proj and down_proj computed group by group: q, o and
    h are bitwise those of the token-order layer, y_attn and y_ffn agree at
    the GEMM bar, and the all-ones reference keeps token order."""
    from masked_group_mask_amd.layer import PrefillLayer
    s = wl.shape("qwen14b_prefill", T=2048, p_attn=0.5, p_ffn=0.5, G_ffn=256)
    host = wl.make_layer(s, seed=11)
    say("layer, per-group GEMM-K vs token order", s.T)
    outs = {}
    for grouped in ((), ("o_proj", "down_proj")):
        layer = PrefillLayer(s, host, with_dense=True, grouped_k=grouped)
        for t in (layer.q, layer.o, layer.h):
            t.zero_()  # inactive entries are never written
        layer.step("masked")
        torch.cuda.synchronize()
        outs[grouped] = {k: getattr(layer, k).detach().clone() for k in ("q", "o", "h", "y_attn", "y_ffn")}
        assert not layer._grouped("o_proj", "dense")
        del layer
    a, b = outs[()], outs[("o_proj", "down_proj")]
    for k in ("q", "o", "h"):
        assert torch.equal(a[k], b[k]), k
    for k in ("y_attn", "y_ffn"):
        check_gemm(f32_of(b[k]), f32_of(a[k]), f"per-group {k} in the layer")
    with pytest.raises(ValueError):
        PrefillLayer(s, host, with_dense=False, ordered_k=("o_proj",), grouped_k=("o_proj",))
