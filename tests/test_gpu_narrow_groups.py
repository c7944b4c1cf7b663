"""GPU parity for group sizes below 64 (and not multiples of 64): the page
allows any G = 2^k with k >= 4 (section 3.1, Eq. 3), and its group-size sweep
starts at 16. GEMM-MN then covers a group with tiles wider than the group
(outputs past the group are not stored); GEMM-K takes each lane's A chunk
predicate from its own (row, group) bit, a 64-deep stage spanning 64 / G
groups. Bars as in the other parity tests."""
import numpy as np
import pytest

from oracle import wide_ref as ref
from masked_group_mask_amd import workloads as wl

from helpers import check_bf16_store, check_gemm, f32_of, say, to_dev, bits_of

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


MN_CASES = [(300, 256, 512, 16), (1000, 384, 1024, 32), (777, 384, 256, 48), (600, 480, 512, 96),
            (257, 64, 640, 16)]


@pytest.mark.parametrize("scheduled", [False, True])
@pytest.mark.parametrize("M,N,K,G", MN_CASES)
def test_gemm_mn_narrow_groups(M, N, K, G, scheduled):
    A = wl.random_bf16(M + 1, (M, K))
    B = wl.random_bf16(N + 2, (N, K), 0.05)
    mask = wl.random_mask(M + G, (M, N // G), 0.5)
    mask[:2] = 0
    say("gemm_mn narrow", M, N, K, G, "scheduled" if scheduled else "plain")
    md = to_dev(mask, torch)
    perm, counts = W().reorder(md[None])
    ws = None
    if scheduled:
        nb = W().gemm_mn_workspace_bytes(M, N, K, G)
        ws = torch.full((max(nb, 16) // 4,), float("nan"), dtype=torch.float32, device="cuda")
    out = torch.zeros((M, N), dtype=torch.float32, device="cuda")
    W().gemm_mn(to_dev(A, torch), to_dev(B, torch), G, perm=perm[0], counts=counts[0], out=out, workspace=ws)
    torch.cuda.synchronize()
    keep = ref.expand(mask, G)
    check_gemm(f32_of(out), ref.gemm_mn(A, B, mask, G), f"gemm_mn G={G}")
    assert (out.cpu().numpy().view(np.uint32)[~keep] == 0).all(), "an inactive entry was written"


@pytest.mark.parametrize("M,N,K,G", [(500, 256, 768, 16), (640, 384, 512, 32), (300, 192, 1024, 48)])
def test_gemm_mn_swiglu_narrow_groups(M, N, K, G):
    A = wl.random_bf16(M + 3, (M, K))
    Wg = wl.random_bf16(N + 4, (N, K), 0.05)
    Wu = wl.random_bf16(N + 5, (N, K), 0.05)
    mask = wl.random_mask(M + 7, (M, N // G), 0.5)
    say("swiglu narrow", M, N, K, G)
    perm, counts = W().reorder(to_dev(mask, torch)[None])
    h = W().gemm_mn_swiglu(to_dev(A, torch), to_dev(Wg, torch), to_dev(Wu, torch), G, perm=perm[0],
                           counts=counts[0])
    torch.cuda.synchronize()
    keep = ref.expand(mask, G)
    want = ref.swiglu(ref.gemm_mn(A, Wg, mask, G), ref.gemm_mn(A, Wu, mask, G))
    check_bf16_store(bits_of(h)[keep], want[keep], f"swiglu G={G}")
    assert (bits_of(h)[~keep] == 0).all()


K_CASES = [(300, 256, 512, 16), (1000, 384, 1024, 32), (513, 256, 1536, 48), (256, 512, 2048, 32)]


@pytest.mark.parametrize("beta", [0, 1])
@pytest.mark.parametrize("M,N,K,G", K_CASES)
def test_gemm_k_narrow_groups(M, N, K, G, beta):
    A = wl.random_bf16(M + 11, (M, K))
    B = wl.random_bf16(N + 12, (N, K), 0.05)
    mask = wl.random_mask(M + 13, (M, K // G), 0.5)
    mask[:3] = 0
    C0 = ref.from_bf16(wl.random_bf16(14, (M, N)).view(np.uint16)).astype(np.float32)
    say("gemm_k narrow", M, N, K, G, "beta", beta)
    Ad, Bd, md = to_dev(A, torch), to_dev(B, torch), to_dev(mask, torch)
    out = to_dev(C0, torch) if beta else torch.full((M, N), float("nan"), device="cuda")
    W().gemm_k(Ad, Bd, G, md, out=out, beta=beta)
    need = W().gemm_k_workspace_bytes(M, N, K)
    outs = [out]
    if need:
        ws = torch.full((need // 4,), float("nan"), dtype=torch.float32, device="cuda")
        o2 = to_dev(C0, torch) if beta else torch.full((M, N), float("nan"), device="cuda")
        W().gemm_k(Ad, Bd, G, md, out=o2, beta=beta, workspace=ws)
        outs.append(o2)
    torch.cuda.synchronize()
    want = ref.gemm_k(A, B, mask, G) + (C0 if beta else 0)
    for o in outs:
        check_gemm(f32_of(o), want, f"gemm_k G={G} beta={beta}")
    if not beta:
        assert (outs[0].cpu().numpy()[:3] == 0).all()


@pytest.mark.parametrize("Mt", [1, 3])
@pytest.mark.parametrize("G", [16, 32])
def test_gemv_narrow_groups(Mt, G):
    K, N = 1024, 512
    A = wl.random_bf16(Mt + 20, (Mt, K))
    B = wl.random_bf16(21, (N, K), 0.05)
    Bk = wl.random_bf16(22, (N, K), 0.05)
    mn_mask = wl.random_mask(23 + Mt, (Mt, N // G), 0.5)
    k_mask = wl.random_mask(24 + Mt, (Mt, K // G), 0.5)
    say("gemv narrow", Mt, G)
    out = W().gemm_mn(to_dev(A, torch), to_dev(B, torch), G, mask=to_dev(mn_mask, torch), out_dtype=torch.float32)
    y = W().gemm_k(to_dev(A, torch), to_dev(Bk, torch), G, to_dev(k_mask, torch))
    torch.cuda.synchronize()
    check_gemm(f32_of(out), ref.gemm_mn(A, B, mn_mask, G), f"gemv_mn G={G}")
    check_gemm(f32_of(y), ref.gemm_k(A, Bk, k_mask, G), f"gemv_k G={G}")
