"""Seeded random shapes of GEMM-K (WIDE Appendix B, Eq. 21) through both entry
points: every tile path the launcher picks (256-wide tiles with or without a
K-split, 4-wave half-width tails, group sizes below a 64-deep stage, and the
pattern-sorted rows) against the oracle on sampled rows, and bitwise repeats."""
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


def random_case(seed):
    """A valid shape: N % 128 == 0, G % 16 == 0, K = G * groups with at most 512
    groups; M spans a ragged last row tile; the mask density is drawn too."""
    r = np.random.default_rng(seed)
    G = int(r.choice([16, 32, 48, 64, 128, 192, 256, 640]))
    NG = int(r.integers(1, max(2, min(40, 4096 // G)) + 1))
    K = G * NG
    N = 128 * int(r.integers(1, 13))
    M = int(r.integers(5, 2600))
    p = float(r.choice([0.1, 0.5, 0.9]))
    return M, N, K, G, p


@pytest.mark.parametrize("seed", range(12))
def test_gemm_k_random_shapes(seed):
    import masked_group_mask_amd as mg
    M, N, K, G, p = random_case(seed)
    say("gemm_k random", seed, M, N, K, G, p)
    A = wl.random_bf16(seed + 1000, (M, K))
    B = wl.random_bf16(seed + 2000, (N, K), 0.05)
    mask = wl.random_mask(seed + 3000, (M, K // G), p)
    Ad, Bd, md = to_dev(A, torch), to_dev(B, torch), to_dev(mask, torch)
    rows = np.unique(np.concatenate([np.random.default_rng(seed).choice(M, size=min(M, 40), replace=False),
                                     [0, M - 1]]))
    want = ref.gemm_k(A[rows], B, mask[rows], G)
    ws = torch.empty(max(mg.gemm_k_workspace_bytes(M, N, K), 16), dtype=torch.uint8, device="cuda")
    plain = mg.gemm_k(Ad, Bd, G, md)
    with_ws = mg.gemm_k(Ad, Bd, G, md, workspace=ws)
    order = mg.order_by_pattern(md)
    ordered = mg.gemm_k(Ad, Bd, G, md, order=order)
    again = mg.gemm_k(Ad, Bd, G, md, workspace=ws)
    torch.cuda.synchronize()
    for name, got in (("plain", plain), ("workspace", with_ws), ("ordered", ordered)):
        check_gemm(f32_of(got)[rows], want, f"gemm_k {name} {M}x{N}x{K} G{G} p{p}")
    assert torch.equal(with_ws, again), "GEMM-K with a workspace is not bitwise repeatable"
    # neither call splits K: the sorted rows give the token-order sums exactly
    assert torch.equal(ordered, plain), "GEMM-K over sorted rows differs from token order"
