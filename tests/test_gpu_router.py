"""GPU parity of the bottleneck router and its routing decision (section 3.1,
Eq. 4 and 5), against the oracle.

The decision is a comparison of two fp32 logits, so it is checked in three
parts: the GPU's mask is exactly its own decision rule applied to its own
logits (R0 >= R1, a tie runs the group); its logits agree with the oracle's
exact ones within the GEMM tolerance, max error eps; and wherever the exact
margin |R0 - R1| exceeds 2 eps the decision is the oracle's, bit for bit
(within 2 eps of a tie either decision is a correct rounding). The reorder
that follows is bit-exact against the oracle's reorder of the GPU's mask.
"""
import numpy as np
import pytest

from oracle import wide_ref as ref
from masked_group_mask_amd import workloads as wl

from helpers import check_gemm, say, to_dev

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


def run_and_check(X, W1, W2, B, what):
    M, D = X.shape
    NG = W2.shape[0] // 2
    T = M // B
    mask, perm, counts, logits = W().router(to_dev(X, torch), to_dev(W1, torch), to_dev(W2, torch), B=B,
                                            with_logits=True, with_reorder=True)
    torch.cuda.synchronize()
    m = mask.cpu().numpy().reshape(M, NG)
    lg = logits.cpu().numpy().astype(np.float64).reshape(M, NG, 2)
    # 1. the mask is the decision rule on the GPU's own logits
    assert np.array_equal(m, (lg[..., 0] >= lg[..., 1]).astype(np.uint8)), f"{what}: mask vs own logits"
    # 2. logits within tolerance of the exact ones
    want = ref.router_logits(X, W1, W2)
    check_gemm(lg.reshape(M, -1), want.reshape(M, -1), f"{what} logits")
    eps = float(np.max(np.abs(lg - want)))
    # 3. away from ties the decision is the oracle's
    margin = want[..., 0] - want[..., 1]
    clear = np.abs(margin) > 2 * eps
    assert clear.mean() > 0.99, f"{what}: too many near-ties ({1 - clear.mean():.4f})"
    assert np.array_equal(m[clear], ref.router_mask(X, W1, W2)[clear]), f"{what}: decisions"
    # 4. the reorder of that mask
    p_want, c_want = ref.reorder(m.reshape(B, T, NG))
    assert np.array_equal(perm.cpu().numpy(), p_want), f"{what}: perm"
    assert np.array_equal(counts.cpu().numpy(), c_want), f"{what}: counts"
    # the mask does not depend on whether logits or the reorder are requested
    m2, p2, c2, l2 = W().router(to_dev(X, torch), to_dev(W1, torch), to_dev(W2, torch), B=B,
                                with_logits=False, with_reorder=False)
    torch.cuda.synchronize()
    assert p2 is None and c2 is None and l2 is None
    assert np.array_equal(m2.cpu().numpy().reshape(M, NG), m), f"{what}: mask-only call"
    return m


@pytest.mark.parametrize("B,T,D,r,NG", [
    (1, 64, 256, 16, 8),       # one workgroup of 32 tokens twice
    (2, 77, 200, 32, 5),       # ragged token tail, D not a multiple of 32
    (1, 300, 1024, 48, 136),   # many groups
    (3, 33, 512, 64, 256),     # largest rank, W2 at the staging limit
])
def test_router_parity(B, T, D, r, NG):
    M = B * T
    X = wl.random_bf16(300 + D, (M, D))
    W1, W2 = wl.router_weights(301 + r, D, r, NG)
    say("router", B, T, D, r, NG)
    m = run_and_check(X, W1, W2, B, f"router {B}x{T} D={D} r={r} NG={NG}")
    assert 0.2 < m.mean() < 0.8


def test_router_ties_run_the_group():
    M, D, r, NG = 96, 512, 32, 16
    X = wl.random_bf16(310, (M, D))
    W1, W2 = wl.router_weights(311, D, r, NG)
    W2[1::2] = W2[0::2]             # both classes of every group identical: every pair ties
    say("router ties")
    mask, _, _, _ = W().router(to_dev(X, torch), to_dev(W1, torch), to_dev(W2, torch), with_reorder=False)
    torch.cuda.synchronize()
    assert mask.cpu().numpy().all()


@pytest.mark.parametrize("NG", [8, 136])   # attention groups (KV heads) and FFN groups, G_ffn = 128
def test_router_full_size_qwen14b(NG):
    """Qwen3-14B-shaped prefill: 8192 tokens, hidden 5120, rank 32; every token."""
    M, D, r = 8192, 5120, 32
    X = wl.make_layer(wl.shape("qwen14b_prefill"), seed=0, parts=())["x"]
    W1, W2 = wl.router_weights(320 + NG, D, r, NG)
    say("router full size", NG)
    run_and_check(X, W1, W2, 1, f"router qwen14b NG={NG}")
