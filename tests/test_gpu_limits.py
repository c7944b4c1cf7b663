"""GPU parity at the documented size limits of the C ABI.

- 32-bit offsets: gathered rows of A are addressed with 32-bit byte offsets,
  and M * lda * 2 just under 2^31 is accepted; the rows with the largest
  offsets are checked (GEMM-MN, and GEMM-K in token order, pattern order and
  per group).
- Group counts: 512 K-groups (GEMM-K's bit table holds 512) and 512 N-groups.
- Reorder: columns longer than the one-workgroup path and many columns.
- The allocation-free decode entry at its scratch limit.
Inputs come from the seeded generators; the big operands repeat a seeded
block so that they can be built quickly on the host.
"""
import numpy as np
import pytest

from oracle import wide_ref as ref
from masked_group_mask_amd import workloads as wl

from helpers import check_attn, check_gemm, f32_of, say, to_dev

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


def tiled_bf16(seed, rows, cols, block=1024, std=1.0):
    """rows x cols bf16 bits: a seeded block of `block` rows repeated."""
    blk = wl.random_bf16(seed, (block, cols), std)
    reps = (rows + block - 1) // block
    return np.ascontiguousarray(np.tile(blk, (reps, 1))[:rows])


# M * K * 2 = 2,147,450,880 < 2^31: the largest A the 32-bit row offsets allow
M_BIG, K_BIG = 65535, 16384


@pytest.fixture(scope="module")
def big():
    say("building the 2 GiB operand", M_BIG, K_BIG)
    A = tiled_bf16(700, M_BIG, K_BIG)
    B = wl.random_bf16(701, (256, K_BIG), 0.05)
    Ad, Bd = to_dev(A, torch), to_dev(B, torch)
    rows = np.array([0, 1, 1023, 1024, 40000, M_BIG - 257, M_BIG - 2, M_BIG - 1])
    yield A, B, Ad, Bd, rows
    del Ad, Bd
    torch.cuda.empty_cache()


def test_gemm_mn_rows_near_2gib(big):
    A, B, Ad, Bd, rows = big
    G = 128
    mask = wl.random_mask(702, (M_BIG, 256 // G), 0.5)
    mask[rows[-1]] = 1
    md = to_dev(mask, torch)
    perm, counts = W().reorder(md[None])
    say("gemm_mn, A of 2 GiB")
    out = torch.zeros((M_BIG, 256), dtype=torch.float32, device="cuda")
    W().gemm_mn(Ad, Bd, G, perm=perm[0], counts=counts[0], out=out)
    torch.cuda.synchronize()
    got = f32_of(out[torch.from_numpy(rows).cuda()])
    check_gemm(got, ref.gemm_mn(A[rows], B, mask[rows], G), "gemm_mn rows near 2 GiB")


@pytest.mark.parametrize("form,N", [("token", 256), ("token", 640), ("token", 384), ("ordered", 256),
                                    ("grouped", 256)])
def test_gemm_k_rows_near_2gib(big, form, N):
    """N = 640 and 384: 256 row tiles x two column tiles of 320 or 192 fill
    two rounds of 256 CUs, so the 320- and 192-wide token-order kernels run."""
    A, B, Ad, Bd, rows = big
    if N != 256:
        B = wl.random_bf16(704 + N, (N, K_BIG), 0.05)
        Bd = to_dev(B, torch)
    G = 128
    mask = wl.random_mask(703, (M_BIG, K_BIG // G), 0.5)
    mask[rows[-1]] = 1
    md = to_dev(mask, torch)
    say("gemm_k, A of 2 GiB", form, N)
    out = torch.full((M_BIG, N), float("nan"), dtype=torch.float32, device="cuda")
    if form == "grouped":
        perm, counts = W().reorder(md[None])
        W().gemm_k_grouped(Ad, Bd, G, perm[0], counts[0], out=out)
    else:
        order = W().order_by_pattern(md) if form == "ordered" else None
        need = W().gemm_k_workspace_bytes(M_BIG, N, K_BIG)
        ws = torch.empty(max(need, 16), dtype=torch.uint8, device="cuda")
        W().gemm_k(Ad, Bd, G, md, out=out, workspace=ws if need else None, order=order)
    torch.cuda.synchronize()
    got = f32_of(out[torch.from_numpy(rows).cuda()])
    check_gemm(got, ref.gemm_k(A[rows], B, mask[rows], G), f"gemm_k {form} rows near 2 GiB")


@pytest.mark.parametrize("form", ["token", "ordered"])
def test_gemm_k_512_groups(form):
    M, N, G = 300, 256, 16
    K = 512 * G
    A = wl.random_bf16(710, (M, K))
    B = wl.random_bf16(711, (N, K), 0.05)
    mask = wl.random_mask(712, (M, K // G), 0.5)
    md = to_dev(mask, torch)
    say("gemm_k with 512 groups", form)
    order = None
    if form == "ordered":
        # the ordered kernel takes multiples of 64: run it at G = 64 over 512 groups
        G = 64
        K = 512 * G
        A = wl.random_bf16(713, (M, K))
        B = wl.random_bf16(714, (N, K), 0.05)
        mask = wl.random_mask(715, (M, K // G), 0.5)
        md = to_dev(mask, torch)
        order = W().order_by_pattern(md)
    got = W().gemm_k(to_dev(A, torch), to_dev(B, torch), G, md, order=order)
    torch.cuda.synchronize()
    check_gemm(f32_of(got), ref.gemm_k(A, B, mask, G), f"gemm_k 512 groups {form}")


def test_gemm_mn_512_groups():
    M, K, G = 300, 256, 16
    N = 512 * G
    A = wl.random_bf16(720, (M, K))
    B = wl.random_bf16(721, (N, K), 0.05)
    mask = wl.random_mask(722, (M, N // G), 0.5)
    perm, counts = W().reorder(to_dev(mask, torch)[None])
    say("gemm_mn with 512 groups")
    out = torch.zeros((M, N), dtype=torch.float32, device="cuda")
    W().gemm_mn(to_dev(A, torch), to_dev(B, torch), G, perm=perm[0], counts=counts[0], out=out)
    torch.cuda.synchronize()
    check_gemm(f32_of(out), ref.gemm_mn(A, B, mask, G), "gemm_mn 512 groups")


@pytest.mark.parametrize("B,T,NG", [(1, 70000, 3), (2, 40000, 9), (300, 100, 17), (1, 16385, 512)])
def test_reorder_long_and_wide(B, T, NG):
    mask = wl.random_mask(730 + B + NG, (B, T, NG), 0.4)
    say("reorder", B, T, NG)
    perm, counts = W().reorder(to_dev(mask, torch))
    torch.cuda.synchronize()
    want_perm, want_counts = ref.reorder(mask)
    assert np.array_equal(counts.cpu().numpy(), want_counts)
    assert np.array_equal(perm.cpu().numpy(), want_perm)


def test_attn_noalloc_at_the_scratch_limit():
    """B * Hq * ceil(Tk / 64) = 63520 of the 63550 splits the built-in
    scratch holds."""
    B, Hq, Hk, d = 1, 32, 8, 128
    Tk = 1985 * 64
    assert B * Hq * ((Tk + 63) // 64) <= 63550
    Q = wl.random_bf16(740, (B, 1, Hq, d))
    K = tiled_bf16(741, Tk, Hk * d, block=4096).reshape(B, Tk, Hk, d)
    V = tiled_bf16(742, Tk, Hk * d, block=4096).reshape(B, Tk, Hk, d)
    mask = np.zeros((B, 1, Hk), np.uint8)
    mask[0, 0, [0, 3, 7]] = 1
    say("attn noalloc at the scratch limit", Tk)
    out = torch.zeros((B, 1, Hq, d), dtype=torch.float32, device="cuda")
    W().attn(to_dev(Q, torch), to_dev(K, torch), to_dev(V, torch), mask=to_dev(mask, torch), out=out,
             noalloc=True)
    torch.cuda.synchronize()
    check_attn(f32_of(out), ref.attention(Q, K, V, mask), "attn noalloc at the limit")
