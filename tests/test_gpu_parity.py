"""GPU parity: every HIP entry point against the CPU oracle, through the C ABI.

Bars: reorder perm/counts bit-exact; GEMM fp32 outputs max|err| <= 1e-2 x RMS
of the oracle; attention fp32 outputs max|err| <= 2e-2; bf16-stored outputs
within one bf16 step of the oracle's rounded value; entries the method does not
compute are left bitwise untouched (the tests pre-zero them).
"""
import numpy as np
import pytest

from oracle import wide_ref as ref
from masked_group_mask_amd import workloads as wl

from helpers import (bits_of, check_attn, check_attn_bf16, check_bf16_store, check_gemm, f32_of,
                     say, to_dev)

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")


@pytest.fixture(scope="module", autouse=True)
def gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import masked_group_mask_amd as mg
    mg.load()   # raises if libwide.so is missing: no fallback exists
    return mg


def W():
    import masked_group_mask_amd as mg
    return mg


# ---------------------------------------------------------------------------
# Reorder
# ---------------------------------------------------------------------------

REORDER_CASES = [
    (1, 64, 8, 0.5), (1, 1, 3, 0.5), (1, 513, 112, 0.28), (2, 1031, 5, 0.7), (3, 700, 68, 0.5),
    (1, 4096, 64, 0.5), (1, 2000, 136, 0.0), (1, 2000, 17, 1.0), (4, 257, 8, 0.34),
    # rows held in registers: 16 and 32 chunks of 512 rows, a ragged last
    # chunk; then past the register budget (mask re-read per chunk)
    (1, 8192, 136, 0.5), (2, 6000, 20, 0.5), (2, 16000, 8, 0.4), (1, 9000, 40, 0.5),
    (1, 17000, 24, 0.5), (1, 16385, 3, 0.5),
]


@pytest.mark.parametrize("B,T,NG,p", REORDER_CASES)
def test_reorder_bit_exact(B, T, NG, p):
    say("reorder", B, T, NG, p)
    mask = wl.random_mask(100 + T + NG, (B, T, NG), p)
    if p == 0.5:
        mask[mask == 1] = 255       # any nonzero byte means active
    perm, counts = W().reorder(to_dev(mask, torch))
    torch.cuda.synchronize()
    want_p, want_c = ref.reorder(mask)
    assert np.array_equal(counts.cpu().numpy(), want_c)
    assert np.array_equal(perm.cpu().numpy(), want_p)


def test_reorder_full_size_llama8b_ffn_and_attention():
    s = wl.shape("llama8b_prefill")
    m = wl.draw_mask(np.random.default_rng(7), s.M, s.NG_ffn, s.p_ffn, "bern")[None]
    a = wl.draw_mask(np.random.default_rng(8), s.M, s.Hk, s.p_attn, "bern")[None]
    for mask in (m, a):
        say("reorder full", mask.shape)
        perm, counts = W().reorder(to_dev(mask, torch))
        torch.cuda.synchronize()
        want_c = mask.astype(bool).sum(axis=1).astype(np.int32)
        assert np.array_equal(counts.cpu().numpy(), want_c)
        # stable partition, checked per column with the library routine
        want_p = np.argsort(mask[0].T == 0, axis=1, kind="stable")
        assert np.array_equal(perm.cpu().numpy()[0], want_p)


def test_reorder_deterministic():
    mask = wl.random_mask(9, (1, 3000, 40), 0.5)
    d = to_dev(mask, torch)
    p1, c1 = W().reorder(d)
    p2, c2 = W().reorder(d)
    assert torch.equal(p1, p2) and torch.equal(c1, c2)


# ---------------------------------------------------------------------------
# GEMM-MN
# ---------------------------------------------------------------------------

def run_mn(A, B, mask2d, G, out_dtype, swiglu_up=None):
    say("gemm_mn", A.shape, B.shape, G, out_dtype, "swiglu" if swiglu_up is not None else "")
    md = to_dev(mask2d[None], torch)
    perm, counts = W().reorder(md)
    Ad, Bd = to_dev(A, torch), to_dev(B, torch)
    if swiglu_up is None:
        out = W().gemm_mn(Ad, Bd, G, perm=perm[0], counts=counts[0], out_dtype=out_dtype)
    else:
        out = W().gemm_mn_swiglu(Ad, Bd, to_dev(swiglu_up, torch), G, perm=perm[0],
                                 counts=counts[0], out_dtype=out_dtype)
    torch.cuda.synchronize()
    return out


MN_CASES = [  # M, N, K, G
    (64, 1024, 256, 128), (300, 512, 320, 128), (300, 512, 200, 64), (1000, 1280, 640, 640),
    (129, 256, 72, 256), (5, 128, 64, 128),
]


@pytest.mark.parametrize("M,N,K,G", MN_CASES)
def test_gemm_mn_fp32(M, N, K, G):
    A = wl.random_bf16(M + 1, (M, K))
    B = wl.random_bf16(N + 2, (N, K), 0.05)
    mask = wl.random_mask(M + N, (M, N // G), 0.5)
    out = run_mn(A, B, mask, G, torch.float32)
    got = f32_of(out)
    want = ref.gemm_mn(A, B, mask, G)
    check_gemm(got, want, f"gemm_mn {M}x{N}x{K} G{G}")
    off = ~ref.expand(mask, G)
    assert (out.cpu().numpy().view(np.uint32)[off] == 0).all(), "inactive entries were written"


@pytest.mark.parametrize("M,N,K", [(700, 512, 1024), (257, 1280, 640), (64, 256, 256)])
def test_depth_routing_single_group(M, N, K):
    """M-axis (depth) routing as the one-group case of both GEMMs: each token
    runs the whole projection or none of it (G = N for GEMM-MN, G = K for
    GEMM-K)."""
    A = wl.random_bf16(M + 11, (M, K))
    B = wl.random_bf16(N + 12, (N, K), 0.05)
    mask = wl.random_mask(M + 13, (M, 1), 0.5)
    mask[0, 0] = 0
    say("depth routing", M, N, K)
    out = run_mn(A, B, mask, N, torch.float32)
    check_gemm(f32_of(out), ref.gemm_mn(A, B, mask, N), f"depth gemm_mn {M}x{N}x{K}")
    assert (out.cpu().numpy().view(np.uint32)[mask[:, 0] == 0] == 0).all()
    Bk = wl.random_bf16(N + 14, (N, K), 0.05)
    yk = W().gemm_k(to_dev(A, torch), to_dev(Bk, torch), K, to_dev(mask, torch))
    torch.cuda.synchronize()
    check_gemm(f32_of(yk), ref.gemm_k(A, Bk, mask, K), f"depth gemm_k {M}x{N}x{K}")
    assert (yk.cpu().numpy()[mask[:, 0] == 0] == 0).all()


@pytest.mark.parametrize("G", [128, 640])
def test_gemm_mn_strided_operands(G):
    """Leading dimensions larger than the rows: A and B padded, and an odd ldc
    (ldc = N + 1) that rules out vector stores; the padding stays untouched."""
    M, N, K = 300, 2 * G, 320
    A = wl.random_bf16(60, (M, K))
    B = wl.random_bf16(61, (N, K), 0.05)
    mask = wl.random_mask(62, (M, N // G), 0.5)
    say("gemm_mn strided", M, N, K, G)
    Ap = torch.zeros((M, K + 8), dtype=torch.bfloat16, device="cuda")
    Bp = torch.zeros((N, K + 16), dtype=torch.bfloat16, device="cuda")
    Ap[:, :K] = to_dev(A, torch)
    Bp[:, :K] = to_dev(B, torch)
    Cp = torch.zeros((M, N + 1), dtype=torch.float32, device="cuda")
    perm, counts = W().reorder(to_dev(mask[None], torch))
    W().gemm_mn(Ap[:, :K], Bp[:, :K], G, perm=perm[0], counts=counts[0], out=Cp[:, :N])
    torch.cuda.synchronize()
    got = Cp.cpu().numpy()
    check_gemm(got[:, :N], ref.gemm_mn(A, B, mask, G), "gemm_mn strided")
    assert (got[:, N] == 0).all(), "the padding column was written"


@pytest.mark.parametrize("p", [0.0, 1.0])
def test_gemm_mn_all_or_nothing(p):
    M, N, K, G = 200, 256, 128, 128
    A = wl.random_bf16(1, (M, K))
    B = wl.random_bf16(2, (N, K), 0.05)
    mask = np.full((M, N // G), int(p), np.uint8)
    got = f32_of(run_mn(A, B, mask, G, torch.float32))
    if p == 0:
        assert (got == 0).all()
    else:
        dense = ref.from_bf16(A) @ ref.from_bf16(B).T
        check_gemm(got, dense, "all-ones = dense")


def test_gemm_mn_bf16_store():
    M, N, K, G = 257, 384, 256, 128
    A = wl.random_bf16(3, (M, K))
    B = wl.random_bf16(4, (N, K), 0.05)
    mask = wl.random_mask(5, (M, N // G), 0.5)
    out = run_mn(A, B, mask, G, torch.bfloat16)
    want = ref.gemm_mn(A, B, mask, G)
    keep = ref.expand(mask, G)
    flips = check_bf16_store(bits_of(out)[keep], want[keep], "gemm_mn bf16")
    assert flips < 0.02
    assert (bits_of(out)[~keep] == 0).all()


@pytest.mark.parametrize("M,N,K,G", [(64, 1024, 256, 128), (300, 512, 192, 64), (77, 640, 512, 128)])
@pytest.mark.parametrize("dt", ["f32", "bf16"])
def test_gemm_mn_swiglu(M, N, K, G, dt):
    A = wl.random_bf16(6, (M, K))
    Wg = wl.random_bf16(7, (N, K), 0.05)
    Wu = wl.random_bf16(8, (N, K), 0.05)
    mask = wl.random_mask(9, (M, N // G), 0.5)
    out = run_mn(A, Wg, mask, G, torch.float32 if dt == "f32" else torch.bfloat16, swiglu_up=Wu)
    want = ref.swiglu(ref.gemm_mn(A, Wg, mask, G), ref.gemm_mn(A, Wu, mask, G))
    keep = ref.expand(mask, G)
    if dt == "f32":
        check_gemm(f32_of(out), want, "swiglu f32")
        assert (out.cpu().numpy().view(np.uint32)[~keep] == 0).all()
    else:
        check_bf16_store(bits_of(out)[keep], want[keep], "swiglu bf16")
        assert (bits_of(out)[~keep] == 0).all()


def _mn_active_tiles(mask2d, G, bn_out, rows=256):
    """Active tiles of the scheduled GEMM-MN path, counted on the host from
    the mask: ceil(count_g / rows) row tiles times G / bn_out column tiles
    (rows = 320 for the 256-wide tiles, plain or fused SwiGLU)."""
    counts = mask2d.astype(bool).sum(axis=0)
    return int(((counts + rows - 1) // rows).sum()) * (G // bn_out)


def _run_mn_ws(Ad, Bd, Bu, perm, counts, G, out_dtype, ws, M, N):
    out = torch.zeros((M, N), dtype=out_dtype, device="cuda")
    if Bu is None:
        W().gemm_mn(Ad, Bd, G, perm=perm, counts=counts, out=out, workspace=ws)
    else:
        W().gemm_mn_swiglu(Ad, Bd, Bu, G, perm=perm, counts=counts, out=out, workspace=ws)
    return out


# M, N, K, G, swiglu, bn_out and rows of the tile the launcher picks, p(active)
MN_WS_CASES = [
    (1000, 1280, 1024, 640, False, 320, 256, 0.5),  # 320-wide tiles, 2 column tiles per group
    (700, 512, 2048, 128, True, 128, 320, 0.5),     # fused SwiGLU tile, 320 rows
    (300, 512, 1000, 64, False, 64, 256, 0.5),      # 4-wave 64-wide tile, K tail inside the last slice
    (5440, 4096, 1024, 128, True, 128, 320, 0.5),   # more tiles than CUs, a short last round
    (500, 640, 4096, 640, False, 320, 256, 0.5),    # 2 tiles in 8 slices
    (1500, 1024, 2048, 256, False, 256, 320, 0.5),  # 256-wide plain tile, 320 rows
    (900, 1024, 1000, 256, False, 256, 320, 0.5),   # 320 rows, K tail inside the last slice
    (2000, 1024, 1536, 256, False, 256, 320, 0.0),  # nothing active: the fixup finds no split tile
]


@pytest.mark.parametrize("M,N,K,G,swiglu,bn_out,rows,p", MN_WS_CASES)
@pytest.mark.parametrize("dt", ["f32", "bf16"])
def test_gemm_mn_scheduled_ksplit(M, N, K, G, swiglu, bn_out, rows, p, dt):
    """With a workspace the tiles are scheduled from counts on the device and
    the tiles of a partly filled last round are split along K (summed by a
    fixup kernel). The workspace starts as NaN garbage; entries of inactive
    (token, group) pairs stay untouched; two runs agree bit for bit."""
    A = wl.random_bf16(M + 90, (M, K))
    B = wl.random_bf16(N + 91, (N, K), 0.05)
    U = wl.random_bf16(N + 92, (N, K), 0.05) if swiglu else None
    mask = wl.random_mask(M + N + 93, (M, N // G), p)
    out_dtype = torch.float32 if dt == "f32" else torch.bfloat16
    need = W().gemm_mn_workspace_bytes(M, N, K, G, swiglu)
    assert need > 0
    cus = torch.cuda.get_device_properties(0).multi_processor_count
    A_t = _mn_active_tiles(mask, G, bn_out, rows)
    split = 0 < A_t % cus <= cus // 2
    if p > 0:
        assert split, f"{A_t} active tiles on {cus} CUs: this case must split its last round"
    say("gemm_mn scheduled", M, N, K, G, "swiglu" if swiglu else "", dt, "tiles", A_t, "split", split)
    perm, counts = W().reorder(to_dev(mask[None], torch))
    Ad, Bd = to_dev(A, torch), to_dev(B, torch)
    Bu = to_dev(U, torch) if swiglu else None
    outs = []
    for _ in range(2):
        ws = torch.full((need // 4,), float("nan"), dtype=torch.float32, device="cuda")
        outs.append(_run_mn_ws(Ad, Bd, Bu, perm[0], counts[0], G, out_dtype, ws, M, N))
    torch.cuda.synchronize()
    want = ref.gemm_mn(A, B, mask, G)
    if swiglu:
        want = ref.swiglu(want, ref.gemm_mn(A, U, mask, G))
    keep = ref.expand(mask, G)
    if dt == "f32":
        check_gemm(f32_of(outs[0]), want, f"gemm_mn scheduled {M}x{N}x{K} G{G}")
        assert (outs[0].cpu().numpy().view(np.uint32)[~keep] == 0).all(), "inactive entries were written"
    else:
        check_bf16_store(bits_of(outs[0])[keep], want[keep], f"gemm_mn scheduled bf16 {M}x{N}x{K}")
        assert (bits_of(outs[0])[~keep] == 0).all(), "inactive entries were written"
    assert torch.equal(outs[0], outs[1]), "scheduled GEMM-MN is not bitwise reproducible"


def test_gemm_mn_workspace_reused_across_shapes():
    """One workspace through consecutive calls of different shapes (the second
    smaller, then a SwiGLU call): stale headers and partials of the earlier
    call must not leak into the later ones."""
    cases = [(1000, 1280, 1024, 640, False), (300, 640, 1024, 640, False), (500, 512, 2048, 128, True)]
    need = max(W().gemm_mn_workspace_bytes(M, N, K, G, sw) for M, N, K, G, sw in cases)
    ws = torch.full((need // 4,), float("nan"), dtype=torch.float32, device="cuda")
    for i, (M, N, K, G, sw) in enumerate(cases):
        A = wl.random_bf16(200 + i, (M, K))
        B = wl.random_bf16(210 + i, (N, K), 0.05)
        U = wl.random_bf16(220 + i, (N, K), 0.05) if sw else None
        mask = wl.random_mask(230 + i, (M, N // G), 0.5)
        say("gemm_mn workspace reuse", i, M, N, K, G, sw)
        perm, counts = W().reorder(to_dev(mask[None], torch))
        Ad, Bd = to_dev(A, torch), to_dev(B, torch)
        Bu = to_dev(U, torch) if sw else None
        got = _run_mn_ws(Ad, Bd, Bu, perm[0], counts[0], G, torch.float32, ws, M, N)
        torch.cuda.synchronize()
        want = ref.gemm_mn(A, B, mask, G)
        if sw:
            want = ref.swiglu(want, ref.gemm_mn(A, U, mask, G))
        check_gemm(f32_of(got), want, f"gemm_mn workspace reuse {i}")
        assert (got.cpu().numpy().view(np.uint32)[~ref.expand(mask, G)] == 0).all()


@pytest.mark.parametrize("N,G,bn_out,rows", [(9216, 128, 128, 256), (20480, 256, 256, 320)])
def test_gemm_mn_scheduled_equals_plain_without_split(N, G, bn_out, rows):
    """When the last round is more than half full nothing is split: the
    scheduled path computes every tile exactly as the plain call does, so the
    two results agree bit for bit (only the tile order differs, and for
    256-wide tiles the scheduled path's 320 rows against the plain 256: each
    output's sum runs over the same products in the same order)."""
    M, K = 700, 1024
    A = wl.random_bf16(240, (M, K))
    B = wl.random_bf16(241, (N, K), 0.05)
    mask = wl.random_mask(242, (M, N // G), 0.5)
    cus = torch.cuda.get_device_properties(0).multi_processor_count
    A_t = _mn_active_tiles(mask, G, bn_out, rows)
    say("gemm_mn scheduled vs plain", M, N, K, G, "tiles", A_t, "cus", cus)
    if 0 < A_t % cus <= cus // 2:
        pytest.skip(f"{A_t} tiles on {cus} CUs would split")
    need = W().gemm_mn_workspace_bytes(M, N, K, G, False)
    assert need > 0
    perm, counts = W().reorder(to_dev(mask[None], torch))
    Ad, Bd = to_dev(A, torch), to_dev(B, torch)
    ws = torch.full((need // 4,), float("nan"), dtype=torch.float32, device="cuda")
    got = _run_mn_ws(Ad, Bd, None, perm[0], counts[0], G, torch.float32, ws, M, N)
    plain = _run_mn_ws(Ad, Bd, None, perm[0], counts[0], G, torch.float32, None, M, N)
    torch.cuda.synchronize()
    assert torch.equal(got, plain)
    check_gemm(f32_of(got), ref.gemm_mn(A, B, mask, G), "gemm_mn scheduled, no split")


@pytest.mark.parametrize("M", [1, 2, 3, 4])
@pytest.mark.parametrize("swiglu", [False, True])
@pytest.mark.parametrize("K", [512, 9000])  # one partial block; three blocks of 4096 with a ragged last one
def test_gemv_mn_mask_direct(M, swiglu, K):
    N, G = 1024, 128
    A = wl.random_bf16(10 + M, (M, K))
    B = wl.random_bf16(11, (N, K), 0.05)
    U = wl.random_bf16(12, (N, K), 0.05)
    mask = wl.random_mask(13 + M, (M, N // G), 0.5)
    say("gemv_mn", M, swiglu)
    Ad, Bd, md = to_dev(A, torch), to_dev(B, torch), to_dev(mask, torch)
    if swiglu:
        out = W().gemm_mn_swiglu(Ad, Bd, to_dev(U, torch), G, mask=md, out_dtype=torch.float32)
        want = ref.swiglu(ref.gemm_mn(A, B, mask, G), ref.gemm_mn(A, U, mask, G))
    else:
        out = W().gemm_mn(Ad, Bd, G, mask=md, out_dtype=torch.float32)
        want = ref.gemm_mn(A, B, mask, G)
    torch.cuda.synchronize()
    check_gemm(f32_of(out), want, "gemv_mn")
    assert (out.cpu().numpy().view(np.uint32)[~ref.expand(mask, G)] == 0).all()


# ---------------------------------------------------------------------------
# GEMM-K
# ---------------------------------------------------------------------------

K_CASES = [  # M, N, K, G
    (64, 256, 1024, 128), (300, 256, 512, 128), (300, 384, 640, 64), (1000, 128, 2560, 640),
    (129, 128, 512, 256), (5, 256, 256, 128),
    # 17 x 16 = 272 tiles of 256 x 256: on 256 CUs the 16 left over run as 32 half-width tiles
    (4352, 4096, 256, 128),
]


@pytest.mark.parametrize("M,N,K,G", K_CASES)
def test_gemm_k(M, N, K, G):
    A = wl.random_bf16(M + 3, (M, K))
    B = wl.random_bf16(N + 4, (N, K), 0.05)
    mask = wl.random_mask(M + K, (M, K // G), 0.5)
    say("gemm_k", M, N, K, G)
    out = W().gemm_k(to_dev(A, torch), to_dev(B, torch), G, to_dev(mask, torch))
    torch.cuda.synchronize()
    want = ref.gemm_k(A, B, mask, G)
    check_gemm(f32_of(out), want, f"gemm_k {M}x{N}x{K} G{G}")
    none = ~mask.any(axis=1)
    assert (out.cpu().numpy()[none] == 0).all()


def test_gemm_k_beta_and_determinism():
    M, N, K, G = 333, 256, 1024, 128
    A = wl.random_bf16(20, (M, K))
    B = wl.random_bf16(21, (N, K), 0.05)
    mask = wl.random_mask(22, (M, K // G), 0.4)
    C0 = wl.random_bf16(23, (M, N)).view(np.uint16)
    C0 = ref.from_bf16(C0).astype(np.float32)
    say("gemm_k beta")
    Ad, Bd, md = to_dev(A, torch), to_dev(B, torch), to_dev(mask, torch)
    out = to_dev(C0, torch)
    W().gemm_k(Ad, Bd, G, md, out=out, beta=1)
    r1 = W().gemm_k(Ad, Bd, G, md)
    r2 = W().gemm_k(Ad, Bd, G, md)
    torch.cuda.synchronize()
    want = ref.gemm_k(A, B, mask, G)
    check_gemm(f32_of(out), want + C0, "gemm_k beta=1")
    assert torch.equal(r1, r2), "GEMM-K is not bitwise reproducible"


def test_gemm_k_leftover_tiles_beta():
    """272 tiles of 256 x 256 on 256 CUs: the 16 left over run as 32 half-width
    workgroups in a second launch; beta = 1 must hold in both launches."""
    M, N, K, G = 4352, 4096, 256, 128
    A = wl.random_bf16(70, (M, K))
    B = wl.random_bf16(71, (N, K), 0.05)
    mask = wl.random_mask(72, (M, K // G), 0.5)
    C0 = ref.from_bf16(wl.random_bf16(73, (M, N)).view(np.uint16)).astype(np.float32)
    say("gemm_k leftover tiles beta=1")
    out = to_dev(C0, torch)
    W().gemm_k(to_dev(A, torch), to_dev(B, torch), G, to_dev(mask, torch), out=out, beta=1)
    torch.cuda.synchronize()
    check_gemm(f32_of(out), ref.gemm_k(A, B, mask, G) + C0, "gemm_k leftover tiles beta=1")


KSPLIT_CASES = [  # M, N, K, G; 256 x 256 tiles and the K slices the plan gives them on 256 CUs
    (256, 256, 4096, 128),    # 1 tile in 8 slices of 8 K-steps
    (512, 768, 2048, 128),    # 6 tiles in 4 slices
    (1000, 512, 1024, 64),    # 8 tiles, ragged last row tile, 2 slices
    (4352, 4096, 1024, 128),  # 272 tiles: 256 whole, the 16 left over in 2 slices
]


@pytest.mark.parametrize("beta", [0, 1])
@pytest.mark.parametrize("M,N,K,G", KSPLIT_CASES)
def test_gemm_k_ksplit(M, N, K, G, beta):
    """With a workspace the partly filled last round of tiles is split along
    K and a second kernel adds the slices; the workspace starts as NaN garbage,
    which must never reach the result."""
    A = wl.random_bf16(M + 80, (M, K))
    B = wl.random_bf16(N + 81, (N, K), 0.05)
    mask = wl.random_mask(M + K + 82, (M, K // G), 0.5)
    mask[:3] = 0  # rows with no active group
    C0 = ref.from_bf16(wl.random_bf16(83, (M, N)).view(np.uint16)).astype(np.float32)
    need = W().gemm_k_workspace_bytes(M, N, K)
    assert need > 0, "this shape must take the K-split plan"
    say("gemm_k ksplit", M, N, K, G, "beta", beta, "workspace", need)
    Ad, Bd, md = to_dev(A, torch), to_dev(B, torch), to_dev(mask, torch)
    results = []
    for _ in range(2):
        ws = torch.full((need // 4,), float("nan"), dtype=torch.float32, device="cuda")
        out = to_dev(C0, torch) if beta else torch.full((M, N), float("nan"), device="cuda")
        W().gemm_k(Ad, Bd, G, md, out=out, beta=beta, workspace=ws)
        results.append(out)
    torch.cuda.synchronize()
    want = ref.gemm_k(A, B, mask, G) + (C0 if beta else 0)
    check_gemm(f32_of(results[0]), want, f"gemm_k ksplit {M}x{N}x{K} G{G} beta={beta}")
    assert torch.equal(results[0], results[1]), "K-split GEMM-K is not bitwise reproducible"
    if not beta:
        assert (results[0].cpu().numpy()[:3] == 0).all()


WIDE_K_CASES = [  # M, N, K, G, activity
    # 8 x 32 = 256 tiles of 256 x 320 fill one round on 256 CUs: the 320-wide
    # kernel, with a ragged last row tile
    (2000, 10240, 512, 64, 0.5),
    (2048, 10240, 1280, 128, 0.3),
    (2000, 10240, 512 * 64, 64, 0.5),   # 512 groups: the most the bit table holds
    (2000, 10240, 1024, 256, 0.0),      # nothing active: exact zeros
    # groups narrower than a 64-deep stage: the same shape in 256 x 256 tiles
    (2000, 10240, 512, 32, 0.5),
    # 8 x 32 = 256 tiles of 256 x 192 fill one round where 256 x 256 tiles
    # (192) would not: the 192-wide kernel
    (2000, 6144, 512, 64, 0.5),
    (2000, 6144, 1024, 128, 0.0),
    (4096, 3072, 8192, 128, 0.5),       # the Llama3.2-3B down_proj shape
]


@pytest.mark.parametrize("M,N,K,G,p", WIDE_K_CASES)
@pytest.mark.parametrize("beta", [0, 1])
def test_gemm_k_round_filling_tiles(M, N, K, G, p, beta):
    """Shapes whose 256 x 320 (or 256 x 192) tiles fill whole rounds of the 256
    compute units run that kernel alone; rows across every row tile, the
    ragged tail and boundary rows are compared with the oracle; two runs agree
    bit for bit."""
    if torch.cuda.get_device_properties(0).multi_processor_count != 256:
        pytest.skip("tile rounds counted for 256 compute units")
    A = wl.random_bf16(M + K + 90, (M, K))
    B = wl.random_bf16(N + 91, (N, K), 0.05)
    mask = wl.random_mask(M + K + G + 92, (M, K // G), p)
    mask[:2] = 0  # rows with no active group
    C0 = wl.random_bf16(93, (M, N))
    say("gemm_k 320-wide tiles", M, N, K, G, p, "beta", beta)
    Ad, Bd, md = to_dev(A, torch), to_dev(B, torch), to_dev(mask, torch)
    outs = []
    for _ in range(2):
        out = to_dev(ref.from_bf16(C0).astype(np.float32), torch) if beta else \
            torch.full((M, N), float("nan"), device="cuda")
        W().gemm_k(Ad, Bd, G, md, out=out, beta=beta)
        outs.append(out)
    torch.cuda.synchronize()
    assert torch.equal(outs[0], outs[1]), "GEMM-K is not bitwise reproducible"
    rng = np.random.default_rng(M + N + K)
    rows = np.unique(np.concatenate([[0, 1, 2, 255, 256, 511, 1023, 1024, 1791, 1792, M - 2, M - 1],
                                     rng.integers(0, M, 16)]))
    got = f32_of(outs[0][torch.from_numpy(rows).cuda()])
    want = ref.gemm_k(A[rows], B, mask[rows], G) + (ref.from_bf16(C0[rows]) if beta else 0)
    check_gemm(got, want, f"gemm_k 320-wide {M}x{N}x{K} G{G} p{p} beta={beta}")
    if not beta:
        assert (got[:2] == 0).all()


@pytest.mark.parametrize("p", [0.0, 1.0])
def test_gemm_k_all_or_nothing(p):
    M, N, K, G = 150, 128, 512, 128
    A = wl.random_bf16(24, (M, K))
    B = wl.random_bf16(25, (N, K), 0.05)
    mask = np.full((M, K // G), int(p), np.uint8)
    out = W().gemm_k(to_dev(A, torch), to_dev(B, torch), G, to_dev(mask, torch))
    torch.cuda.synchronize()
    got = f32_of(out)
    if p == 0:
        assert (got == 0).all()
    else:
        check_gemm(got, ref.from_bf16(A) @ ref.from_bf16(B).T, "all-ones = dense")


@pytest.mark.parametrize("M", [1, 2, 3, 4])
@pytest.mark.parametrize("K,G", [(2048, 128), (14336, 128), (4096, 512)])
def test_gemv_k(M, K, G):
    N = 512
    A = wl.random_bf16(30 + M, (M, K))
    B = wl.random_bf16(31, (N, K), 0.05)
    mask = wl.random_mask(32 + M, (M, K // G), 0.5)
    say("gemv_k", M, K, G)
    out = W().gemm_k(to_dev(A, torch), to_dev(B, torch), G, to_dev(mask, torch))
    torch.cuda.synchronize()
    check_gemm(f32_of(out), ref.gemm_k(A, B, mask, G), "gemv_k")


def test_gemv_k_beta():
    M, N, K, G = 2, 256, 4096, 128
    A = wl.random_bf16(40, (M, K))
    B = wl.random_bf16(41, (N, K), 0.05)
    mask = wl.random_mask(42, (M, K // G), 0.5)
    C0 = np.random.default_rng(43).standard_normal((M, N)).astype(np.float32)
    say("gemv_k beta")
    out = torch.from_numpy(C0.copy()).to("cuda")
    W().gemm_k(to_dev(A, torch), to_dev(B, torch), G, to_dev(mask, torch), out=out, beta=1)
    torch.cuda.synchronize()
    check_gemm(f32_of(out), C0.astype(np.float64) + ref.gemm_k(A, B, mask, G), "gemv_k beta")


# ---------------------------------------------------------------------------
# Attention
# ---------------------------------------------------------------------------

def run_attn(Q, K, V, mask, causal=True, leftpad=None, out_dtype=torch.float32):
    B, Tq, Hq, d = Q.shape
    say("attn", Q.shape, K.shape, causal, leftpad, out_dtype)
    perm, counts = W().reorder(to_dev(mask, torch))
    lp = None if leftpad is None else to_dev(np.array(leftpad, np.int32), torch)
    out = W().attn(to_dev(Q, torch), to_dev(K, torch), to_dev(V, torch), perm=perm, counts=counts,
                   causal=causal, leftpad=lp, out_dtype=out_dtype)
    torch.cuda.synchronize()
    return out


ATTN_CASES = [  # B, Tq, Tk, Hq, Hk
    (1, 64, 64, 4, 1), (2, 300, 300, 8, 2), (1, 200, 333, 8, 2), (1, 257, 257, 10, 2),
    (1, 130, 130, 32, 8),
]


@pytest.mark.parametrize("B,Tq,Tk,Hq,Hk", ATTN_CASES)
@pytest.mark.parametrize("causal", [True, False])
def test_attention_prefill(B, Tq, Tk, Hq, Hk, causal):
    d = 128
    Q = wl.random_bf16(40 + Tq, (B, Tq, Hq, d), 1.0)
    K = wl.random_bf16(41 + Tk, (B, Tk, Hk, d), 1.0)
    V = wl.random_bf16(42 + Tk, (B, Tk, Hk, d), 1.0)
    mask = wl.random_mask(43 + Hq, (B, Tq, Hk), 0.5)
    out = run_attn(Q, K, V, mask, causal)
    want = ref.attention(Q, K, V, mask, causal=causal)
    check_attn(f32_of(out), want, "attn prefill")
    keep = np.repeat(mask != 0, Hq // Hk, axis=2)
    assert (out.cpu().numpy().view(np.uint32)[~keep] == 0).all()


def test_attention_leftpad_and_bf16():
    B, T, Hq, Hk, d = 2, 200, 8, 2, 128
    Q = wl.random_bf16(50, (B, T, Hq, d), 1.0)
    K = wl.random_bf16(51, (B, T, Hk, d), 1.0)
    V = wl.random_bf16(52, (B, T, Hk, d), 1.0)
    mask = wl.random_mask(53, (B, T, Hk), 0.6)
    lp = [0, 77]
    want = ref.attention(Q, K, V, mask, leftpad=lp)
    check_attn(f32_of(run_attn(Q, K, V, mask, leftpad=lp)), want, "leftpad")
    keep = np.repeat(mask != 0, Hq // Hk, axis=2)
    out = run_attn(Q, K, V, mask, leftpad=lp, out_dtype=torch.bfloat16)
    check_attn_bf16(bits_of(out)[keep], want[keep], "attn bf16")
    assert (bits_of(out)[~keep] == 0).all()


@pytest.mark.parametrize("Hq,Hk,Tk", [(32, 8, 1000), (40, 8, 4097), (8, 8, 256), (32, 4, 300), (32, 2, 130),
                                      (8, 2, 20000)])  # the last: more than 256 splits per head
@pytest.mark.parametrize("mode", ["mask", "counts"])
def test_attention_decode(Hq, Hk, Tk, mode):
    B, d = 2, 128
    Q = wl.random_bf16(60, (B, 1, Hq, d), 1.0)
    K = wl.random_bf16(61, (B, Tk, Hk, d), 1.0)
    V = wl.random_bf16(62, (B, Tk, Hk, d), 1.0)
    mask = wl.random_mask(63, (B, 1, Hk), 0.5)
    mask[0, 0, 0] = 1
    say("decode", Hq, Hk, Tk, mode)
    md = to_dev(mask, torch)
    if mode == "mask":
        out = W().attn(to_dev(Q, torch), to_dev(K, torch), to_dev(V, torch), mask=md,
                       out_dtype=torch.float32)
    else:
        perm, counts = W().reorder(md)
        out = W().attn(to_dev(Q, torch), to_dev(K, torch), to_dev(V, torch), perm=perm,
                       counts=counts, out_dtype=torch.float32)
    torch.cuda.synchronize()
    want = ref.attention(Q, K, V, mask)
    check_attn(f32_of(out), want, "decode")
    keep = np.repeat(mask != 0, Hq // Hk, axis=2)
    assert (out.cpu().numpy().view(np.uint32)[~keep] == 0).all()


@pytest.mark.parametrize("NG", [4, 8])   # two heads per routing group, then one
def test_attention_sub_gqa_groups_prefill(NG):
    """Routing groups finer than the KV heads (sub-GQA granularity): query
    head h is gated by group h // (Hq/NG) and reads KV head h // (Hq/Hk)."""
    B, T, Hq, Hk, d = 2, 300, 8, 2, 128
    Q = wl.random_bf16(130, (B, T, Hq, d))
    K = wl.random_bf16(131, (B, T, Hk, d), 0.5)
    V = wl.random_bf16(132, (B, T, Hk, d))
    mask = wl.random_mask(133 + NG, (B, T, NG), 0.5)
    lp = [0, 40]
    say("attention sub-GQA prefill", NG)
    md = to_dev(mask, torch)
    perm, counts = W().reorder(md)
    out = W().attn(to_dev(Q, torch), to_dev(K, torch), to_dev(V, torch), perm=perm, counts=counts,
                   leftpad=to_dev(np.array(lp, np.int32), torch), out_dtype=torch.float32, groups=NG)
    torch.cuda.synchronize()
    want = ref.attention(Q, K, V, mask, leftpad=lp)
    check_attn(f32_of(out), want, f"sub-GQA prefill NG={NG}")
    keep = np.repeat(mask != 0, Hq // NG, axis=2)
    assert (out.cpu().numpy().view(np.uint32)[~keep] == 0).all()


@pytest.mark.parametrize("NG", [16, 32])
def test_attention_sub_gqa_groups_decode(NG):
    B, Tk, Hq, Hk, d = 2, 1500, 32, 8, 128
    Q = wl.random_bf16(140, (B, 1, Hq, d), 1.0)
    K = wl.random_bf16(141, (B, Tk, Hk, d), 1.0)
    V = wl.random_bf16(142, (B, Tk, Hk, d), 1.0)
    mask = wl.random_mask(143 + NG, (B, 1, NG), 0.5)
    say("attention sub-GQA decode", NG)
    out = W().attn(to_dev(Q, torch), to_dev(K, torch), to_dev(V, torch), mask=to_dev(mask, torch),
                   out_dtype=torch.float32, groups=NG)
    torch.cuda.synchronize()
    want = ref.attention(Q, K, V, mask)
    check_attn(f32_of(out), want, f"sub-GQA decode NG={NG}")
    keep = np.repeat(mask != 0, Hq // NG, axis=2)
    assert (out.cpu().numpy().view(np.uint32)[~keep] == 0).all()


def test_attention_decode_workspace_reuse():
    """One workspace (uninitialised) through consecutive decoding calls of
    different sizes: nothing a call leaves there may leak into the next."""
    Hq, Hk, d = 32, 8, 128
    ws = torch.empty(W().attn_workspace_bytes(2, 1, 3000, Hq, Hk, d), dtype=torch.uint8, device="cuda")
    for i, (B, Tk) in enumerate([(2, 3000), (1, 700), (2, 257), (2, 3000)]):
        Q = wl.random_bf16(80 + i, (B, 1, Hq, d), 1.0)
        K = wl.random_bf16(90 + i, (B, Tk, Hk, d), 1.0)
        V = wl.random_bf16(100 + i, (B, Tk, Hk, d), 1.0)
        mask = wl.random_mask(110 + i, (B, 1, Hk), 0.5)
        say("decode workspace reuse", i, B, Tk)
        out = W().attn(to_dev(Q, torch), to_dev(K, torch), to_dev(V, torch), mask=to_dev(mask, torch),
                       out_dtype=torch.float32, workspace=ws)
        torch.cuda.synchronize()
        check_attn(f32_of(out), ref.attention(Q, K, V, mask), f"decode call {i}")


def test_attention_decode_no_valid_key():
    """Left padding that covers every key: active heads get O = 0."""
    B, Tk, Hq, Hk, d = 2, 600, 16, 4, 128
    Q = wl.random_bf16(120, (B, 1, Hq, d), 1.0)
    K = wl.random_bf16(121, (B, Tk, Hk, d), 1.0)
    V = wl.random_bf16(122, (B, Tk, Hk, d), 1.0)
    mask = np.ones((B, 1, Hk), np.uint8)
    lp = [Tk, 5]
    say("decode no valid key")
    out = W().attn(to_dev(Q, torch), to_dev(K, torch), to_dev(V, torch), mask=to_dev(mask, torch),
                   leftpad=to_dev(np.array(lp, np.int32), torch), out_dtype=torch.float32)
    torch.cuda.synchronize()
    want = ref.attention(Q, K, V, mask, leftpad=lp)
    assert (want[0] == 0).all()
    check_attn(f32_of(out), want, "decode no valid key")
    assert (f32_of(out)[0] == 0).all()


def test_attention_decode_leftpad():
    B, Tk, Hq, Hk, d = 2, 700, 16, 4, 128
    Q = wl.random_bf16(70, (B, 1, Hq, d), 1.0)
    K = wl.random_bf16(71, (B, Tk, Hk, d), 1.0)
    V = wl.random_bf16(72, (B, Tk, Hk, d), 1.0)
    mask = np.ones((B, 1, Hk), np.uint8)
    lp = [300, 0]
    say("decode leftpad")
    out = W().attn(to_dev(Q, torch), to_dev(K, torch), to_dev(V, torch), mask=to_dev(mask, torch),
                   leftpad=to_dev(np.array(lp, np.int32), torch), out_dtype=torch.float32)
    torch.cuda.synchronize()
    check_attn(f32_of(out), ref.attention(Q, K, V, mask, leftpad=lp), "decode leftpad")


# ---------------------------------------------------------------------------
# Group counts at the tile boundaries
# ---------------------------------------------------------------------------

BOUNDARY_COUNTS = [0, 1, 255, 256, 257, 512, 600]   # M = 600: none, one row, BM-1, BM, BM+1, 2 BM, all


def boundary_mask(seed, M=600):
    """[M][7] mask whose group g keeps exactly BOUNDARY_COUNTS[g] rows, at
    random positions (rows 0 and M-1 among them where the count allows)."""
    rng = np.random.default_rng(seed)
    mask = np.zeros((M, len(BOUNDARY_COUNTS)), np.uint8)
    for g, c in enumerate(BOUNDARY_COUNTS):
        rows = rng.permutation(M)[:c]
        mask[rows, g] = 1
    return mask


@pytest.mark.parametrize("scheduled", [False, True])
def test_boundary_counts_gemms(scheduled):
    """GEMM-MN (plain or scheduled with a workspace), fused SwiGLU and GEMM-K
    with group counts 0, 1, BM-1, BM, BM+1, 2 BM and M."""
    M, G, K = 600, 128, 1024
    NG = len(BOUNDARY_COUNTS)
    N = NG * G
    mask = boundary_mask(400)
    assert (mask.sum(axis=0) == BOUNDARY_COUNTS).all()
    A = wl.random_bf16(401, (M, K))
    B = wl.random_bf16(402, (N, K), 0.05)
    U = wl.random_bf16(403, (N, K), 0.05)
    say("boundary counts", "scheduled" if scheduled else "plain")
    perm, counts = W().reorder(to_dev(mask[None], torch))
    assert np.array_equal(counts.cpu().numpy()[0], BOUNDARY_COUNTS)
    Ad, Bd, Ud = to_dev(A, torch), to_dev(B, torch), to_dev(U, torch)
    ws = None
    if scheduled:
        ws = torch.full((W().gemm_mn_workspace_bytes(M, N, K, G, True) // 4,), float("nan"),
                        dtype=torch.float32, device="cuda")
    q = _run_mn_ws(Ad, Bd, None, perm[0], counts[0], G, torch.float32, ws, M, N)
    h = _run_mn_ws(Ad, Bd, Ud, perm[0], counts[0], G, torch.float32, ws, M, N)
    torch.cuda.synchronize()
    keep = ref.expand(mask, G)
    want_q = ref.gemm_mn(A, B, mask, G)
    check_gemm(f32_of(q), want_q, "boundary gemm_mn")
    assert (q.cpu().numpy().view(np.uint32)[~keep] == 0).all()
    want_h = ref.swiglu(want_q, ref.gemm_mn(A, U, mask, G))
    check_gemm(f32_of(h), want_h, "boundary swiglu")
    assert (h.cpu().numpy().view(np.uint32)[~keep] == 0).all()
    # GEMM-K over the same groups: A is [M][NG*G]
    Ak = wl.random_bf16(404, (M, N))
    Bk = wl.random_bf16(405, (512, N), 0.05)
    y = W().gemm_k(to_dev(Ak, torch), to_dev(Bk, torch), G, to_dev(mask, torch))
    torch.cuda.synchronize()
    check_gemm(f32_of(y), ref.gemm_k(Ak, Bk, mask, G), "boundary gemm_k")


def test_boundary_counts_attention():
    """Attention prefill with the same per-group counts (one routing group per
    KV head, 7 KV heads, 2 query heads each), causal and not."""
    B, T, Hk, d = 1, 600, len(BOUNDARY_COUNTS), 128
    Hq = 2 * Hk
    mask = boundary_mask(410)[None]
    Q = wl.random_bf16(411, (B, T, Hq, d), 1.0)
    K = wl.random_bf16(412, (B, T, Hk, d), 1.0)
    V = wl.random_bf16(413, (B, T, Hk, d), 1.0)
    keep = np.repeat(mask != 0, Hq // Hk, axis=2)
    for causal in (True, False):
        out = run_attn(Q, K, V, mask, causal)
        check_attn(f32_of(out), ref.attention(Q, K, V, mask, causal=causal), f"boundary attn causal={causal}")
        assert (out.cpu().numpy().view(np.uint32)[~keep] == 0).all()


def _random_mn_cases(n=16, seed=2024):
    """Seeded random shapes for the scheduled GEMM-MN path: group sizes 64 to
    640 (each tile width the launcher picks), K with and without a tail,
    M from 5 to 3000, activity from none to all, both epilogues and stores."""
    rng = np.random.default_rng(seed)
    cases = []
    while len(cases) < n:
        G = int(rng.choice([64, 128, 192, 256, 320, 640]))
        sw = bool(rng.integers(0, 2))
        NG = int(rng.integers(1, 6))
        K = int(rng.choice([1024, 1096, 1536, 2000, 4096]))
        M = int(rng.choice([5, 77, 256, 300, 1000, 3000]))
        if M * NG * G * K * (2 if sw else 1) > 4e9:    # keep the fp64 oracle quick
            continue
        cases.append((M, NG * G, K, G, sw, float(rng.choice([0.0, 0.1, 0.5, 0.9, 1.0])),
                      str(rng.choice(["f32", "bf16"]))))
    return cases


@pytest.mark.parametrize("M,N,K,G,swiglu,p,dt", _random_mn_cases())
def test_gemm_mn_scheduled_random_shapes(M, N, K, G, swiglu, p, dt):
    A = wl.random_bf16(M + 500, (M, K))
    B = wl.random_bf16(N + 501, (N, K), 0.05)
    U = wl.random_bf16(N + 502, (N, K), 0.05) if swiglu else None
    mask = wl.random_mask(M + N + K + 503, (M, N // G), p)
    need = W().gemm_mn_workspace_bytes(M, N, K, G, swiglu)
    say("gemm_mn scheduled random", M, N, K, G, swiglu, p, dt, "workspace", need)
    ws = torch.full((max(need, 16) // 4,), float("nan"), dtype=torch.float32, device="cuda")
    perm, counts = W().reorder(to_dev(mask[None], torch))
    out_dtype = torch.float32 if dt == "f32" else torch.bfloat16
    out = _run_mn_ws(to_dev(A, torch), to_dev(B, torch), to_dev(U, torch) if swiglu else None, perm[0], counts[0],
                     G, out_dtype, ws if need else None, M, N)
    torch.cuda.synchronize()
    want = ref.gemm_mn(A, B, mask, G)
    if swiglu:
        want = ref.swiglu(want, ref.gemm_mn(A, U, mask, G))
    keep = ref.expand(mask, G)
    if dt == "f32":
        check_gemm(f32_of(out), want, "scheduled random")
        assert (out.cpu().numpy().view(np.uint32)[~keep] == 0).all()
    else:
        if keep.any():
            check_bf16_store(bits_of(out)[keep], want[keep], "scheduled random bf16")
        assert (bits_of(out)[~keep] == 0).all()
