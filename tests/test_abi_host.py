"""Host-side checks of the C ABI (no GPU needed, no kernel is launched).

The library must load, export every function declared in include/wide.h, and
reject invalid arguments on the host before touching the device.
"""
import ctypes
import os
import re

import pytest

from masked_group_mask_amd import _lib

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "wide.h")

INVALID, UNSUPPORTED, NO_DEVICE = -1, -2, -3


def declared_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(wide_[a-z_0-9]+)\s*\(", text)))


@pytest.fixture(scope="module")
def lib():
    if not os.path.exists(_lib.LIB_PATH):
        pytest.fail("libwide.so is not built; run masked_group_mask_amd.build.build()")
    return _lib.load()


def test_exports_every_declared_symbol(lib):
    names = declared_functions()
    assert {"wide_reorder", "wide_gemm_mn", "wide_gemm_k", "wide_attn"} <= set(names)
    for n in names:
        assert hasattr(lib, n), n
    assert set(names) == set(_lib.EXPORTED)


def test_status_strings(lib):
    assert _lib.status_string(0) == "ok"
    assert _lib.status_string(INVALID) == "invalid argument"
    assert _lib.status_string(UNSUPPORTED) == "unsupported shape or mode"
    assert _lib.status_string(12345) == "unknown status"
    assert lib.wide_abi_version() == 2


FAKE = 1 << 20      # a 16-byte aligned, non-null address that is never dereferenced


def P(i=0):
    return ctypes.c_void_p(FAKE * (i + 1))


def test_reorder_validation(lib):
    assert lib.wide_reorder(None, 1, 8, 2, P(1), P(2), None) == INVALID
    assert lib.wide_reorder(P(0), 0, 8, 2, P(1), P(2), None) == INVALID
    assert lib.wide_reorder(P(0), 1, 8, 0, P(1), P(2), None) == INVALID
    assert lib.wide_reorder(P(0), 1, 1 << 31, 2, P(1), P(2), None) == INVALID
    assert lib.wide_reorder(P(0), 1, 64, 2, P(0), P(2), None) == INVALID     # perm aliases mask


def mn(lib, **kw):
    a = dict(A=P(0), lda=64, B=P(1), ldb=64, C=P(2), ldc=256, dt=0, M=32, N=256, K=64, G=128,
             perm=P(3), counts=P(4), mask=None)
    a.update(kw)
    return lib.wide_gemm_mn(a["A"], a["lda"], a["B"], a["ldb"], a["C"], a["ldc"], a["dt"], a["M"],
                            a["N"], a["K"], a["G"], a["perm"], a["counts"], a["mask"], None)


def test_gemm_mn_validation(lib):
    assert mn(lib, A=None) == INVALID
    assert mn(lib, N=200) == INVALID                 # N % G
    assert mn(lib, K=60, lda=64, ldb=64) == INVALID  # K % 8
    assert mn(lib, lda=32) == INVALID                # lda < K
    assert mn(lib, ldc=100) == INVALID               # ldc < N
    assert mn(lib, dt=7) == INVALID
    assert mn(lib, A=ctypes.c_void_p(FAKE + 2)) == INVALID        # misaligned
    assert mn(lib, perm=None, mask=None) == INVALID
    assert mn(lib, perm=None, mask=P(5), M=5) == INVALID          # mask path needs M <= 4
    assert mn(lib, counts=None) == INVALID
    assert mn(lib, C=P(0)) == INVALID                             # C aliases A
    assert mn(lib, G=8, N=256) == UNSUPPORTED        # groups narrower than 16
    assert mn(lib, G=24, N=264, ldc=264) == UNSUPPORTED


def test_gemm_mn_swiglu_validation(lib):
    f = lib.wide_gemm_mn_swiglu
    assert f(P(0), 64, P(1), None, 64, P(2), 256, 0, 32, 256, 64, 128, P(3), P(4), None, None) == INVALID
    assert f(P(0), 64, P(1), P(2), 64, P(2), 256, 0, 32, 256, 64, 128, P(3), P(4), None, None) == INVALID


def mnw(lib, ws, wsb, M, N, K, G, swiglu=False, perm=True):
    """wide_gemm_mn_ws / wide_gemm_mn_swiglu_ws on fake pointers spaced far
    enough apart for these sizes."""
    base = 1 << 40
    A, B, U, C, pm, cn = (ctypes.c_void_p(base + i * (1 << 34)) for i in range(6))
    if not perm:
        pm, cn = None, None
    mask = ctypes.c_void_p(base + 6 * (1 << 34))
    if swiglu:
        return lib.wide_gemm_mn_swiglu_ws(A, K, B, U, K, C, N, 1, M, N, K, G, pm, cn, mask, ws, wsb, None)
    return lib.wide_gemm_mn_ws(A, K, B, K, C, N, 1, M, N, K, G, pm, cn, mask, ws, wsb, None)


def test_gemm_mn_workspace_plan(lib):
    """Workspace of the scheduled GEMM-MN path: a header plus one fp32 tile
    (320 rows for the 256-wide tiles, else 256) x the tile width per compute
    unit (256 CUs when no device answers), and none when K is too short for
    any split (fewer than 16 K-steps of 64)."""
    f = lib.wide_gemm_mn_workspace_bytes
    hdr = 4 * 4 * 1025
    cus = f(8192, 5120, 5120, 640, 0) - hdr
    assert cus % (256 * 320 * 4) == 0 and cus > 0
    cus //= 256 * 320 * 4
    assert f(8192, 5120, 5120, 640, 0) == hdr + cus * 256 * 320 * 4    # 320-wide tiles
    assert f(8192, 17408, 5120, 128, 1) == hdr + cus * 320 * 256 * 4   # fused SwiGLU tile
    assert f(8192, 4096, 4096, 512, 0) == hdr + cus * 320 * 256 * 4    # 256-wide tiles
    assert f(1000, 512, 1000, 64, 0) == hdr + cus * 256 * 64 * 4       # 64-wide tiles
    assert f(1000, 512, 960, 64, 0) == 0                                # 15 K-steps
    assert f(8192, 17408, 5120, 64, 1) == 0 and f(8192, 17408, 5120, 192, 1) == 0  # SwiGLU raster
    assert f(8192, 17408, 5120, 32, 1) > 0                              # narrower: scheduled
    assert f(0, 512, 4096, 64, 0) == 0 and f(10, 500, 4096, 64, 0) == 0  # bad sizes


def test_gemm_mn_workspace_validation(lib):
    M, N, K, G = 1000, 1280, 1024, 640
    need = lib.wide_gemm_mn_workspace_bytes(M, N, K, G, 0)
    ws = ctypes.c_void_p((1 << 40) + 8 * (1 << 34))
    assert mnw(lib, ws, need - 16, M, N, K, G) == INVALID                      # too small
    assert mnw(lib, ctypes.c_void_p(ws.value + 4), need, M, N, K, G) == INVALID  # misaligned
    alias = ctypes.c_void_p((1 << 40) + 3 * (1 << 34))                         # C's address
    assert mnw(lib, alias, need, M, N, K, G) == INVALID
    alias = ctypes.c_void_p((1 << 40) + 4 * (1 << 34))                         # perm's address
    assert mnw(lib, alias, need, M, N, K, G) == INVALID
    need_sw = lib.wide_gemm_mn_workspace_bytes(M, N, K, 128, 1)
    alias = ctypes.c_void_p((1 << 40) + 2 * (1 << 34))                         # up weights
    assert mnw(lib, alias, need_sw, M, N, K, 128, swiglu=True) == INVALID
    # without perm (matrix-vector path, M <= 4) the workspace is ignored
    assert mnw(lib, ctypes.c_void_p(ws.value + 4), 0, 4, N, K, G, perm=False) != INVALID


def gk(lib, **kw):
    a = dict(A=P(0), lda=256, B=P(1), ldb=256, C=P(2), ldc=128, beta=0, M=32, N=128, K=256,
             G=128, order=None, mask=P(3))
    a.update(kw)
    return lib.wide_gemm_k(a["A"], a["lda"], a["B"], a["ldb"], a["C"], a["ldc"], a["beta"],
                           a["M"], a["N"], a["K"], a["G"], a["order"], a["mask"], None)


def gkw(lib, ws, wsb, M, N, K, G=128, order=None):
    """wide_gemm_k_ws on fake pointers spaced far enough apart for these sizes."""
    base = 1 << 40
    A, B, C, mask = (ctypes.c_void_p(base + i * (1 << 34)) for i in range(4))
    return lib.wide_gemm_k_ws(A, K, B, K, C, N, 0, M, N, K, G, order, mask, ws, wsb, None)


def test_gemm_k_workspace_plan(lib):
    """Workspace sizes of the K-split plan (the answers hold for any device
    with at least 8 compute units and none above 512 in the last case)."""
    f = lib.wide_gemm_k_workspace_bytes
    tile = 256 * 256 * 4
    assert f(256, 256, 4096) == 7 * tile    # one tile: 8 slices of 8 K-steps
    assert f(256, 256, 512) == 0            # 8 K-steps: too short to split
    assert f(4, 256, 4096) == 0             # matrix-vector path
    assert f(256, 384, 4096) == 0           # N not a multiple of 256: no split
    assert f(8192, 4096, 4096) == 0         # 512 tiles: whole rounds (256 CUs) or a last round over half full
    assert f(0, 256, 4096) == 0 and f(256, -1, 4096) == 0


def test_gemm_k_workspace_validation(lib):
    need = lib.wide_gemm_k_workspace_bytes(256, 256, 4096)
    ws = ctypes.c_void_p((1 << 40) + 8 * (1 << 34))
    assert gkw(lib, ws, need - 16, 256, 256, 4096) == INVALID                 # too small
    assert gkw(lib, ctypes.c_void_p(ws.value + 4), need, 256, 256, 4096) == INVALID  # misaligned
    alias = ctypes.c_void_p((1 << 40) + 2 * (1 << 34))                        # C's address
    assert gkw(lib, alias, need, 256, 256, 4096) == INVALID
    # the workspace may not overlap the order either
    order = ctypes.c_void_p((1 << 40) + 9 * (1 << 34))
    assert gkw(lib, order, need, 256, 256, 4096, order=order) == INVALID


def test_gemm_k_validation(lib):
    assert gk(lib, mask=None) == INVALID
    assert gk(lib, K=200, lda=256, ldb=256) == INVALID     # K % G
    assert gk(lib, beta=2) == INVALID
    assert gk(lib, ldc=130) == INVALID                      # ldc % 4
    assert gk(lib, C=P(1)) == INVALID                       # C aliases B
    assert gk(lib, G=8, K=256) == UNSUPPORTED
    far = {k: ctypes.c_void_p((i + 1) << 40) for i, k in enumerate(("A", "B", "C", "mask"))}
    K513 = 16 * 513                                         # more than 512 groups
    assert gk(lib, G=16, K=K513, lda=K513, ldb=K513, **far) == UNSUPPORTED
    assert gk(lib, N=64, ldc=64) == UNSUPPORTED
    assert gk(lib, order=P(2)) == INVALID                   # C overlaps the order


def gkg(lib, **kw):
    """wide_gemm_k_grouped on fake pointers spaced far apart."""
    far = {k: ctypes.c_void_p((i + 1) << 40) for i, k in enumerate(("A", "B", "C", "perm", "counts"))}
    a = dict(lda=256, ldb=256, ldc=256, beta=0, M=32, N=256, K=256, G=64, **far)
    a.update(kw)
    return lib.wide_gemm_k_grouped(a["A"], a["lda"], a["B"], a["ldb"], a["C"], a["ldc"], a["beta"],
                                   a["M"], a["N"], a["K"], a["G"], a["perm"], a["counts"], None)


def test_gemm_k_grouped_validation(lib):
    assert gkg(lib, perm=None) == INVALID
    assert gkg(lib, counts=None) == INVALID
    assert gkg(lib, K=200) == INVALID                       # K % G
    assert gkg(lib, beta=2) == INVALID
    assert gkg(lib, ldc=258) == INVALID                     # ldc % 4
    assert gkg(lib, lda=128) == INVALID                     # lda < K
    assert gkg(lib, C=ctypes.c_void_p((4 << 40) + 64)) == INVALID   # C overlaps perm
    assert gkg(lib, C=ctypes.c_void_p(((5 << 40) - 64))) == INVALID  # C overlaps counts
    assert gkg(lib, G=32, K=256) == UNSUPPORTED             # groups narrower than a 64-deep stage
    assert gkg(lib, N=64, ldc=64) == UNSUPPORTED            # N % 128
    assert gkg(lib, M=1 << 20, lda=2048, K=2048, ldb=2048) == UNSUPPORTED  # 32-bit offsets into A
    torch = pytest.importorskip("torch")
    if not torch.cuda.is_available():
        assert gkg(lib) == NO_DEVICE


def test_order_by_pattern_validation(lib):
    f = lib.wide_order_by_pattern
    assert f(None, 64, 8, P(1), None) == INVALID
    assert f(P(0), 64, 8, None, None) == INVALID
    assert f(P(0), 0, 8, P(1), None) == INVALID
    assert f(P(0), 64, 0, P(1), None) == INVALID
    assert f(P(0), 1 << 31, 8, P(1), None) == INVALID
    assert f(P(0), 64, 8, P(0), None) == INVALID            # order overlaps the mask


def at(lib, **kw):
    a = dict(Q=P(0), K=P(1), V=P(2), O=P(3), dt=0, B=1, Tq=16, Tk=16, Hq=8, Hk=2, d=128, causal=1,
             scale=0.0, leftpad=None, perm=P(4), counts=P(5), mask=None, ws=None, wsb=0)
    a.update(kw)
    return lib.wide_attn(a["Q"], a["K"], a["V"], a["O"], a["dt"], a["B"], a["Tq"], a["Tk"], a["Hq"],
                         a["Hk"], a["d"], a["causal"], a["scale"], a["leftpad"], a["perm"],
                         a["counts"], a["mask"], a["ws"], a["wsb"], None)


def test_attn_validation(lib):
    assert at(lib, Q=None) == INVALID
    assert at(lib, Hq=6, Hk=4) == INVALID          # Hq % Hk
    assert at(lib, Tk=8) == INVALID                 # Tk < Tq
    assert at(lib, perm=None) == INVALID            # prefill needs the reorder
    assert at(lib, scale=-1.0) == INVALID
    assert at(lib, causal=3) == INVALID
    assert at(lib, d=64) == UNSUPPORTED
    # decode needs a workspace of the advertised size
    need = lib.wide_attn_workspace_bytes(1, 1, 4096, 8, 2, 128)
    assert need > 0 and lib.wide_attn_workspace_bytes(1, 16, 16, 8, 2, 128) == 0
    assert at(lib, Tq=1, Tk=4096, perm=None, counts=None, mask=P(6)) == INVALID
    assert at(lib, Tq=1, Tk=4096, perm=None, counts=None, mask=P(6), ws=P(7), wsb=need - 4) == INVALID


def test_attn_noalloc_validation(lib):
    def na(**kw):
        a = dict(Q=P(0), K=P(1), V=P(2), O=P(3), dt=0, B=1, Tq=1, Tk=16, Hq=8, Hk=2, d=128, causal=1,
                 scale=0.0, leftpad=None, perm=None, counts=None, mask=P(5))
        a.update(kw)
        return lib.wide_attn_noalloc(a["Q"], a["K"], a["V"], a["O"], a["dt"], a["B"], a["Tq"], a["Tk"],
                                     a["Hq"], a["Hk"], a["d"], a["causal"], a["scale"], a["leftpad"],
                                     a["perm"], a["counts"], a["mask"], None)
    TOO_LARGE = -5
    assert na(Q=None) == INVALID
    assert na(Hq=6, Hk=4) == INVALID
    # 16 x 64 heads x 1024 splits of 132 floats: 69 MB > 32 MiB of built-in scratch
    big = dict(B=16, Tk=65536, Hq=64, Hk=8)
    assert na(**big) == TOO_LARGE
    assert _lib.status_string(TOO_LARGE).startswith("needs more scratch")
    torch = pytest.importorskip("torch")
    if not torch.cuda.is_available():
        assert na() == NO_DEVICE


def test_attn_grouped_validation(lib):
    def call(groups, Hq=8, Hk=2):
        return lib.wide_attn_grouped(P(0), P(1), P(2), P(3), 1, 1, 16, 16, Hq, Hk, groups, 128, 1,
                                     ctypes.c_float(0.0), None, P(4), P(5), None, None, 0, None)
    assert call(3) == INVALID       # not a multiple of Hk
    assert call(1) == INVALID       # fewer groups than KV heads
    assert call(12, Hq=8) == INVALID  # does not divide Hq


def test_router_validation(lib):
    def call(X=P(0), ldx=64, W1=P(1), W2=P(2), B=1, T=32, D=64, r=32, NG=8, mask=P(3), logits=None,
             perm=None, counts=None):
        return lib.wide_router(X, ldx, W1, W2, B, T, D, r, NG, mask, logits, perm, counts, None)
    assert call(X=None) == INVALID
    assert call(mask=None) == INVALID
    assert call(perm=P(4)) == INVALID                 # perm without counts
    assert call(counts=P(5)) == INVALID               # counts without perm
    assert call(D=60, ldx=64) == INVALID              # D % 8
    assert call(ldx=32) == INVALID                    # ldx < D
    assert call(r=8) == UNSUPPORTED
    assert call(r=24) == UNSUPPORTED
    assert call(NG=1024, r=32) == UNSUPPORTED         # W2 does not fit the staging LDS
    assert call(X=ctypes.c_void_p(FAKE + 8)) == INVALID   # misaligned
    assert call(mask=ctypes.c_void_p(FAKE * 1 + 16)) == INVALID   # mask overlaps X
    assert call(T=1 << 26, ldx=64) == UNSUPPORTED     # 32-bit offsets into X


def test_valid_call_without_device_reports_no_device(lib):
    torch = pytest.importorskip("torch")
    if torch.cuda.is_available():
        pytest.skip("a GPU is present; this checks the host-only path")
    assert mn(lib) == NO_DEVICE
