"""The entry point that allocates nothing: wide_attn_noalloc against
wide_attn (same kernels, caller workspace) and against the oracle, called
through the C ABI twice in a row, the second call with a smaller problem (the
built-in scratch keeps the first call's partials, which must not leak)."""
import numpy as np
import pytest

from oracle import wide_ref as ref
from masked_group_mask_amd import workloads as wl

from helpers import check_attn, f32_of, say, to_dev

pytestmark = pytest.mark.gpu
torch = pytest.importorskip("torch")


@pytest.fixture(scope="module", autouse=True)
def gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import masked_group_mask_amd as mg
    mg.load()


def _decode_case(seed, B, Tk, Hq, Hk):
    d = 128
    Q = wl.random_bf16(seed, (B, 1, Hq, d))
    K = wl.random_bf16(seed + 1, (B, Tk, Hk, d))
    V = wl.random_bf16(seed + 2, (B, Tk, Hk, d))
    mask = wl.random_mask(seed + 3, (B, 1, Hk), 0.5)
    mask[0, 0, 0] = 1
    return Q, K, V, mask


@pytest.mark.parametrize("first,second", [((4, 16384, 32, 8), (2, 3000, 32, 8)),
                                          ((2, 8192, 40, 8), (1, 777, 8, 2))])
def test_attn_noalloc_matches_workspace_call(first, second):
    import masked_group_mask_amd as mg
    for i, (B, Tk, Hq, Hk) in enumerate((first, second)):
        say("attn noalloc call", i, "B", B, "Tk", Tk, "Hq", Hq, "Hk", Hk)
        Q, K, V, mask = _decode_case(100 + 10 * i + B, B, Tk, Hq, Hk)
        Qd, Kd, Vd, md = (to_dev(x, torch) for x in (Q, K, V, mask))
        got = torch.zeros((B, 1, Hq, 128), dtype=torch.float32, device="cuda")
        mg.attn(Qd, Kd, Vd, mask=md, out=got, noalloc=True)
        want_gpu = mg.attn(Qd, Kd, Vd, mask=md, out_dtype=torch.float32)
        torch.cuda.synchronize()
        assert torch.equal(got, want_gpu), "noalloc differs from the workspace call"
        check_attn(f32_of(got), ref.attention(Q, K, V, mask), f"attn noalloc {B}x{Tk}")


def test_attn_noalloc_prefill_needs_no_scratch():
    import masked_group_mask_amd as mg
    B, T, Hq, Hk, d = 1, 300, 8, 2, 128
    Q = wl.random_bf16(200, (B, T, Hq, d))
    K = wl.random_bf16(201, (B, T, Hk, d))
    V = wl.random_bf16(202, (B, T, Hk, d))
    mask = wl.random_mask(203, (B, T, Hk), 0.5)
    md = to_dev(mask, torch)
    perm, counts = mg.reorder(md)
    say("attn noalloc prefill")
    got = torch.zeros((B, T, Hq, d), dtype=torch.float32, device="cuda")
    mg.attn(to_dev(Q, torch), to_dev(K, torch), to_dev(V, torch), perm=perm, counts=counts, out=got, noalloc=True)
    torch.cuda.synchronize()
    check_attn(f32_of(got), ref.attention(Q, K, V, mask), "attn noalloc prefill")


def test_attn_noalloc_refuses_sizes_beyond_the_scratch():
    import masked_group_mask_amd as mg
    B, Tk, Hq, Hk, d = 16, 65536, 64, 8, 128     # 16 * 64 * 1024 splits > 63550
    Q = torch.zeros((B, 1, Hq, d), dtype=torch.bfloat16, device="cuda")
    K = torch.zeros((B, Tk, Hk, d), dtype=torch.bfloat16, device="cuda")
    mask = torch.ones((B, 1, Hk), dtype=torch.uint8, device="cuda")
    out = torch.zeros((B, 1, Hq, d), dtype=torch.bfloat16, device="cuda")
    with pytest.raises(mg.WideError, match="scratch"):
        mg.attn(Q, K, K, mask=mask, out=out, noalloc=True)
