"""Every entry point enqueues on the caller's stream (the binding passes torch's
current stream): work launched on a side stream must follow the producers on
that stream and give the same bits as on the default stream."""
import numpy as np
import pytest

from masked_group_mask_amd import workloads as wl

from helpers import say, to_dev

pytestmark = pytest.mark.gpu
torch = pytest.importorskip("torch")


@pytest.fixture(scope="module", autouse=True)
def gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import masked_group_mask_amd as mg
    mg.load()


def _spin(ms):
    """Keep the current stream busy for about `ms` (torch's bounded spin kernel)."""
    sleep = getattr(torch.cuda, "_sleep", None)
    if sleep is None:
        pytest.skip("torch.cuda._sleep is not available")
    sleep(int(ms * 1e6))  # cycles; ~1 ms at the shader clock or less


def test_ops_follow_their_producer_on_a_side_stream():
    """On a side stream: a spin, then a torch op that writes the GEMM inputs,
    then the reorder, GEMM-MN and GEMM-K. Had any entry point launched on
    another stream it would read the inputs before the torch op wrote them."""
    import masked_group_mask_amd as mg
    M, N, K, G = 1024, 512, 1024, 128
    A = to_dev(wl.random_bf16(1, (M, K)), torch)
    B = to_dev(wl.random_bf16(2, (N, K), 0.05), torch)
    mask = to_dev(wl.random_mask(3, (1, M, N // G), 0.5), torch)
    kmask = to_dev(wl.random_mask(4, (M, K // G), 0.5), torch)
    # reference on the default stream, from the final inputs
    A2_ref = A * 2
    perm_r, cnt_r = mg.reorder(mask)
    c_ref = mg.gemm_mn(A2_ref, B, G, perm=perm_r[0], counts=cnt_r[0])
    k_ref = mg.gemm_k(A2_ref, B, G, kmask)
    torch.cuda.synchronize()

    say("side stream: spin, producer, reorder, gemm_mn, gemm_k")
    side = torch.cuda.Stream()
    A2 = torch.zeros_like(A)
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        _spin(2.0)
        torch.mul(A, 2, out=A2)
        perm, cnt = mg.reorder(mask)
        c = mg.gemm_mn(A2, B, G, perm=perm[0], counts=cnt[0])
        k = mg.gemm_k(A2, B, G, kmask)
    side.synchronize()
    assert torch.equal(perm, perm_r) and torch.equal(cnt, cnt_r)
    assert torch.equal(c, c_ref), "GEMM-MN on the side stream read its input early or differs"
    assert torch.equal(k, k_ref), "GEMM-K on the side stream read its input early or differs"


def test_prefill_and_decode_steps_on_a_side_stream():
    """A whole masked prefill step and a decode step on a side stream give the
    same bits as on the default stream."""
    from masked_group_mask_amd.layer import DecodeLayer, PrefillLayer
    s = wl.shape("qwen14b_prefill", T=1024, p_attn=0.5, p_ffn=0.5, G_ffn=128)
    layer = PrefillLayer(s, wl.make_layer(s, seed=12), with_dense=False)
    names = ("perm_a", "cnt_a", "perm_f", "cnt_f", "q", "o", "y_attn", "h", "y_ffn")

    def snap(obj, keys):
        return [getattr(obj, k).detach().view(torch.uint8).cpu().numpy().copy() for k in keys]

    for t in (layer.q, layer.o, layer.h):
        t.zero_()
    layer.step("masked")
    torch.cuda.synchronize()
    want = snap(layer, names)
    for t in (layer.q, layer.o, layer.h, layer.y_attn, layer.y_ffn):
        t.zero_()
    torch.cuda.synchronize()
    say("prefill step on a side stream", s.T)
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        _spin(1.0)
        layer.step("masked")
    side.synchronize()
    for name, a, b in zip(names, snap(layer, names), want):
        assert np.array_equal(a, b), f"prefill on a side stream: {name} differs"

    d = wl.shape("llama8b_decode", B=1, Tk=2048)
    dec = DecodeLayer(d, wl.make_layer(d, seed=13), sets=1)
    outs = [k for k in ("q", "o", "y_attn", "h", "y_ffn") if hasattr(dec, k)]
    dec.step(0)
    torch.cuda.synchronize()
    want = snap(dec, outs)
    say("decode step on a side stream")
    with torch.cuda.stream(side):
        _spin(1.0)
        dec.step(0)
    side.synchronize()
    for name, a, b in zip(outs, snap(dec, outs), want):
        assert np.array_equal(a, b), f"decode on a side stream: {name} differs"


def test_two_streams_with_their_own_workspaces():
    """Scheduled GEMM-MN (device-side tile schedule in the workspace) and K-split
    GEMM-K on two streams at once, each with its own workspace: both results
    equal the same calls made one after the other."""
    import masked_group_mask_amd as mg
    M, N, K, G = 2048, 1280, 1280, 640
    cases = []
    for seed in (21, 22):
        A = to_dev(wl.random_bf16(seed, (M, K)), torch)
        B = to_dev(wl.random_bf16(seed + 100, (N, K), 0.05), torch)
        mask = to_dev(wl.random_mask(seed + 200, (1, M, N // G), 0.5), torch)
        kmask = to_dev(wl.random_mask(seed + 300, (M, K // G), 0.5), torch)
        perm, cnt = mg.reorder(mask)
        ws_mn = torch.empty(max(mg.gemm_mn_workspace_bytes(M, N, K, G, False), 16), dtype=torch.uint8, device="cuda")
        ws_k = torch.empty(max(mg.gemm_k_workspace_bytes(M, N, K), 16), dtype=torch.uint8, device="cuda")
        c_ref = mg.gemm_mn(A, B, G, perm=perm[0], counts=cnt[0], workspace=ws_mn)
        k_ref = mg.gemm_k(A, B, G, kmask, workspace=ws_k)
        cases.append((A, B, perm, cnt, kmask, ws_mn, ws_k, c_ref, k_ref))
    torch.cuda.synchronize()
    say("two streams, own workspaces")
    streams = [torch.cuda.Stream(), torch.cuda.Stream()]
    outs = []
    for st in streams:
        st.wait_stream(torch.cuda.current_stream())
    for st, (A, B, perm, cnt, kmask, ws_mn, ws_k, _, _) in zip(streams, cases):
        with torch.cuda.stream(st):
            ws_mn.fill_(255)  # stale workspace contents must not matter
            ws_k.fill_(255)
            outs.append((mg.gemm_mn(A, B, G, perm=perm[0], counts=cnt[0], workspace=ws_mn),
                         mg.gemm_k(A, B, G, kmask, workspace=ws_k)))
    for st in streams:
        st.synchronize()
    for (c, k), case in zip(outs, cases):
        assert torch.equal(c, case[7]), "scheduled GEMM-MN differs when run beside another stream"
        assert torch.equal(k, case[8]), "GEMM-K differs when run beside another stream"
