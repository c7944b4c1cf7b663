"""The Llama3.1-8B decode step captured as a HIP graph (the way the benchmark
replays it): every replay, with eager work and synchronisations between the
replays, reproduces the eager step bit for bit. The step's kernels have a fixed
summation order, so eager and replayed results must be identical."""
import numpy as np
import pytest

from masked_group_mask_amd import workloads as wl

from helpers import say

pytestmark = pytest.mark.gpu
torch = pytest.importorskip("torch")


@pytest.fixture(scope="module", autouse=True)
def gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import masked_group_mask_amd as mg
    mg.load()


def outputs(layer):
    return [layer.q, layer.o, layer.y_attn, layer.h, layer.y_ffn]


def snapshot(layer):
    return [t.detach().view(torch.uint8).cpu().numpy().copy() for t in outputs(layer)]


def test_decode_graph_replays_match_eager():
    from masked_group_mask_amd.layer import DecodeLayer
    s = wl.shape("llama8b_decode")
    say("decode graph replay")
    layer = DecodeLayer(s, wl.make_layer(s, seed=5), sets=1)
    for t in outputs(layer):
        t.zero_()
    layer.step(0)
    torch.cuda.synchronize()
    want = snapshot(layer)

    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        layer.step(0)
    torch.cuda.synchronize()
    names = ["q", "o", "y_attn", "h", "y_ffn"]
    for r in range(4):
        for t in outputs(layer):
            t.zero_()                                   # eager fill kernels between replays
        junk = torch.randn(512, 512, device="cuda") @ torch.randn(512, 512, device="cuda")
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        got = snapshot(layer)
        for name, a, b in zip(names, got, want):
            assert np.array_equal(a, b), f"replay {r}: {name} differs from the eager step"
        del junk
    # the eager step still agrees after the replays
    for t in outputs(layer):
        t.zero_()
    layer.step(0)
    torch.cuda.synchronize()
    for name, a, b in zip(names, snapshot(layer), want):
        assert np.array_equal(a, b), f"eager after replays: {name} differs"


def prefill_outputs(layer):
    return [layer.perm_a, layer.cnt_a, layer.perm_f, layer.cnt_f, layer.q, layer.o, layer.y_attn,
            layer.h, layer.y_ffn]


@pytest.mark.parametrize("ordered", [(), ("o_proj",)], ids=["token_order", "ordered_o_proj"])
def test_prefill_graph_replays_match_eager(ordered):
    """The masked prefill step (reorders, scheduled GEMM-MN with K-split last
    rounds and their fixups, attention, K-split GEMM-K) captured as a HIP
    graph: the workspace header the fixups read is rewritten by every replay,
    and every replay reproduces the eager step bit for bit, also with o_proj
    over pattern-sorted rows (the sort kernel and the ordered GEMM-K)."""
    from masked_group_mask_amd.layer import PrefillLayer
    s = wl.shape("qwen14b_prefill", T=1024, p_attn=0.5, p_ffn=0.5, G_ffn=128)
    say("prefill graph replay", s.T, s.D, s.Dff, ordered)
    layer = PrefillLayer(s, wl.make_layer(s, seed=6), with_dense=False, ordered_k=ordered)
    names = ["perm_a", "cnt_a", "perm_f", "cnt_f", "q", "o", "y_attn", "h", "y_ffn"]
    if ordered:
        names.append("order_a")

    def snap():
        outs = prefill_outputs(layer) + ([layer.order_a] if ordered else [])
        return [t.detach().view(torch.uint8).cpu().numpy().copy() for t in outs]

    for t in prefill_outputs(layer) + ([layer.order_a] if ordered else []):
        t.zero_()
    layer.step("masked")
    torch.cuda.synchronize()
    want = snap()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        layer.step("masked")
    torch.cuda.synchronize()
    for r in range(3):
        for t in prefill_outputs(layer) + ([layer.order_a] if ordered else []):
            t.zero_()
        layer.ws.fill_(255)                              # stale workspace between replays
        junk = torch.randn(512, 512, device="cuda") @ torch.randn(512, 512, device="cuda")
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        for name, a, b in zip(names, snap(), want):
            assert np.array_equal(a, b), f"replay {r}: {name} differs from the eager step"
        del junk
