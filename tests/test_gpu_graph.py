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
