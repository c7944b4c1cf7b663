"""GPU parity at the full workload sizes, in the launch sequence the bench times.

Each workload runs one masked step through masked_group_mask_amd.layer (the
same driver bench.py times); the oracle then recomputes sampled token rows of
every routed operator from the same inputs, with each operator fed the bf16
intermediate the GPU actually produced. The reorder is checked in full.
"""
import numpy as np
import pytest

from oracle import wide_ref as ref
from masked_group_mask_amd import workloads as wl

from helpers import bits_of, check_attn_bf16, check_bf16_store, check_gemm, say, to_dev

pytestmark = pytest.mark.gpu
torch = pytest.importorskip("torch")

N_SAMPLE = 24


@pytest.fixture(scope="module", autouse=True)
def gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import masked_group_mask_amd as mg
    mg.load()


def sample_rows(M, seed):
    rng = np.random.default_rng(seed)
    rows = set(rng.choice(M, size=min(N_SAMPLE, M), replace=False).tolist()) | {0, M - 1}
    return np.array(sorted(rows))


def check_reorder(mask, perm, counts):
    """Full check: counts are the mask sums and perm is the stable partition
    (numpy's stable argsort of the inactive flags, column by column)."""
    m = mask.astype(bool)
    assert np.array_equal(counts, m.sum(axis=0).astype(np.int32))
    want = np.argsort(~m.T, axis=1, kind="stable")
    assert np.array_equal(perm, want)


def active_only(bits, keep):
    """The GPU's bf16 intermediate with the entries it never writes (inactive
    groups: the buffers are not cleared) set to +0, which is all the next
    operator may depend on."""
    return np.where(keep, bits, np.uint16(0))


def check_ffn(s, host, rows, h_gpu_bits, y_gpu):
    m2 = host["mask_ffn"].reshape(s.M, s.NG_ffn)
    X = host["x"][rows]
    mr = m2[rows]
    gate = ref.gemm_mn(X, host["w_gate"], mr, s.G_ffn)
    up = ref.gemm_mn(X, host["w_up"], mr, s.G_ffn)
    want_h = ref.swiglu(gate, up)
    keep = ref.expand(mr, s.G_ffn)
    check_bf16_store(h_gpu_bits[keep], want_h[keep], f"{s.name} gate/up+SwiGLU")
    want_y = ref.gemm_k(active_only(h_gpu_bits, keep), host["w_down"], mr, s.G_ffn)
    check_gemm(y_gpu, want_y, f"{s.name} down_proj")


# (workload, shape overrides, GEMM-K ops over pattern-sorted rows)
PREFILL = [
    ("llama8b_prefill", {}, ()),
    ("llama8b_prefill", {}, ("o_proj",)),
    ("qwen14b_prefill", {"p_attn": 0.5, "p_ffn": 0.5, "G_ffn": 128}, ()),
    ("qwen14b_prefill", {"p_attn": 0.5, "p_ffn": 0.5, "G_ffn": 64}, ()),
    ("qwen14b_prefill", {"p_attn": 0.5, "p_ffn": 0.5, "G_ffn": 256}, ()),
    ("qwen14b_prefill", {"p_attn": 0.75, "p_ffn": 0.75, "G_ffn": 64}, ()),
    ("qwen14b_prefill", {"p_attn": 0.75, "p_ffn": 0.75, "G_ffn": 128}, ()),
    ("qwen14b_prefill", {"p_attn": 0.75, "p_ffn": 0.75, "G_ffn": 256}, ()),
]


@pytest.mark.parametrize("name,over,ordered", PREFILL, ids=lambda v: str(v))
def test_prefill_layer_full_size(name, over, ordered):
    from masked_group_mask_amd.layer import PrefillLayer
    s = wl.shape(name, **over)
    say("full-size prefill", s.name, over, ordered)
    host = wl.make_layer(s, seed=0)
    layer = PrefillLayer(s, host, with_dense=False, ordered_k=ordered)
    layer.step("masked")
    torch.cuda.synchronize()

    check_reorder(host["mask_attn"][0], layer.perm_a.cpu().numpy()[0], layer.cnt_a.cpu().numpy()[0])
    check_reorder(host["mask_ffn"][0], layer.perm_f.cpu().numpy()[0], layer.cnt_f.cpu().numpy()[0])
    if ordered:
        # the row order the sorted GEMM-K ran over is a permutation of the tokens
        assert np.array_equal(np.sort(layer.order_a.cpu().numpy()), np.arange(s.M))

    rows = sample_rows(s.M, 11)
    ma2 = host["mask_attn"].reshape(s.M, s.Hk)
    mr = ma2[rows]
    # q_proj
    q_bits = bits_of(layer.q)
    want_q = ref.gemm_mn(host["x"][rows], host["w_q"], mr, s.G_attn)
    keep = ref.expand(mr, s.G_attn)
    check_bf16_store(q_bits[rows][keep], want_q[keep], f"{s.name} q_proj")
    # attention, on the GPU's own Q
    q_in = active_only(q_bits, ref.expand(ma2, s.G_attn))
    want_o = ref.attention(q_in.reshape(s.B, s.T, s.Hq, s.d), host["k"], host["v"],
                           host["mask_attn"], queries=[(0, int(t)) for t in rows])
    o_bits = bits_of(layer.o).reshape(s.M, s.Hq, s.d)[rows]
    keep_h = np.repeat(mr != 0, s.Hq // s.Hk, axis=1)
    check_attn_bf16(o_bits[keep_h], want_o[keep_h], f"{s.name} attention")
    # o_proj on the GPU's own O
    o_in = active_only(o_bits, keep_h[..., None]).reshape(len(rows), -1)
    want_y = ref.gemm_k(o_in, host["w_o"], mr, s.G_attn)
    check_gemm(layer.y_attn.cpu().numpy()[rows].astype(np.float64), want_y, f"{s.name} o_proj")
    # FFN
    check_ffn(s, host, rows, bits_of(layer.h)[rows], layer.y_ffn.cpu().numpy()[rows].astype(np.float64))


def test_prefill_layer_batched_leftpad():
    """Two left-padded sequences of 4096 tokens through the layer driver
    (Qwen3-14B shape, 50% of the groups off): per-sequence attention reorder,
    flattened GEMM reorder, keys before each sequence's padding excluded
    (Appendix B, Algorithm 4 with leftpad)."""
    from masked_group_mask_amd.layer import PrefillLayer
    s = wl.shape("qwen14b_prefill", B=2, T=4096)
    leftpad = [0, 777]
    say("batched left-padded prefill", s.B, s.T, leftpad)
    host = wl.make_layer(s, seed=3)
    layer = PrefillLayer(s, host, with_dense=False, leftpad=leftpad)
    layer.step("masked")
    torch.cuda.synchronize()
    pa, ca = layer.perm_a.cpu().numpy(), layer.cnt_a.cpu().numpy()
    for b in range(s.B):
        check_reorder(host["mask_attn"][b], pa[b], ca[b])
    check_reorder(host["mask_attn"].reshape(s.M, s.Hk), layer.perm_q.cpu().numpy()[0], layer.cnt_q.cpu().numpy()[0])
    rows = np.array(sorted(set(sample_rows(s.M, 21).tolist()) | {s.T, s.T + 5, s.T + 776, s.T + 777}))
    ma2 = host["mask_attn"].reshape(s.M, s.Hk)
    mr = ma2[rows]
    q_bits = bits_of(layer.q)
    want_q = ref.gemm_mn(host["x"][rows], host["w_q"], mr, s.G_attn)
    keep = ref.expand(mr, s.G_attn)
    check_bf16_store(q_bits[rows][keep], want_q[keep], "batched q_proj")
    q_in = active_only(q_bits, ref.expand(ma2, s.G_attn))
    queries = [(int(r) // s.T, int(r) % s.T) for r in rows]
    want_o = ref.attention(q_in.reshape(s.B, s.T, s.Hq, s.d), host["k"], host["v"], host["mask_attn"],
                           leftpad=leftpad, queries=queries)
    o_bits = bits_of(layer.o).reshape(s.M, s.Hq, s.d)[rows]
    keep_h = np.repeat(mr != 0, s.Hq // s.Hk, axis=1)
    check_attn_bf16(o_bits[keep_h], want_o[keep_h], "batched left-padded attention")
    # padded queries of sequence 1 see no key: exact zeros where active
    pad = np.array([r // s.T == 1 and r % s.T < leftpad[1] for r in rows])
    assert (o_bits[pad][keep_h[pad]] == 0).all()
    o_in = active_only(o_bits, keep_h[..., None]).reshape(len(rows), -1)
    check_gemm(layer.y_attn.cpu().numpy()[rows].astype(np.float64), ref.gemm_k(o_in, host["w_o"], mr, s.G_attn),
               "batched o_proj")
    check_ffn(s, host, rows, bits_of(layer.h)[rows], layer.y_ffn.cpu().numpy()[rows].astype(np.float64))


def test_llama3b_ffn_full_size():
    """Llama3.2-3B-shaped FFN, T=4096, per-group Beta(2,2) activation rates,
    through the FFN-only layer driver (the launch sequence bench.py times for
    this workload: reorder, scheduled gate/up + SwiGLU, down_proj)."""
    from masked_group_mask_amd.layer import FFN_OPS, PrefillLayer
    s = wl.shape("llama3b_ffn")
    say("full-size ffn", s.name)
    host = wl.make_layer(s, seed=0)
    assert "mask_attn" not in host
    layer = PrefillLayer(s, host, with_dense=False)
    assert layer.ops == FFN_OPS
    layer.step("masked")
    torch.cuda.synchronize()
    check_reorder(host["mask_ffn"][0], layer.perm_f.cpu().numpy()[0], layer.cnt_f.cpu().numpy()[0])
    rows = sample_rows(s.M, 12)
    check_ffn(s, host, rows, bits_of(layer.h)[rows], layer.y_ffn.cpu().numpy()[rows].astype(np.float64))
    with pytest.raises(ValueError):
        layer.run("attention")


def test_tiny_ffn_every_entry():
    """T=64, hidden 256, ffn 1024, G=128: every output entry against the oracle."""
    import masked_group_mask_amd as mg
    s = wl.shape("tiny_ffn")
    host = wl.make_layer(s, seed=0, parts=("ffn",))
    say("tiny ffn")
    md = to_dev(host["mask_ffn"], torch)
    perm, counts = mg.reorder(md)
    h = mg.gemm_mn_swiglu(to_dev(host["x"], torch), to_dev(host["w_gate"], torch),
                          to_dev(host["w_up"], torch), s.G_ffn, perm=perm[0], counts=counts[0])
    y = mg.gemm_k(h, to_dev(host["w_down"], torch), s.G_ffn, md.view(s.M, s.NG_ffn))
    torch.cuda.synchronize()
    want_p, want_c = ref.reorder(host["mask_ffn"])
    assert np.array_equal(perm.cpu().numpy(), want_p) and np.array_equal(counts.cpu().numpy(), want_c)
    rows = np.arange(s.M)
    check_ffn(s, host, rows, bits_of(h), y.cpu().numpy().astype(np.float64))
    m2 = host["mask_ffn"].reshape(s.M, s.NG_ffn)
    assert (bits_of(h)[~ref.expand(m2, s.G_ffn)] == 0).all()


@pytest.mark.parametrize("B", [1, 4])
def test_decode_step_full_size(B):
    """Llama3.1-8B decode: B sequences with one new token each, KV cache 16384,
    half the groups off for every token (each token its own half)."""
    from masked_group_mask_amd.layer import DecodeLayer
    s = wl.shape("llama8b_decode", B=B)
    say("full-size decode", B)
    host = wl.make_layer(s, seed=1)
    layer = DecodeLayer(s, host, sets=1)
    layer.step(0)
    torch.cuda.synchronize()
    ma2 = host["mask_attn"].reshape(B, s.Hk)
    mf2 = host["mask_ffn"].reshape(B, s.NG_ffn)
    q_bits = bits_of(layer.q)
    want_q = ref.gemm_mn(host["x"], host["w_q"], ma2, s.G_attn)
    keep = ref.expand(ma2, s.G_attn)
    check_bf16_store(q_bits[keep], want_q[keep], "decode q_proj")
    want_o = ref.attention(active_only(q_bits, keep).reshape(B, 1, s.Hq, s.d), host["k"], host["v"],
                           host["mask_attn"])
    o_bits = bits_of(layer.o).reshape(B, s.Hq, s.d)
    keep_h = np.repeat(ma2 != 0, s.Hq // s.Hk, axis=1)
    check_attn_bf16(o_bits[keep_h], want_o.reshape(B, s.Hq, s.d)[keep_h], "decode attention")
    want_y = ref.gemm_k(active_only(o_bits, keep_h[..., None]).reshape(B, -1), host["w_o"], ma2, s.G_attn)
    check_gemm(layer.y_attn.cpu().numpy().astype(np.float64), want_y, "decode o_proj")
    check_ffn(s, host, np.arange(B), bits_of(layer.h), layer.y_ffn.cpu().numpy().astype(np.float64))
