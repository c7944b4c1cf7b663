"""The bench's work counters agree with the oracle's own counters (CPU)."""
import numpy as np

from masked_group_mask_amd import metrics, workloads as wl
from oracle import wide_ref as ref


def test_layer_flops_match_oracle_counts():
    s = wl.shape("qwen14b_prefill", T=96, D=256, Dff=512, Hq=10, Hk=2, G_ffn=64)
    ma = wl.random_mask(1, (1, s.T, s.Hk), 0.5)
    mf = wl.random_mask(2, (1, s.T, s.NG_ffn), 0.5)
    got = metrics.layer_flops(s, ma, mf)
    m2a = ma.reshape(s.M, s.Hk)
    m2f = mf.reshape(s.M, s.NG_ffn)
    assert got["q_proj"] == ref.flops_gemm_mn(m2a, s.D, s.G_attn)
    assert got["o_proj"] == ref.flops_gemm_k(m2a, s.D, s.G_attn)
    assert got["attention"] == ref.flops_attention(ma, s.T, s.Hq, s.d)
    assert got["gate_up_swiglu"] == 2 * ref.flops_gemm_mn(m2f, s.D, s.G_ffn)
    assert got["down_proj"] == ref.flops_gemm_k(m2f, s.D, s.G_ffn)


def test_attention_flops_decode_and_offset():
    m = wl.random_mask(3, (2, 5, 4), 0.5)
    assert metrics.attention_flops(m, 9, 8, 16) == ref.flops_attention(m, 9, 8, 16)
    assert metrics.attention_flops(m, 9, 8, 16, causal=False) == ref.flops_attention(m, 9, 8, 16, causal=False)


def test_decode_bytes_match_oracle():
    s = wl.shape("llama8b_decode")
    x = wl.make_layer(s, seed=1, parts=())
    ma = np.array([1, 0, 1, 1, 0, 0, 1, 0])
    mf = (np.arange(112) % 2).astype(np.uint8)
    got = sum(metrics.decode_bytes(s, ma, mf).values())
    assert got == ref.decode_bytes(ma, mf, s.D, s.Hq, s.Hk, s.d, s.G_ffn, s.Tk)
    assert x["x"].shape == (1, 4096)


def test_decode_bytes_batched_match_oracle():
    s = wl.shape("llama8b_decode", B=4)
    h = wl.make_layer(s, seed=2, parts=("attn", "ffn"))
    ma, mf = h["mask_attn"], h["mask_ffn"]
    got = sum(metrics.decode_bytes(s, ma, mf).values())
    assert got == ref.decode_bytes(ma.reshape(4, s.Hk), mf.reshape(4, s.NG_ffn), s.D, s.Hq, s.Hk, s.d,
                                   s.G_ffn, s.Tk)
    assert int(ma.sum()) == 4 * s.Hk // 2     # "half" rule: every token keeps exactly half


def test_attention_flops_with_leftpad_match_oracle():
    m = wl.random_mask(4, (3, 11, 2), 0.6)
    for lp in ([0, 4, 11], [2, 0, 7]):
        assert metrics.attention_flops(m, 11, 6, 16, leftpad=lp) == ref.flops_attention(m, 11, 6, 16, leftpad=lp)
        assert metrics.attention_flops(m, 15, 6, 16, leftpad=lp) == ref.flops_attention(m, 15, 6, 16, leftpad=lp)
