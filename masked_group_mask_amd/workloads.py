"""Seeded synthetic inputs for the masked-layer workloads.

This module only draws random numbers and lays them out; it contains none of
the method's arithmetic. Both the HIP path (through the tests and the bench)
and the CPU oracle consume exactly the arrays made here.

Conventions
-----------
* Every floating-point tensor is returned as raw bfloat16 bits (``uint16``),
  rounded from float32 with round-to-nearest-even.
* Masks are ``uint8`` 0/1 arrays laid out token-major, ``[B][T][N_G]``
  (WIDE p1 section 3.1, Eq. 2 and Eq. 3: one binary decision per token and
  per group).
* Weights are ``[out_features][in_features]`` row-major, so a projection is
  ``C = A @ B^T`` with ``B`` of shape ``[N][K]`` (WIDE p1 section 3.3).
* Each tensor has its own PCG64 stream spawned from ``SeedSequence(seed)`` in
  the fixed order ``STREAM_ORDER``; adding a tensor never changes another's
  values.
"""
from __future__ import annotations

import dataclasses
from typing import Dict, Optional

import numpy as np

STREAM_ORDER = (
    "mask_attn", "mask_ffn", "x", "w_q", "w_o", "w_gate", "w_up", "w_down",
    "k", "v", "q", "aux",
)


@dataclasses.dataclass(frozen=True)
class LayerShape:
    """Shape of one masked transformer layer (names follow WIDE p1 section 3.1)."""
    name: str
    B: int            # batch
    T: int            # query tokens per sequence (Tq)
    D: int            # hidden size
    Dff: int          # FFN intermediate size D'
    G_ffn: int        # FFN group size
    Hq: int = 0       # query heads (0: FFN-only workload)
    Hk: int = 0       # key/value heads
    d: int = 128      # head size
    Tk: int = 0       # keys per sequence (0: same as T, prefill)
    p_attn: float = 0.5     # probability that an attention group is active
    p_ffn: float = 0.5      # probability that an FFN group is active
    ffn_rule: str = "bern"  # "bern" | "beta22" | "half"
    attn_rule: str = "bern"  # "bern" | "half"

    @property
    def M(self) -> int:
        return self.B * self.T

    @property
    def Tkv(self) -> int:
        return self.Tk if self.Tk else self.T

    @property
    def G_attn(self) -> int:
        return (self.Hq // self.Hk) * self.d if self.Hk else 0

    @property
    def NG_ffn(self) -> int:
        return self.Dff // self.G_ffn

    @property
    def NG_attn(self) -> int:
        return self.Hk


def shape(name: str, **over) -> LayerShape:
    """The five workloads, by name, optionally with fields overridden."""
    base = {
        # Tiny masked SwiGLU FFN, T=64, hidden 256, ffn 1024, G=128, Bern(0.5).
        "tiny_ffn": LayerShape("tiny_ffn", B=1, T=64, D=256, Dff=1024, G_ffn=128,
                               p_ffn=0.5),
        # Llama3.2-3B-shaped FFN prefill, T=4096, per-group Beta(2,2) rates.
        "llama3b_ffn": LayerShape("llama3b_ffn", B=1, T=4096, D=3072, Dff=8192,
                                  G_ffn=128, p_ffn=0.5, ffn_rule="beta22"),
        # Llama3.1-8B-shaped prefill layer, T=16384, 66% attention / 28% FFN
        # sparsity (the learned rates reported in WIDE p1 section 4.4).
        "llama8b_prefill": LayerShape("llama8b_prefill", B=1, T=16384, D=4096,
                                      Dff=14336, G_ffn=128, Hq=32, Hk=8,
                                      p_attn=0.34, p_ffn=0.72),
        # Llama3.1-8B-shaped decode step, KV cache 16384, half the groups off.
        "llama8b_decode": LayerShape("llama8b_decode", B=1, T=1, Tk=16384,
                                     D=4096, Dff=14336, G_ffn=128, Hq=32, Hk=8,
                                     attn_rule="half", ffn_rule="half"),
        # Qwen3-14B-shaped full-layer prefill, T=8192 (sparsity and G_ffn swept).
        "qwen14b_prefill": LayerShape("qwen14b_prefill", B=1, T=8192, D=5120,
                                      Dff=17408, G_ffn=128, Hq=40, Hk=8,
                                      p_attn=0.5, p_ffn=0.5),
    }[name]
    return dataclasses.replace(base, **over) if over else base


def f32_to_bf16_bits(x: np.ndarray) -> np.ndarray:
    """Round float32 to bfloat16 bits, round-to-nearest-even (finite inputs)."""
    u = np.ascontiguousarray(x, dtype=np.float32).view(np.uint32)
    bias = ((u >> np.uint32(16)) & np.uint32(1)) + np.uint32(0x7FFF)
    return ((u + bias) >> np.uint32(16)).astype(np.uint16)


def bf16_bits_to_f32(bits: np.ndarray) -> np.ndarray:
    """Widen bfloat16 bits to float32 (exact)."""
    return (np.asarray(bits, dtype=np.uint16).astype(np.uint32) << np.uint32(16)).view(np.float32)


def _rng(seed: int):
    ss = np.random.SeedSequence(seed)
    kids = ss.spawn(len(STREAM_ORDER))
    return {name: np.random.Generator(np.random.PCG64(k)) for name, k in zip(STREAM_ORDER, kids)}


def normal_bf16(rng: np.random.Generator, shp, std: float) -> np.ndarray:
    out = rng.standard_normal(size=shp, dtype=np.float32)
    if std != 1.0:
        out *= np.float32(std)
    return f32_to_bf16_bits(out)


def draw_mask(rng: np.random.Generator, M: int, NG: int, p: float, rule: str) -> np.ndarray:
    """Binary mask [M][NG], uint8.

    bern   : independent Bernoulli(p) per (token, group).
    beta22 : per-group rate p_g ~ Beta(2,2), rescaled so the mean rate is p and
             clipped to [0,1]; then Bernoulli(p_g) per token.
    half   : exactly NG//2 groups active for every token, the active set drawn
             by one seeded permutation (a decode step has a single token).
    """
    if rule == "bern":
        return (rng.random((M, NG)) < p).astype(np.uint8)
    if rule == "beta22":
        pg = rng.beta(2.0, 2.0, size=NG)
        pg = np.clip(pg * (p / pg.mean()), 0.0, 1.0)
        return (rng.random((M, NG)) < pg[None, :]).astype(np.uint8)
    if rule == "half":
        m = np.zeros((M, NG), np.uint8)
        for i in range(M):
            m[i, rng.permutation(NG)[: NG // 2]] = 1
        return m
    raise ValueError(f"unknown mask rule {rule!r}")


def make_layer(s: LayerShape, seed: int = 0, parts=("attn", "ffn"),
               w_std: float = 0.02, kv_std: Optional[float] = None) -> Dict[str, np.ndarray]:
    """All inputs of one masked layer as numpy arrays.

    Keys: x [M][D]; mask_ffn [B][T][NG_ffn]; w_gate, w_up [Dff][D]; w_down [D][Dff];
    and for attention: mask_attn [B][T][Hk]; w_q [Hq*d][D]; w_o [D][Hq*d];
    k, v [B][Tkv][Hk][d].

    K and V stand for the dense K/V projections, which lie outside the masked
    path; they are drawn directly, N(0, kv_std). kv_std defaults to
    sqrt(D)*w_std (the scale of X W^T for X ~ N(0,1)) for prefill and to 1.0
    for a decode KV cache.
    """
    r = _rng(seed)
    out: Dict[str, np.ndarray] = {}
    out["x"] = normal_bf16(r["x"], (s.M, s.D), 1.0)
    if "ffn" in parts:
        out["mask_ffn"] = draw_mask(r["mask_ffn"], s.M, s.NG_ffn, s.p_ffn,
                                    s.ffn_rule).reshape(s.B, s.T, s.NG_ffn)
        out["w_gate"] = normal_bf16(r["w_gate"], (s.Dff, s.D), w_std)
        out["w_up"] = normal_bf16(r["w_up"], (s.Dff, s.D), w_std)
        out["w_down"] = normal_bf16(r["w_down"], (s.D, s.Dff), w_std)
    if "attn" in parts and s.Hq:
        if kv_std is None:
            kv_std = 1.0 if s.T == 1 else float(np.sqrt(s.D) * w_std)
        out["mask_attn"] = draw_mask(r["mask_attn"], s.M, s.Hk, s.p_attn,
                                     s.attn_rule).reshape(s.B, s.T, s.Hk)
        out["w_q"] = normal_bf16(r["w_q"], (s.Hq * s.d, s.D), w_std)
        out["w_o"] = normal_bf16(r["w_o"], (s.D, s.Hq * s.d), w_std)
        out["k"] = normal_bf16(r["k"], (s.B, s.Tkv, s.Hk, s.d), kv_std)
        out["v"] = normal_bf16(r["v"], (s.B, s.Tkv, s.Hk, s.d), kv_std)
    return out


def router_weights(seed: int, D: int, r: int, NG: int):
    """Seeded bottleneck-router weights in the library's [out][in] layout:
    W1 [r][D] ~ N(0, 1/sqrt(D)) and W2 [2 NG][r] ~ N(0, 1/sqrt(r)), so that for
    X ~ N(0, 1) the logits are O(1) and about half the groups run."""
    rng = np.random.Generator(np.random.PCG64(np.random.SeedSequence([seed, 0x5EED])))
    w1 = normal_bf16(rng, (r, D), float(D) ** -0.5)
    w2 = normal_bf16(rng, (2 * NG, r), float(r) ** -0.5)
    return w1, w2


def random_bf16(seed: int, shp, std: float = 1.0) -> np.ndarray:
    """A single seeded bf16 tensor (for unit-level tests)."""
    return normal_bf16(np.random.Generator(np.random.PCG64(seed)), shp, std)


def random_mask(seed: int, shp, p: float = 0.5) -> np.ndarray:
    """A single seeded Bernoulli(p) uint8 mask of any shape."""
    return (np.random.Generator(np.random.PCG64(seed)).random(shp) < p).astype(np.uint8)
