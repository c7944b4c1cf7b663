"""GPU parity of prefill attention on seeded random shapes: batch, query and
key lengths around the 64-key stage and 256-row tile boundaries, bottom-right
alignment (Tk > Tq), per-sequence left padding (rows left with no valid key
must be 0), causal and not, routing groups at and below the KV-head
granularity, activity from none to all, fp32 and bf16 outputs. Bars as in
the other attention tests."""
import numpy as np
import pytest

from oracle import wide_ref as ref
from masked_group_mask_amd import workloads as wl

from helpers import bits_of, check_attn, check_attn_bf16, f32_of, say, to_dev

pytestmark = pytest.mark.gpu
torch = pytest.importorskip("torch")


@pytest.fixture(scope="module", autouse=True)
def gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import masked_group_mask_amd as mg
    mg.load()


def _cases(n=20, seed=77):
    rng = np.random.default_rng(seed)
    heads = [(8, 2), (16, 8), (40, 8), (4, 4), (32, 8)]
    cases = []
    while len(cases) < n:
        B = int(rng.integers(1, 4))
        Hq, Hk = heads[int(rng.integers(len(heads)))]
        finer = [g for g in (2 * Hk, 4 * Hk) if Hq % g == 0]
        NG = int(rng.choice([Hk] + finer)) if finer and rng.random() < 0.4 else Hk
        Tq = int(rng.choice([2, 63, 64, 65, 255, 256, 257, 700, 1200]))
        Tk = Tq + int(rng.choice([0, 0, 1, 100, 513]))
        if B * Tq * Hq * Tk * 128 > 3e9:    # keep the fp64 oracle quick
            continue
        causal = bool(rng.integers(0, 2))
        lp = None
        if rng.random() < 0.5:
            lp = [int(rng.choice([0, rng.integers(0, Tk)])) for _ in range(B)]
        p = float(rng.choice([0.0, 0.3, 0.7, 1.0]))
        dt = str(rng.choice(["f32", "bf16"]))
        cases.append((B, Tq, Tk, Hq, Hk, NG, causal, lp, p, dt, int(rng.integers(1 << 30))))
    return cases


@pytest.mark.parametrize("B,Tq,Tk,Hq,Hk,NG,causal,lp,p,dt,seed", _cases())
def test_attention_prefill_random_shapes(B, Tq, Tk, Hq, Hk, NG, causal, lp, p, dt, seed):
    import masked_group_mask_amd as mg
    d = 128
    Q = wl.random_bf16(seed, (B, Tq, Hq, d))
    K = wl.random_bf16(seed + 1, (B, Tk, Hk, d))
    V = wl.random_bf16(seed + 2, (B, Tk, Hk, d))
    mask = wl.random_mask(seed + 3, (B, Tq, NG), p)
    say("attention random", B, Tq, Tk, Hq, Hk, NG, causal, lp, p, dt)
    perm, counts = mg.reorder(to_dev(mask, torch))
    lpd = None if lp is None else to_dev(np.array(lp, np.int32), torch)
    out_dtype = torch.float32 if dt == "f32" else torch.bfloat16
    out = torch.zeros((B, Tq, Hq, d), dtype=out_dtype, device="cuda")
    mg.attn(to_dev(Q, torch), to_dev(K, torch), to_dev(V, torch), perm=perm, counts=counts, causal=causal,
            leftpad=lpd, out=out, groups=NG)
    torch.cuda.synchronize()
    want = ref.attention(Q, K, V, mask, causal=causal, leftpad=lp)
    keep = np.repeat(mask != 0, Hq // NG, axis=2)
    if dt == "f32":
        check_attn(f32_of(out), want, "random prefill")
        assert (out.cpu().numpy().view(np.uint32)[~keep] == 0).all()
    else:
        bits = bits_of(out)
        if keep.any():
            check_attn_bf16(bits[keep], want[keep], "random prefill bf16")
        assert (bits[~keep] == 0).all()
