"""Test helpers: moving seeded numpy inputs to the device and comparing results
with the oracle at the stated tolerances."""
import sys

import numpy as np

from oracle import wide_ref as ref

# GEMM outputs (fp32 stores): max |err| <= GEMM_RTOL * RMS(oracle over all entries).
GEMM_RTOL = 1e-2
# Attention outputs (fp32 stores): max |err| <= ATTN_ATOL.
ATTN_ATOL = 2e-2


def say(*a):
    """Name the GPU case about to run (flushed, so a crash still shows it)."""
    print("[gpu]", *a, file=sys.stderr, flush=True)


def to_dev(x, torch):
    """numpy array -> device tensor; uint16 arrays are bf16 bit patterns."""
    x = np.ascontiguousarray(x)
    if x.dtype == np.uint16:
        return torch.from_numpy(x.view(np.int16)).view(torch.bfloat16).cuda()
    return torch.from_numpy(x).cuda()


def bits_of(t):
    """bf16 device tensor -> numpy uint16 bit patterns."""
    import torch
    return t.detach().view(torch.int16).cpu().numpy().view(np.uint16)


def f32_of(t):
    return t.detach().float().cpu().numpy().astype(np.float64)


def check_gemm(got, want, what=""):
    rms = float(np.sqrt(np.mean(want ** 2))) if want.size else 0.0
    err = float(np.max(np.abs(got - want))) if want.size else 0.0
    assert err <= GEMM_RTOL * rms + 1e-30, f"{what}: max|err| {err:.3e} > 1e-2 x RMS {rms:.3e}"
    return err, rms


def check_attn(got, want, what=""):
    err = float(np.max(np.abs(got - want))) if want.size else 0.0
    assert err <= ATTN_ATOL, f"{what}: max|err| {err:.3e} > {ATTN_ATOL}"
    return err


def check_attn_bf16(got_bits, want64, what=""):
    """bf16-stored attention output: the fp32 bar plus one bf16 rounding."""
    err = np.abs(ref.from_bf16(got_bits) - want64)
    bound = ATTN_ATOL + 2.0 ** -8 * np.abs(want64)
    bad = np.count_nonzero(err > bound)
    assert bad == 0, f"{what}: {bad} outputs beyond 2e-2 + one bf16 step (max err {err.max():.3e})"
    return float(err.max()) if err.size else 0.0


def check_bf16_store(got_bits, want64, what=""):
    """A bf16-stored result is within one bf16 step of the oracle's rounded value.

    Where the exact result is small against the output's RMS (cancellation in
    the fp32 sum), the fp32 accumulation error, not the rounding, dominates;
    there an absolute error of 1e-3 x RMS is accepted as well.
    """
    want_bits = ref.to_bf16_bits(want64).astype(np.int32)
    g = got_bits.astype(np.int32)
    same_sign = (g >> 15) == (want_bits >> 15)
    step = np.abs(g - want_bits)
    rms = float(np.sqrt(np.mean(want64 ** 2))) if want64.size else 0.0
    err = np.abs(ref.from_bf16(got_bits) - want64)
    ok = (same_sign & (step <= 1)) | (err <= 2.0 ** -8 * np.abs(want64) + 1e-3 * rms)
    bad = np.count_nonzero(~ok)
    if bad:
        i = np.flatnonzero(~ok)[:5]
        detail = ", ".join(f"got {float(ref.from_bf16(got_bits[j])):.6g} want {float(want64[j]):.6g}" for j in i)
        raise AssertionError(f"{what}: {bad} bf16 outputs more than one step from the oracle "
                             f"(RMS {rms:.3g}): {detail}")
    return float(np.mean(g != want_bits)) if g.size else 0.0
