"""Host-side checks of the Python binding (no GPU needed, nothing launched).

The C ABI receives bare pointers, so the binding is the last place where a
routing tensor of the wrong size (say the FFN mask handed to o_proj) can be
caught. These tests pass CPU tensors: every size check must fire before the
device check, and a call whose sizes are all right must stop at the device
check, so no pointer of a mis-sized tensor can reach a kernel.
"""
import pytest
import torch

import masked_group_mask_amd as mg

bf16, i32, u8 = torch.bfloat16, torch.int32, torch.uint8


def z(*shape, dtype=bf16):
    return torch.zeros(shape, dtype=dtype)


M, K, N, G = 64, 256, 512, 128          # GEMM-MN: NG = N / G = 4; GEMM-K: K / G = 2


def raises(match, fn, *a, **kw):
    with pytest.raises(ValueError, match=match):
        fn(*a, **kw)


def test_gemm_mn_routing_sizes():
    A, B = z(M, K), z(N, K)
    good = dict(perm=z(N // G, M, dtype=i32), counts=z(N // G, dtype=i32))
    raises("device", mg.gemm_mn, A, B, G, **good)
    raises("perm", mg.gemm_mn, A, B, G, perm=z(N // G, M - 1, dtype=i32), counts=good["counts"])
    raises("perm", mg.gemm_mn, A, B, G, perm=z(2 * N // G, M, dtype=i32), counts=good["counts"])
    raises("counts", mg.gemm_mn, A, B, G, perm=good["perm"], counts=z(N // G + 1, dtype=i32))
    raises("go together", mg.gemm_mn, A, B, G, perm=good["perm"])
    raises("mask", mg.gemm_mn, z(2, K), B, G, mask=z(2, N // G + 1, dtype=u8))
    raises("multiple", mg.gemm_mn, A, B, 100, **good)
    raises("device", mg.gemm_mn, z(2, K), B, G, mask=z(2, N // G, dtype=u8))


def test_gemm_mn_swiglu_routing_sizes_and_output():
    A, W = z(M, K), z(N, K)
    perm, counts = z(N // G, M, dtype=i32), z(N // G, dtype=i32)
    raises("device", mg.gemm_mn_swiglu, A, W, W, G, perm=perm, counts=counts)
    raises("perm", mg.gemm_mn_swiglu, A, W, W, G, perm=z(N // G, M + 1, dtype=i32), counts=counts)
    raises("out", mg.gemm_mn_swiglu, A, W, W, G, perm=perm, counts=counts, out=z(M, N - 8))
    # a host output tensor is refused even with every size right
    raises("device", mg.gemm_mn_swiglu, A, W, W, G, perm=perm, counts=counts, out=z(M, N))


def test_gemm_k_grouped_routing_sizes():
    A, B = z(M, K), z(N, K)
    perm, counts = z(K // G, M, dtype=i32), z(K // G, dtype=i32)
    raises("device", mg.gemm_k_grouped, A, B, G, perm, counts)
    raises("device", mg.gemm_k_grouped, A, B, G, perm[None], counts[None])   # reorder's batch-1 shapes
    # the FFN reorder handed to a smaller GEMM-K
    raises("perm", mg.gemm_k_grouped, A, B, G, z(4 * K // G, M, dtype=i32), counts)
    raises("counts", mg.gemm_k_grouped, A, B, G, perm, z(K // G + 1, dtype=i32))
    raises("needs perm", mg.gemm_k_grouped, A, B, G, None, counts)
    raises("multiple", mg.gemm_k_grouped, A, B, 96, perm, counts)
    raises("out", mg.gemm_k_grouped, A, B, G, perm, counts, out=z(M, N - 4, dtype=torch.float32))


def test_gemm_k_mask_size():
    A, B = z(M, K), z(N, K)
    raises("device", mg.gemm_k, A, B, G, z(M, K // G, dtype=u8))
    # the FFN-sized mask handed to a smaller GEMM-K
    raises("mask", mg.gemm_k, A, B, G, z(M, 4 * K // G, dtype=u8))
    raises("mask", mg.gemm_k, A, B, G, z(M - 1, K // G, dtype=u8))
    raises("multiple", mg.gemm_k, A, B, 96, z(M, 2, dtype=u8))
    raises("out", mg.gemm_k, A, B, G, z(M, K // G, dtype=u8), out=z(M, N, dtype=torch.float32)[:, :8])


def test_attn_routing_sizes():
    Bt, Tq, Hq, Hk, d = 2, 16, 8, 2, 128
    Q, KV = z(Bt, Tq, Hq, d), z(Bt, Tq, Hk, d)
    perm, counts = z(Bt, Hk, Tq, dtype=i32), z(Bt, Hk, dtype=i32)
    raises("device", mg.attn, Q, KV, KV, perm=perm, counts=counts)
    raises("perm", mg.attn, Q, KV, KV, perm=z(Bt, Hk, Tq - 1, dtype=i32), counts=counts)
    raises("counts", mg.attn, Q, KV, KV, perm=perm, counts=z(Bt, 4, dtype=i32))
    raises("leftpad", mg.attn, Q, KV, KV, perm=perm, counts=counts, leftpad=z(Bt + 1, dtype=i32))
    raises("mask", mg.attn, z(Bt, 1, Hq, d), KV, KV, mask=z(Bt, 1, Hk + 1, dtype=u8))
    # finer routing groups: perm/counts sized by the group count
    raises("perm", mg.attn, Q, KV, KV, perm=perm, counts=z(Bt, 4, dtype=i32), groups=4)
    raises("device", mg.attn, Q, KV, KV, perm=z(Bt, 4, Tq, dtype=i32), counts=z(Bt, 4, dtype=i32), groups=4)
