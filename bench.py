#!/usr/bin/env python3
"""Benchmark of the masked group-mask layer on one MI355X.

One step = one pass of the whole routed path of a transformer layer over one
batch of seeded synthetic input resident in HBM: reorder of the attention and
FFN masks, q_proj (GEMM-MN), head-group-masked causal GQA attention, o_proj
(GEMM-K), gate/up projections fused with SwiGLU (GEMM-MN) and down_proj
(GEMM-K). Default workload: Qwen3-14B-shaped layer prefill, T=8192, 50% of
the attention groups and 50% of the FFN groups inactive, FFN group size 128.

Prints one JSON line: active-FLOP TFLOP/s of the masked layer, the speedup
over the same kernels run with all-ones masks, the roofline of the dominant
kernel (timed with HIP events on the launch stream), decode steps of the
Llama3.1-8B shape for one and for four sequences (HBM bytes/s), and the CPU
oracle timed on a sample of the same workload.
"""
from __future__ import annotations

import argparse
import json
import os
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

METRIC = "active-FLOP TFLOP/s & speedup vs dense per masked layer at 50% sparsity"
PEAK_BF16_TFLOPS = 2500.0     # MI355X dense bf16 MFMA
PEAK_HBM_GBS = 8000.0         # MI355X HBM3E


def log(*a):
    print("[bench]", *a, file=sys.stderr, flush=True)


def time_steps(layer, which, steps, warmup, torch):
    ops = layer.ops
    for _ in range(warmup):
        layer.step(which)
    torch.cuda.synchronize()
    n_ev = len(ops) + 1
    evs = [[torch.cuda.Event(enable_timing=True) for _ in range(n_ev)] for _ in range(steps)]
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for i in range(steps):
        layer.step(which, evs[i])
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    per_op = {op: float(np.mean([evs[i][j].elapsed_time(evs[i][j + 1]) for i in range(steps)]))
              for j, op in enumerate(ops)}
    step_ms = [evs[i][0].elapsed_time(evs[i][-1]) for i in range(steps)]
    spread = {"p10": float(np.percentile(step_ms, 10)), "median": float(np.median(step_ms)),
              "p90": float(np.percentile(step_ms, 90))}
    return wall / steps * 1e3, per_op, spread


def hold_gpu(torch, ms: float) -> None:
    """Keep the current stream busy for about `ms` with torch's bounded spin
    kernel, so that the host can queue many short launches before the first
    one runs (their events then time the GPU, not the Python issue rate)."""
    sleep = getattr(torch.cuda, "_sleep", None)
    if sleep is None:
        return
    if not hasattr(hold_gpu, "cycles_per_ms"):
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record()
        sleep(1_000_000)
        e1.record()
        torch.cuda.synchronize()
        hold_gpu.cycles_per_ms = 1_000_000 / max(e0.elapsed_time(e1), 1e-3)
    sleep(int(ms * hold_gpu.cycles_per_ms))


def _time_decode(torch, layer, ops, steps, sets):
    """(per-op medians, whole step as individual launches, whole step as a
    replayed HIP graph), all in ms."""
    for i in range(5):
        layer.step(i)
    torch.cuda.synchronize()
    evs = [[torch.cuda.Event(enable_timing=True) for _ in range(len(ops) + 1)] for _ in range(steps)]
    hold_gpu(torch, 20.0)
    for i in range(steps):
        layer.step(i, evs[i])
    torch.cuda.synchronize()
    per_op = {op: float(np.median([evs[i][j].elapsed_time(evs[i][j + 1]) for i in range(steps)]))
              for j, op in enumerate(ops)}
    launch_ms = float(np.median([evs[i][0].elapsed_time(evs[i][-1]) for i in range(steps)]))
    graphs = []
    for k in range(sets):
        g = torch.cuda.CUDAGraph()
        with torch.cuda.graph(g):
            layer.step(k)
        graphs.append(g)
    for k in range(2 * sets):
        graphs[k % sets].replay()
    torch.cuda.synchronize()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    hold_gpu(torch, 5.0)
    e0.record()
    for i in range(steps):
        graphs[i % sets].replay()
    e1.record()
    torch.cuda.synchronize()
    return per_op, launch_ms, e0.elapsed_time(e1) / steps


def bench_decode(torch, wl, metrics, B=1, steps=50, sets=3):
    """Decode step of the Llama3.1-8B shape: B sequences with one new token
    each, KV cache of 16384 per sequence, half of the attention and FFN groups
    off for every token. Weight/KV sets rotate so the 256 MB
    Infinity Cache cannot hold the active set across steps.

    Timed two ways: as individual launches (HIP events around each op, the
    GPU held busy first so the host has queued every timed launch), and as a
    captured HIP graph of the step replayed back to back (whole step, gaps
    between kernels included). The headline rate is the graph replay's. The
    same kernels on all-ones masks (every weight and KV byte read) give the
    decode speedup."""
    from masked_group_mask_amd.layer import DECODE_OPS, DecodeLayer
    s = wl.shape("llama8b_decode", B=B)
    host = wl.make_layer(s, seed=1)
    nbytes = metrics.decode_bytes(s, host["mask_attn"], host["mask_ffn"])
    total = sum(nbytes.values())
    layer = DecodeLayer(s, host, sets=sets)
    per_op, launch_ms, graph_ms = _time_decode(torch, layer, DECODE_OPS, steps, sets)
    del layer
    ones = dict(host, mask_attn=np.ones_like(host["mask_attn"]), mask_ffn=np.ones_like(host["mask_ffn"]))
    dense_bytes = sum(metrics.decode_bytes(s, ones["mask_attn"], ones["mask_ffn"]).values())
    dense = DecodeLayer(s, ones, sets=sets)
    d_per_op, _, d_graph_ms = _time_decode(torch, dense, DECODE_OPS, steps, sets)
    del dense
    torch.cuda.empty_cache()
    return {
        "workload": ("llama8b_decode (B=%d, KV 16384 per sequence, 4/8 attention and 56/112 FFN groups "
                     "on per token)" % B),
        "active_bytes": total,
        "graph_ms_per_step": graph_ms,
        "launch_ms_per_step": launch_ms,
        "GB_per_s": total / (graph_ms * 1e-3) / 1e9,
        "frac_of_hbm_peak": total / (graph_ms * 1e-3) / 1e9 / PEAK_HBM_GBS,
        "per_op_ms": per_op,
        "per_op_GB_per_s": {op: nbytes[op] / (per_op[op] * 1e-3) / 1e9 for op in DECODE_OPS},
        "dense_graph_ms_per_step": d_graph_ms,
        "dense_GB_per_s": dense_bytes / (d_graph_ms * 1e-3) / 1e9,
        "dense_per_op_ms": d_per_op,
        "speedup_vs_dense": d_graph_ms / graph_ms,
        "ideal_speedup": dense_bytes / total,
        "timing": ("graph: %d back-to-back replays of the captured step; per op: median over %d steps "
                   "of HIP events around each launch; %d rotated weight/KV sets; dense = the same "
                   "kernels on all-ones masks" % (steps, steps, sets)),
    }


def bench_decode_groups(torch, wl, steps=50, sets=3, group_counts=(8, 16, 32)):
    """Decode of the attention sub-layer (q_proj, attention, o_proj) of the
    Llama3.1-8B shape (KV 16384) with routing groups of G_attn = (Hq / NG) d:
    NG = 8 (one group per KV head), 16 and 32 (one query head per group),
    half of the groups on, against the same kernels with every group on (the
    page's decode sweep over the attention group size, Appendix C, Fig. 13).
    A replayed HIP graph of the three ops, 3 rotated weight/KV sets."""
    import masked_group_mask_amd as mg
    s = wl.shape("llama8b_decode")
    host = wl.make_layer(s, seed=11, parts=("attn",))
    rng = np.random.default_rng(13)
    dev = "cuda"
    to = lambda a: torch.from_numpy(np.ascontiguousarray(a).view(np.int16)).view(torch.bfloat16).to(dev)  # noqa: E731
    base = {k: to(host[k]) for k in ("w_q", "w_o", "k", "v")}
    wsets = [base] + [{k: t.clone() for k, t in base.items()} for _ in range(sets - 1)]
    x = to(host["x"])
    q = torch.empty((1, s.Hq * s.d), dtype=torch.bfloat16, device=dev)
    o = torch.empty((1, 1, s.Hq, s.d), dtype=torch.bfloat16, device=dev)
    y = torch.empty((1, s.D), dtype=torch.float32, device=dev)
    ws = torch.empty(mg.attn_workspace_bytes(1, 1, s.Tkv, s.Hq, s.Hk, s.d), dtype=torch.uint8, device=dev)
    rows = []
    for NG in group_counts:
        G = s.Hq * s.d // NG
        half = np.zeros((1, 1, NG), np.uint8)
        half[0, 0, rng.permutation(NG)[: NG // 2]] = 1
        res = {}
        for name, m in (("masked", half), ("all_ones", np.ones_like(half))):
            md = torch.from_numpy(m).to(dev)

            def step(w, md=md):
                mg.gemm_mn(x, w["w_q"], G, mask=md.view(1, NG), out=q)
                mg.attn(q.view(1, 1, s.Hq, s.d), w["k"], w["v"], mask=md, out=o, workspace=ws, groups=NG)
                mg.gemm_k(o.view(1, -1), w["w_o"], G, md.view(1, NG), out=y)
            for i in range(3):
                step(wsets[i % sets])
            graphs = []
            for k in range(sets):
                g = torch.cuda.CUDAGraph()
                with torch.cuda.graph(g):
                    step(wsets[k])
                graphs.append(g)
            for k in range(2 * sets):
                graphs[k % sets].replay()
            torch.cuda.synchronize()
            e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            hold_gpu(torch, 5.0)
            e0.record()
            for i in range(steps):
                graphs[i % sets].replay()
            e1.record()
            torch.cuda.synchronize()
            res[name] = e0.elapsed_time(e1) / steps
        rows.append({"groups": NG, "G_attn": G, "masked_us": res["masked"] * 1e3,
                     "all_ones_us": res["all_ones"] * 1e3, "speedup": res["all_ones"] / res["masked"]})
        log(f"decode attention sub-layer NG={NG} (G_attn={G}): {res['masked'] * 1e3:.1f} us masked, "
            f"{res['all_ones'] * 1e3:.1f} us all-ones, {res['all_ones'] / res['masked']:.2f}x")
    return {"workload": "llama8b_decode attention sub-layer (q_proj, attention, o_proj), KV 16384, "
                        "half of the routing groups on", "rows": rows}


def bench_router(torch, wl, s, steps=50, rank=32):
    """The two routers of the bench layer (attention: Hk groups, FFN: NG_ffn
    groups; rank 32, seeded weights) on the same X, each followed by its
    reorder, as one call each. Reported beside the masked step, which starts
    from given masks."""
    import masked_group_mask_amd as mg
    X = torch.randn(s.M, s.D, device="cuda").to(torch.bfloat16)
    out = {"workload": "%s routers, rank %d, %d tokens" % (s.name, rank, s.M)}
    per = {}
    routers = ([("attention", s.Hk)] if s.Hk else []) + [("ffn", s.NG_ffn)]
    for name, NG in routers:
        w1, w2 = wl.router_weights(7, s.D, rank, NG)
        w1 = torch.from_numpy(w1.view(np.int16)).view(torch.bfloat16).cuda()
        w2 = torch.from_numpy(w2.view(np.int16)).view(torch.bfloat16).cuda()
        for _ in range(3):
            mg.router(X, w1, w2)
        torch.cuda.synchronize()
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        hold_gpu(torch, 5.0)
        e0.record()
        for _ in range(steps):
            mg.router(X, w1, w2)
        e1.record()
        torch.cuda.synchronize()
        per[name] = e0.elapsed_time(e1) / steps
    out["ms_with_reorder"] = per
    out["x_read_GB_per_s"] = {k: s.M * s.D * 2 / (v * 1e-3) / 1e9 for k, v in per.items()}
    return out


def bench_torch_dense(torch, s, ours_dense_ms: dict, steps=10, warmup=3):
    """Context row: the layer's dense bf16 GEMMs through torch (hipBLASLt),
    beside this library's kernels run on all-ones masks (the all-ones
    overhead; the page reports 98.60% of dense throughput at 0% sparsity).
    Attention is not compared. gate/up is two GEMMs plus torch's SiLU and
    product."""
    import torch.nn.functional as F
    dev = "cuda"
    r = lambda *shp: torch.randn(*shp, device=dev).to(torch.bfloat16)  # noqa: E731
    X = r(s.M, s.D)
    O = r(s.M, s.Hq * s.d)
    H = r(s.M, s.Dff)
    Wq, Wo = r(s.Hq * s.d, s.D) * 0.02, r(s.D, s.Hq * s.d) * 0.02
    Wg, Wu, Wd = r(s.Dff, s.D) * 0.02, r(s.Dff, s.D) * 0.02, r(s.D, s.Dff) * 0.02
    ops = {
        "q_proj": lambda: F.linear(X, Wq),
        "o_proj": lambda: F.linear(O, Wo),
        "gate_up_swiglu": lambda: F.silu(F.linear(X, Wg)) * F.linear(X, Wu),
        "down_proj": lambda: F.linear(H, Wd),
    }
    per = {}
    for name, fn in ops.items():
        for _ in range(warmup):
            fn()
        torch.cuda.synchronize()
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record()
        for _ in range(steps):
            fn()
        e1.record()
        torch.cuda.synchronize()
        per[name] = e0.elapsed_time(e1) / steps
    return {
        "what": "torch F.linear (hipBLASLt) dense bf16 GEMMs of the same layer; attention not compared",
        "per_op_ms": per,
        "library_all_ones_ms": {k: ours_dense_ms[k] for k in per},
        "library_throughput_vs_torch": {k: per[k] / ours_dense_ms[k] for k in per},
    }


def bench_app_a(torch, mg, sizes=(2048, 4096, 8192), G=128, reps=3, naive_limit_gb=80.0):
    """The page's GEMM pruning comparison (Appendix A, Fig. 11) on MI355X: for
    M-, N- and K-axis routing of C = A B^T with M = N = K = S and half of the
    routing units on, the time, active TFLOP/s and peak extra device memory of

      dense    -- torch F.linear (hipBLASLt) over the whole problem;
      naive    -- gather-scatter in torch ops: the selected rows (M axis) or
                  every token's own weight subset (N and K axes, a
                  [tokens][units][K] tensor) are materialised, multiplied
                  (batched matrix-vector products) and scattered back;
      grouped  -- after this library's reorder, one torch GEMM per group over
                  that group's active rows (the counts are read on the host,
                  a device-to-host synchronisation per call);
      fused    -- this library's kernels: reorder + GEMM-MN (M and N axes,
                  the M axis being the one-group case) or GEMM-K (K axis).

    Every token keeps exactly half of the groups (a random half per token),
    so the naive per-token gather has a fixed width. Peak memory excludes
    the dense output C (pre-allocated for every variant). A naive run whose
    gathered tensor would pass naive_limit_gb is skipped and reported so."""
    import torch.nn.functional as F
    dev = "cuda"
    out = {"what": "C = A B^T, bf16, half of the routing units on per token, G = %d; "
                   "time = median of %d runs (ms), peak = extra device memory beyond A, B and C (GB)" % (G, reps),
           "rows": []}

    def timed(fn):
        fn()
        torch.cuda.synchronize()
        base = torch.cuda.memory_allocated()
        torch.cuda.reset_peak_memory_stats()
        ts = []
        for _ in range(reps):
            e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            e0.record()
            fn()
            e1.record()
            torch.cuda.synchronize()
            ts.append(e0.elapsed_time(e1))
        return float(np.median(ts)), (torch.cuda.max_memory_allocated() - base) / 1e9

    for S in sizes:
        M = N = K = S
        gen = torch.Generator(device="cpu").manual_seed(S)
        A = torch.randn(M, K, generator=gen).to(torch.bfloat16).to(dev)
        B = (torch.randn(N, K, generator=gen) * 0.02).to(torch.bfloat16).to(dev)
        C = torch.empty(M, N, dtype=torch.bfloat16, device=dev)
        C32 = torch.empty(M, N, dtype=torch.float32, device=dev)
        NG = S // G
        R = NG // 2
        # every token keeps R random groups: sorted indices [M][R] and the mask [M][NG]
        pick = torch.rand(M, NG, generator=gen).argsort(dim=1)[:, :R].sort(dim=1).values
        mask = torch.zeros(M, NG, dtype=torch.uint8)
        mask.scatter_(1, pick, 1)
        pick, mask = pick.to(dev), mask.to(dev)
        rows = torch.randperm(M, generator=gen)[: M // 2].sort().values.to(dev)   # M axis: half the tokens
        mrow = torch.zeros(M, 1, dtype=torch.uint8, device=dev)
        mrow[rows] = 1
        units = (torch.arange(G, device=dev)[None, None, :] + pick[:, :, None] * G).reshape(M, R * G)
        dense_flops = 2.0 * M * N * K

        def add(axis, variant, ms, peak, note=""):
            out["rows"].append({"axis": axis, "S": S, "variant": variant, "ms": ms,
                                "active_tflops": dense_flops / 2 / (ms * 1e-3) / 1e12 if ms else None,
                                "peak_extra_gb": peak, "note": note})
            shown = "skipped" if ms is None else f"{ms:.3f} ms"
            pk_s = "n/a" if peak is None else f"+{peak:.2f} GB"
            log(f"app-A {axis} S={S} {variant}: {shown}, peak {pk_s} {note}")

        ms, pk = timed(lambda: torch.matmul(A, B.T, out=C))
        add("dense", "dense", ms, pk, "torch matmul, all units")

        # ---- M axis (depth routing: half of the token rows) ----
        def naive_m():
            Cm = torch.zeros(M, N, dtype=torch.bfloat16, device=dev)
            Cm[rows] = F.linear(A.index_select(0, rows), B)
            return Cm
        ms, pk = timed(naive_m)
        add("M", "naive", ms, pk - M * N * 2 / 1e9)
        pm = torch.empty(1, 1, M, dtype=torch.int32, device=dev)
        cm = torch.empty(1, 1, dtype=torch.int32, device=dev)

        def fused_m():
            mg.reorder(mrow.view(1, M, 1), pm, cm)
            mg.gemm_mn(A, B, N, perm=pm[0], counts=cm[0], out=C)
        ms, pk = timed(fused_m)
        add("M", "fused", ms, pk, "reorder + GEMM-MN with one group")

        # ---- N axis ----
        gathered_gb = M * R * G * K * 2 / 1e9
        if gathered_gb <= naive_limit_gb:
            def naive_n():
                Bsub = B.index_select(0, units.reshape(-1)).view(M, R * G, K)       # every token's rows of B
                Csub = torch.bmm(Bsub, A.unsqueeze(2)).squeeze(2)                    # [M][R G]
                Cn = torch.zeros(M, N, dtype=torch.bfloat16, device=dev)
                Cn.scatter_(1, units, Csub)
                return Cn
            ms, pk = timed(naive_n)
            add("N", "naive", ms, pk - M * N * 2 / 1e9)
        else:
            add("N", "naive", None, None, "skipped: the gathered weight tensor alone needs %.0f GB" % gathered_gb)
        perm, counts = mg.reorder(mask.view(1, M, NG))
        Bg = [B[g * G:(g + 1) * G].contiguous() for g in range(NG)]

        def grouped_n():
            cnt = counts[0].tolist()                       # device-to-host synchronisation
            for g in range(NG):
                r = perm[0, g, : cnt[g]].long()
                C[r, g * G:(g + 1) * G] = F.linear(A.index_select(0, r), Bg[g])
        ms, pk = timed(grouped_n)
        add("N", "grouped", ms, pk, "one torch GEMM per group after the reorder")

        def fused_n():
            mg.reorder(mask.view(1, M, NG), perm, counts)
            mg.gemm_mn(A, B, G, perm=perm[0], counts=counts[0], out=C)
        ms, pk = timed(fused_n)
        add("N", "fused", ms, pk, "reorder + GEMM-MN")

        # ---- K axis ----
        if gathered_gb <= naive_limit_gb:
            def naive_k():
                Asub = torch.gather(A, 1, units)                                     # [M][R G]
                Bsub = B.index_select(1, units.reshape(-1)).view(N, M, R * G).permute(1, 0, 2).contiguous()
                return torch.bmm(Bsub, Asub.unsqueeze(2)).squeeze(2)                 # [M][N]
            ms, pk = timed(naive_k)
            add("K", "naive", ms, pk - M * N * 2 / 1e9)
        else:
            add("K", "naive", None, None, "skipped: the gathered weight tensor alone needs %.0f GB" % gathered_gb)
        BgK = [B[:, g * G:(g + 1) * G].contiguous() for g in range(NG)]

        def grouped_k():
            cnt = counts[0].tolist()
            C32.zero_()
            for g in range(NG):
                r = perm[0, g, : cnt[g]].long()
                part = F.linear(A.index_select(0, r)[:, g * G:(g + 1) * G].contiguous(), BgK[g])
                C32.index_add_(0, r, part.float())
        ms, pk = timed(grouped_k)
        add("K", "grouped", ms, pk, "one torch GEMM per group after the reorder, index_add into fp32 C")

        def fused_k():
            mg.gemm_k(A, B, G, mask, out=C32)
        ms, pk = timed(fused_k)
        add("K", "fused", ms, pk, "GEMM-K (fp32 output)")
        del A, B, C, C32, Bg, BgK
        torch.cuda.empty_cache()
    return out


def bench_batched_leftpad(torch, wl, metrics, steps=5, warmup=5, T=4096, leftpad=(0, 1024)):
    """Two left-padded sequences through the same layer driver (the bench
    shape with B = 2, T = 4096: the same 8192 tokens, the keys before each
    sequence's padding excluded): masked and all-ones steps."""
    from masked_group_mask_amd.layer import PrefillLayer
    s = wl.shape("qwen14b_prefill", B=2, T=T)
    host = wl.make_layer(s, seed=5)
    layer = PrefillLayer(s, host, leftpad=leftpad)
    flops = sum(metrics.layer_flops(s, host["mask_attn"], host["mask_ffn"], leftpad=leftpad).values())
    ms, per_op, _ = time_steps(layer, "masked", steps, warmup, torch)
    dense_ms, _, _ = time_steps(layer, "dense", steps, warmup, torch)
    del layer
    torch.cuda.empty_cache()
    return {"workload": "qwen14b_prefill, B=2 x T=%d, leftpad %s, 50%% of the groups off" % (T, list(leftpad)),
            "ms_per_step": ms, "active_tflops": flops / (ms * 1e-3) / 1e12, "dense_ms_per_step": dense_ms,
            "speedup_vs_dense": dense_ms / ms, "per_op_ms": per_op}


def measured_peaks(torch, mg, copy_bytes=1 << 30, reps=10):
    """Rates this device sustains, beside the vendor figures: the bf16 MFMA
    rate of the library's probe kernel (independent MFMA chains from
    registers, 8 workgroups of 4 waves per compute unit) and a plain device
    copy (read + write of copy_bytes)."""
    props = torch.cuda.get_device_properties(0)
    blocks, iters = 8 * props.multi_processor_count, 4096
    sink = torch.empty(blocks * 4, dtype=torch.float32, device="cuda")
    mg.mfma_probe(blocks, 64, sink)
    torch.cuda.synchronize()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record()
    for _ in range(reps):
        mg.mfma_probe(blocks, iters, sink)
    e1.record()
    torch.cuda.synchronize()
    mfma = blocks * 4 * iters * 8 * 16384 / (e0.elapsed_time(e1) / reps * 1e-3) / 1e12
    n = copy_bytes // 4
    src = torch.ones(n, dtype=torch.float32, device="cuda")
    dst = torch.empty_like(src)
    torch.mul(src, 1.0, out=dst)
    torch.cuda.synchronize()
    e0.record()
    for _ in range(reps):
        torch.mul(src, 1.0, out=dst)
    e1.record()
    torch.cuda.synchronize()
    copy = 2 * n * 4 / (e0.elapsed_time(e1) / reps * 1e-3) / 1e9
    del src, dst
    torch.cuda.empty_cache()
    return {"mfma_bf16_tflops": mfma, "copy_read_write_GB_per_s": copy,
            "how": ("MFMA: wide_mfma_probe, %d workgroups x 4 waves x %d rounds of 8 independent "
                    "16x16x32 bf16 MFMAs; copy: torch elementwise copy of %d MiB, read + write"
                    % (blocks, iters, copy_bytes >> 20))}


def measured_traffic(op: str):
    """Bytes per launch of `op` from profiles/traffic.json (two rocprofv3
    counter passes, scaled by the same counters on a copy of known size), or
    None when no record covers `op` or its kernel sources changed since."""
    import hashlib
    path = os.path.join(ROOT, "profiles", "traffic.json")
    try:
        with open(path) as f:
            rec = json.load(f)
    except (OSError, ValueError):
        return None
    if rec.get("op") != op:
        return None
    for rel, sha in rec.get("sources_sha256", {}).items():
        try:
            with open(os.path.join(ROOT, rel), "rb") as f:
                if hashlib.sha256(f.read()).hexdigest() != sha:
                    return None
        except OSError:
            return None
    return float(rec["traffic_bytes_per_launch"])


def cpu_baseline(s, host, rows: int):
    """The CPU oracle on `rows` token rows of the same layer (all routed ops)."""
    from oracle import wide_ref as ref
    from masked_group_mask_amd import metrics
    # the oracle's BLAS runs on every core this process may use, and that is
    # the core count reported
    cores = len(os.sched_getaffinity(0))
    try:
        from threadpoolctl import threadpool_limits
        limiter = threadpool_limits(limits=cores, user_api="blas")
    except Exception:  # pragma: no cover - threadpoolctl missing
        limiter = None
    rng = np.random.default_rng(123)
    sel = np.sort(rng.choice(s.M, size=min(rows, s.M), replace=False))
    mf = host["mask_ffn"].reshape(s.M, s.NG_ffn)[sel]
    X = host["x"][sel]
    fl = 0
    t0 = time.perf_counter()
    if s.Hq:
        ma = host["mask_attn"].reshape(s.M, s.Hk)[sel]
        q = ref.round_bf16(ref.gemm_mn(X, host["w_q"], ma, s.G_attn))
        full_mask = host["mask_attn"]
        # attention needs Q only at the sampled positions; other rows are unused
        Qs = np.zeros((s.B, s.T, s.Hq, s.d), np.uint16)
        Qs[0, sel] = ref.to_bf16_bits(q).reshape(len(sel), s.Hq, s.d)
        o = ref.attention(Qs, host["k"], host["v"], full_mask, queries=[(0, int(t)) for t in sel])
        ref.gemm_k(ref.to_bf16_bits(ref.round_bf16(o)).reshape(len(sel), -1), host["w_o"], ma, s.G_attn)
    hh = ref.round_bf16(ref.swiglu(ref.gemm_mn(X, host["w_gate"], mf, s.G_ffn),
                                   ref.gemm_mn(X, host["w_up"], mf, s.G_ffn)))
    ref.gemm_k(ref.to_bf16_bits(hh), host["w_down"], mf, s.G_ffn)
    dt = time.perf_counter() - t0
    if limiter is not None:
        limiter.unregister()
    # active FLOPs of exactly the sampled rows
    fl += 2 * metrics.gemm_mn_flops(mf, s.D, s.G_ffn) + metrics.gemm_k_flops(mf, s.D, s.G_ffn)
    if s.Hq:
        fl += metrics.gemm_mn_flops(ma, s.D, s.G_attn) + metrics.gemm_k_flops(ma, s.D, s.G_attn)
        rep = s.Hq // s.Hk
        fl += int(sum(4 * s.d * rep * int(ma[i].sum()) * (int(t) + 1) for i, t in enumerate(sel)))
    cpu = "unknown"
    try:
        with open("/proc/cpuinfo") as f:
            cpu = next((ln.split(":", 1)[1].strip() for ln in f if ln.startswith("model name")), cpu)
    except OSError:
        pass
    return {"value": fl / dt / 1e12, "unit": "TFLOP/s", "cores": int(cores), "kind": "oracle",
            "cpu": cpu, "blas": np.show_config(mode="dicts").get("Build Dependencies", {}).get("blas", {}).get("name", "?"),
            "sample": f"{len(sel)} of {s.M} token rows of the same layer (all routed ops, float64), {dt:.1f} s",
            "seconds": dt}


def main():
    ap = argparse.ArgumentParser(description=__doc__, formatter_class=argparse.RawDescriptionHelpFormatter)
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=10)
    ap.add_argument("--warmup", type=int, default=10)
    ap.add_argument("--workload", default="qwen14b_prefill")
    ap.add_argument("--sparsity", type=float, default=None,
                    help="fraction of the attention and FFN groups off (default: the workload's own)")
    ap.add_argument("--sparsity-attn", type=float, default=None, help="overrides --sparsity for attention")
    ap.add_argument("--sparsity-ffn", type=float, default=None, help="overrides --sparsity for the FFN")
    ap.add_argument("--g-ffn", type=int, default=None, help="FFN group size (default: the workload's own)")
    ap.add_argument("--cpu-rows", type=int, default=8192)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-dense", action="store_true")
    ap.add_argument("--no-decode", action="store_true")
    ap.add_argument("--no-router", action="store_true")
    ap.add_argument("--no-torch-dense", action="store_true")
    ap.add_argument("--no-leftpad", action="store_true", help="skip the two left-padded sequences leg")
    ap.add_argument("--no-app-a", action="store_true",
                    help="skip the naive / grouped / fused GEMM pruning comparison (the page's Appendix A)")
    ap.add_argument("--ordered-k", default="", metavar="OPS",
                    help="comma-separated GEMM-K ops (o_proj, down_proj) to run over rows sorted by "
                         "routing pattern")
    ap.add_argument("--grouped-k", default="", metavar="OPS",
                    help="comma-separated GEMM-K ops (o_proj, down_proj) to compute group by group from the "
                         "reorder with atomic partial writes (the page's Algorithm 3)")
    ap.add_argument("--only", metavar="OP", default=None,
                    help="profiling aid: after one full masked step, run only this op --steps times")
    ap.add_argument("--copy-bytes", type=int, default=0,
                    help="profiling aid: run a plain device copy of this many bytes --steps times "
                         "(reference for the HBM byte counters)")
    args = ap.parse_args()

    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) != 1:
        print("bench.py measures one GPU only: the masked layer runs on a single MI355X and "
              "this library has no multi-GPU path (--gpus must be 1).", file=sys.stderr)
        sys.exit(2)

    import torch
    import masked_group_mask_amd as mg
    from masked_group_mask_amd import metrics, workloads as wl

    if not torch.cuda.is_available():
        print("bench.py needs a GPU", file=sys.stderr)
        sys.exit(1)
    mg.load()
    torch.cuda.set_device(0)
    if args.copy_bytes:
        n = args.copy_bytes // 4
        src = torch.ones(n, dtype=torch.float32, device="cuda")
        dst = torch.empty_like(src)
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        torch.mul(src, 1.0, out=dst)  # reads n*4 bytes, writes n*4 bytes
        torch.cuda.synchronize()
        e0.record()
        for _ in range(args.steps):
            torch.mul(src, 1.0, out=dst)
        e1.record()
        torch.cuda.synchronize()
        ms = e0.elapsed_time(e1) / args.steps
        log(f"copied {n * 4} bytes {args.steps} times: {ms:.3f} ms each, "
            f"{2 * n * 4 / (ms * 1e-3) / 1e9:.0f} GB/s read + write")
        return

    over = {}
    for key, v in (("p_attn", args.sparsity_attn), ("p_ffn", args.sparsity_ffn)):
        v = args.sparsity if v is None else v
        if v is not None:
            over[key] = 1.0 - v
    if args.g_ffn is not None:
        over["G_ffn"] = args.g_ffn
    s = wl.shape(args.workload, **over)
    if s.T == 1:
        print("bench.py times prefill workloads; the decode step is its own leg", file=sys.stderr)
        sys.exit(2)
    log(f"generating {s.name}: T={s.T} D={s.D} D'={s.Dff} Hq={s.Hq} Hk={s.Hk} G_ffn={s.G_ffn} "
        f"p_attn={s.p_attn} p_ffn={s.p_ffn} ({s.ffn_rule})")
    t0 = time.perf_counter()
    host = wl.make_layer(s, seed=0)
    log(f"inputs ready in {time.perf_counter() - t0:.1f} s")
    from masked_group_mask_amd.layer import PrefillLayer
    ordered = tuple(o for o in args.ordered_k.split(",") if o)
    grouped = tuple(o for o in args.grouped_k.split(",") if o)
    layer = PrefillLayer(s, host, with_dense=not args.no_dense, ordered_k=ordered, grouped_k=grouped)
    flops = metrics.layer_flops(s, host.get("mask_attn"), host["mask_ffn"])
    ones_a = np.ones_like(host["mask_attn"]) if s.Hq else None
    ones_f = np.ones_like(host["mask_ffn"])
    dense_flops = metrics.layer_flops(s, ones_a, ones_f)
    total_flops = sum(flops.values())

    if args.only:
        layer.step("masked")
        for _ in range(args.steps):
            layer.run(args.only, "masked")
        torch.cuda.synchronize()
        log(f"ran {args.only} {args.steps} times")
        return

    log("timing masked layer")
    ms, per_op, spread = time_steps(layer, "masked", args.steps, args.warmup, torch)
    log(f"masked: {ms:.3f} ms/step  " + " ".join(f"{k}={v:.3f}" for k, v in per_op.items()))
    dense_ms, dense_per_op = (None, None)
    if not args.no_dense:
        dense_ms, dense_per_op, _ = time_steps(layer, "dense", args.steps, args.warmup, torch)
        log(f"dense:  {dense_ms:.3f} ms/step  " + " ".join(f"{k}={v:.3f}" for k, v in dense_per_op.items()))

    value = total_flops / (ms * 1e-3) / 1e12
    # Dominant kernel: the routed op with the largest share of the masked step.
    dom = max((op for op in per_op if op != "reorder"), key=lambda k: per_op[k])
    achieved = flops[dom] / (per_op[dom] * 1e-3) / 1e12
    roof = {"kernel": dom, "bound": "mfma", "achieved": achieved, "peak": PEAK_BF16_TFLOPS,
            "unit": "TFLOP/s", "frac": achieved / PEAK_BF16_TFLOPS,
            # L2-to-memory bytes per launch (rocprofv3 FETCH_SIZE/WRITE_SIZE, copy-scaled)
            "traffic": measured_traffic(dom),
            "flops_per_launch": flops[dom], "avg_launch_ms": per_op[dom]}

    out = {
        "metric": METRIC, "value": value, "unit": "TFLOP/s", "n_gpus": 1, "steps": args.steps,
        "warmup": args.warmup, "ms_per_step": ms, "higher_is_better": True, "scaling": "weak",
        "vs_baseline": None, "dtype": "bf16", "data": "synthetic",
        "config": {"workload": s.name, "B": s.B, "T": s.T, "hidden": s.D, "ffn": s.Dff,
                   "q_heads": s.Hq, "kv_heads": s.Hk, "head_dim": s.d, "G_attn": s.G_attn,
                   "G_ffn": s.G_ffn, "sparsity_attn": round(1.0 - s.p_attn, 6) if s.Hq else None,
                   "sparsity_ffn": round(1.0 - s.p_ffn, 6), "ffn_mask_rule": s.ffn_rule, "seed": 0,
                   # GEMM-K form of o_proj / down_proj in the masked step (all-ones: token order)
                   "gemm_k": {op: ("pattern_order" if op in ordered else "per_group" if op in grouped
                                   else "token_order") for op in ("o_proj", "down_proj") if op in flops}},
        "speedup_vs_dense": (dense_ms / ms) if dense_ms else None,
        "ideal_speedup": sum(dense_flops.values()) / total_flops,
        "dense_ms_per_step": dense_ms,
        "active_gflop_per_step": total_flops / 1e9,
        "per_op_ms": per_op,
        "step_ms_events": spread,
        "per_op_tflops": {k: flops[k] / (per_op[k] * 1e-3) / 1e12 for k in flops},
        "dense_per_op_ms": dense_per_op,
        "roofline": roof,
    }
    out["measured_peaks"] = measured_peaks(torch, mg)
    log(f"measured peaks: MFMA bf16 {out['measured_peaks']['mfma_bf16_tflops']:.0f} TFLOP/s, "
        f"copy {out['measured_peaks']['copy_read_write_GB_per_s']:.0f} GB/s")
    out["roofline"]["measured_peak"] = out["measured_peaks"]["mfma_bf16_tflops"]
    out["roofline"]["frac_of_measured_peak"] = achieved / out["measured_peaks"]["mfma_bf16_tflops"]
    if not args.no_dense and not args.no_torch_dense and s.Hq:
        out["torch_dense"] = bench_torch_dense(torch, s, out["dense_per_op_ms"])
        log("torch dense GEMMs (ms): " + ", ".join(f"{k} {v:.3f}" for k, v in out["torch_dense"]["per_op_ms"].items()))
    if not args.no_dense and not args.no_leftpad:
        log("timing two left-padded sequences")
        out["prefill_b2_leftpad"] = bench_batched_leftpad(torch, wl, metrics)
        log(f"B=2 leftpad: {out['prefill_b2_leftpad']['ms_per_step']:.3f} ms/step, "
            f"{out['prefill_b2_leftpad']['speedup_vs_dense']:.2f}x all-ones")
    if not args.no_app_a:
        log("timing the naive / grouped / fused GEMM pruning comparison")
        out["app_a_gemm_pruning"] = bench_app_a(torch, mg)
    if not args.no_router:
        out["router"] = bench_router(torch, wl, s)
        log("routers (+reorder): " + ", ".join(f"{k} {v * 1e3:.1f} us"
                                                for k, v in out["router"]["ms_with_reorder"].items()))
    if not args.no_decode:
        log("timing decode step")
        out["decode"] = bench_decode(torch, wl, metrics, B=1)
        log(f"decode: {out['decode']['graph_ms_per_step'] * 1e3:.1f} us, "
            f"{out['decode']['GB_per_s']:.0f} GB/s, {out['decode']['speedup_vs_dense']:.2f}x all-ones "
            f"({out['decode']['dense_GB_per_s']:.0f} GB/s)")
        out["decode_groups"] = bench_decode_groups(torch, wl)
        out["decode_b4"] = bench_decode(torch, wl, metrics, B=4)
        log(f"decode B=4: {out['decode_b4']['graph_ms_per_step'] * 1e3:.1f} us, "
            f"{out['decode_b4']['GB_per_s']:.0f} GB/s")
    if not args.no_cpu_baseline:
        log(f"timing CPU oracle on {args.cpu_rows} rows")
        out["cpu_baseline"] = cpu_baseline(s, host, args.cpu_rows)
        log(f"cpu: {out['cpu_baseline']['value'] * 1e3:.2f} GFLOP/s in {out['cpu_baseline']['seconds']:.1f} s")
    print(json.dumps(out), flush=True)


if __name__ == "__main__":
    main()
