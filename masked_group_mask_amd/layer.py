"""Device-resident masked layer: buffers and the launch sequence of one step.

A prefill step runs, on the current stream: the reorder of the attention and
FFN masks, q_proj (GEMM-MN), attention, o_proj (GEMM-K), the gate/up
projections fused with SwiGLU (GEMM-MN) and down_proj (GEMM-K). A decode step
runs the matrix-vector variants and split-KV attention on one token, reading
the mask bytes directly. All buffers are allocated once here; a step launches
kernels only.
"""
from __future__ import annotations

import numpy as np
import torch

from . import _lib as mg

PREFILL_OPS = ("reorder", "q_proj", "attention", "o_proj", "gate_up_swiglu", "down_proj")
# A shape without query heads is an FFN-only layer: the FFN reorder, gate/up, down.
FFN_OPS = ("reorder", "gate_up_swiglu", "down_proj")
DECODE_OPS = ("q_proj", "attention", "o_proj", "gate_up_swiglu", "down_proj")


def to_device(x: np.ndarray) -> torch.Tensor:
    """numpy -> device tensor; uint16 arrays are bf16 bit patterns."""
    x = np.ascontiguousarray(x)
    if x.dtype == np.uint16:
        return torch.from_numpy(x.view(np.int16)).view(torch.bfloat16).cuda()
    return torch.from_numpy(x).cuda()


class PrefillLayer:
    """One masked layer of shape `s` (workloads.LayerShape) on the GPU; with
    s.Hq == 0 only its FFN (the ops in FFN_OPS)."""

    def __init__(self, s, host: dict, with_dense: bool = True, scheduled_mn: dict | None = None,
                 ordered_k: tuple = (), leftpad=None, grouped_k: tuple = ()):
        self.s = s
        # GEMM-K ops that run over rows sorted by routing pattern in the
        # masked step (their tiles skip the K-groups and 16-row fragments
        # whose rows all skip a group). All-ones masks have nothing to skip,
        # so the dense reference keeps token order there.
        # Off by default: measured on MI355X at the Qwen3-14B shape, the
        # ordered o_proj runs 0.35 against 0.37 ms in token order but its
        # sort adds ~0.02 ms (one workgroup, latency-bound), inline or on a
        # side stream, so the step gains nothing.
        self.ordered_k = tuple(ordered_k)
        # GEMM-K ops computed group by group from the reorder with atomic
        # partial writes (the page's Algorithm 3) in the masked step. Off by
        # default: measured on MI355X at the Qwen3-14B shape the atomic adds
        # bound it (o_proj 0.6 against 0.37 ms, down_proj at G = 256 4.3
        # against 1.16 ms).
        self.grouped_k = tuple(grouped_k)
        if set(self.ordered_k) & set(self.grouped_k):
            raise ValueError("an op runs either over pattern-sorted rows or group by group")
        # GEMM-MN ops that take the workspace (tiles scheduled from counts on
        # the device, group by group, and a short last round split along K),
        # per mask set. Routed masks give every group its own row set, so
        # tiles of one group running together share its weights; all-ones
        # masks give every group the same rows, where the static raster (tiles
        # of several groups over the same rows at once) is faster (MI355X,
        # Qwen3-14B prefill shape: gate/up 2.32 against 2.47 ms), so the dense
        # reference keeps it.
        if scheduled_mn is None:
            scheduled_mn = {"masked": ("q_proj", "gate_up_swiglu"), "dense": ()}
        self.scheduled_mn = {k: tuple(v) for k, v in scheduled_mn.items()}
        self.attn = s.Hq > 0
        self.ops = PREFILL_OPS if self.attn else FFN_OPS
        if not self.attn and (leftpad is not None or "o_proj" in self.ordered_k + self.grouped_k):
            raise ValueError("an FFN-only layer has no o_proj and no left padding")
        d = lambda k: to_device(host[k])  # noqa: E731
        self.x = d("x")
        self.wg, self.wu, self.wd = d("w_gate"), d("w_up"), d("w_down")
        mf = d("mask_ffn")
        ma = d("mask_attn") if self.attn else None
        self.masks = {"masked": (ma, mf)}
        if with_dense:
            self.masks["dense"] = (None if ma is None else torch.ones_like(ma), torch.ones_like(mf))
        dev = self.x.device
        M, B, T = s.M, s.B, s.T
        i32 = torch.int32
        self.perm_f = torch.empty((1, s.NG_ffn, M), dtype=i32, device=dev)
        self.cnt_f = torch.empty((1, s.NG_ffn), dtype=i32, device=dev)
        self.order_f = torch.empty(M, dtype=i32, device=dev)
        # Every consumer reads only the active entries of its input (GEMM-K
        # loads only the active (row, group) segments, attention gathers active
        # rows), so the intermediate buffers need no zero-initialisation.
        self.h = torch.empty((M, s.Dff), dtype=torch.bfloat16, device=dev)
        self.y_ffn = torch.empty((M, s.D), dtype=torch.float32, device=dev)
        wsb = max(mg.gemm_k_workspace_bytes(M, s.D, s.Dff), mg.gemm_mn_workspace_bytes(M, s.Dff, s.D, s.G_ffn, True))
        if not self.attn:
            self.ws = torch.empty(max(wsb, 16), dtype=torch.uint8, device=dev)
            return
        self.wq, self.wo = d("w_q"), d("w_o")
        self.k, self.v = d("k"), d("v")
        # Attention reorders each sequence's routing columns (batch B, rows
        # T); the GEMMs reorder the flattened tokens (batch 1, rows B*T). With
        # B = 1 the two coincide and one reorder serves both.
        self.perm_a = torch.empty((B, s.Hk, T), dtype=i32, device=dev)
        self.cnt_a = torch.empty((B, s.Hk), dtype=i32, device=dev)
        if B > 1:
            self.perm_q = torch.empty((1, s.Hk, M), dtype=i32, device=dev)
            self.cnt_q = torch.empty((1, s.Hk), dtype=i32, device=dev)
        else:
            self.perm_q, self.cnt_q = self.perm_a, self.cnt_a
        # left padding of each sequence: keys before it are not attended
        self.leftpad = None if leftpad is None else torch.tensor(list(leftpad), dtype=i32, device=dev)
        self.order_a = torch.empty(M, dtype=i32, device=dev)
        self.q = torch.empty((M, s.Hq * s.d), dtype=torch.bfloat16, device=dev)
        self.o = torch.empty((B, T, s.Hq, s.d), dtype=torch.bfloat16, device=dev)
        self.y_attn = torch.empty((M, s.D), dtype=torch.float32, device=dev)
        # One workspace for every GEMM of the step (they run in turn on one stream).
        wsb = max(wsb, mg.gemm_k_workspace_bytes(M, s.D, s.Hq * s.d),
                  mg.gemm_mn_workspace_bytes(M, s.Hq * s.d, s.D, s.G_attn, False))
        self.ws = torch.empty(max(wsb, 16), dtype=torch.uint8, device=dev)

    def _ordered(self, op: str, which: str) -> bool:
        return which == "masked" and op in self.ordered_k

    def _grouped(self, op: str, which: str) -> bool:
        return which == "masked" and op in self.grouped_k

    def _mn_ws(self, op: str, which: str):
        return self.ws if op in self.scheduled_mn.get(which, ()) else None

    def run(self, op: str, which: str = "masked") -> None:
        """Enqueue one op of the step on the current stream; it reads whatever
        the buffers hold (run the ops in `self.ops` order for a layer pass)."""
        s = self.s
        ma, mf = self.masks[which]
        if op == "reorder":
            if self.attn:
                mg.reorder(ma, self.perm_a, self.cnt_a)
                if s.B > 1:
                    mg.reorder(ma.view(1, s.M, s.Hk), self.perm_q, self.cnt_q)
            mg.reorder(mf.view(1, s.M, s.NG_ffn), self.perm_f, self.cnt_f)
            if self._ordered("o_proj", which):
                mg.order_by_pattern(ma.view(s.M, s.Hk), self.order_a)
            if self._ordered("down_proj", which):
                mg.order_by_pattern(mf.view(s.M, s.NG_ffn), self.order_f)
        elif op not in self.ops:
            raise ValueError(f"op {op!r} is not part of this layer")
        elif op == "q_proj":
            mg.gemm_mn(self.x, self.wq, s.G_attn, perm=self.perm_q[0], counts=self.cnt_q[0],
                       out=self.q, workspace=self._mn_ws("q_proj", which))
        elif op == "attention":
            mg.attn(self.q.view(s.B, s.T, s.Hq, s.d), self.k, self.v, perm=self.perm_a,
                    counts=self.cnt_a, out=self.o, leftpad=self.leftpad)
        elif op == "o_proj" and self._grouped("o_proj", which):
            mg.gemm_k_grouped(self.o.view(s.M, s.Hq * s.d), self.wo, s.G_attn, self.perm_q[0], self.cnt_q[0],
                              out=self.y_attn)
        elif op == "o_proj":
            mg.gemm_k(self.o.view(s.M, s.Hq * s.d), self.wo, s.G_attn, ma.view(s.M, s.Hk),
                      out=self.y_attn, workspace=self.ws,
                      order=self.order_a if self._ordered("o_proj", which) else None)
        elif op == "gate_up_swiglu":
            mg.gemm_mn_swiglu(self.x, self.wg, self.wu, s.G_ffn, perm=self.perm_f[0],
                              counts=self.cnt_f[0], out=self.h, workspace=self._mn_ws("gate_up_swiglu", which))
        elif op == "down_proj" and self._grouped("down_proj", which):
            mg.gemm_k_grouped(self.h, self.wd, s.G_ffn, self.perm_f[0], self.cnt_f[0], out=self.y_ffn)
        elif op == "down_proj":
            mg.gemm_k(self.h, self.wd, s.G_ffn, mf.view(s.M, s.NG_ffn), out=self.y_ffn,
                      workspace=self.ws, order=self.order_f if self._ordered("down_proj", which) else None)
        else:
            raise ValueError(f"unknown op {op!r}")

    def step(self, which: str = "masked", events=None) -> None:
        """One pass of the routed path; events[i] / events[i + 1] bracket op i."""
        if events is not None:
            events[0].record()
        for i, op in enumerate(self.ops):
            self.run(op, which)
            if events is not None:
                events[i + 1].record()


class DecodeLayer:
    """Decode step of shape `s`: B sequences with one new token each (B <= 4:
    the matrix-vector kernels read the mask bytes directly), with `sets`
    rotated weight/KV copies."""

    def __init__(self, s, host: dict, sets: int = 1):
        self.s = s
        B = s.B
        d = lambda k: to_device(host[k])  # noqa: E731
        base = {k: d(k) for k in ("w_q", "w_o", "w_gate", "w_up", "w_down", "k", "v")}
        self.wsets = [base] + [{k: t.clone() for k, t in base.items()} for _ in range(sets - 1)]
        self.x = d("x")                                            # [B][D]
        self.ma = d("mask_attn")                                   # [B][1][Hk]
        self.mf = d("mask_ffn").view(B, s.NG_ffn)
        dev = self.x.device
        self.q = torch.empty((B, s.Hq * s.d), dtype=torch.bfloat16, device=dev)
        self.o = torch.empty((B, 1, s.Hq, s.d), dtype=torch.bfloat16, device=dev)
        self.h = torch.empty((B, s.Dff), dtype=torch.bfloat16, device=dev)
        self.y_attn = torch.empty((B, s.D), dtype=torch.float32, device=dev)
        self.y_ffn = torch.empty((B, s.D), dtype=torch.float32, device=dev)
        self.ws = torch.empty(mg.attn_workspace_bytes(B, 1, s.Tkv, s.Hq, s.Hk, s.d),
                              dtype=torch.uint8, device=dev)

    def step(self, i: int = 0, events=None) -> None:
        s = self.s
        B = s.B
        w = self.wsets[i % len(self.wsets)]
        rec = (lambda j: events[j].record()) if events is not None else (lambda j: None)
        rec(0)
        mg.gemm_mn(self.x, w["w_q"], s.G_attn, mask=self.ma.view(B, s.Hk), out=self.q)
        rec(1)
        mg.attn(self.q.view(B, 1, s.Hq, s.d), w["k"], w["v"], mask=self.ma, out=self.o,
                workspace=self.ws)
        rec(2)
        mg.gemm_k(self.o.view(B, s.Hq * s.d), w["w_o"], s.G_attn, self.ma.view(B, s.Hk),
                  out=self.y_attn)
        rec(3)
        mg.gemm_mn_swiglu(self.x, w["w_gate"], w["w_up"], s.G_ffn, mask=self.mf, out=self.h)
        rec(4)
        mg.gemm_k(self.h, w["w_down"], s.G_ffn, self.mf, out=self.y_ffn)
        rec(5)
