"""Sequencing of the library's entry points for one routed-expert MoE FFN layer.

No arithmetic here: each step is one call into libpq on the current stream,
writing into buffers allocated once per shape (so a timed loop allocates
nothing).

Decode (Parakon Runtime README, "How it works"):
    q8(x) -> top-k route -> group by expert -> fused gate/up mat-vec with
    SwiGLU + q8 epilogue -> down mat-vec -> weighted combine.
    For a few tokens the first three are one launch (pq_moe_decode_prep), and
    for a single token the combine is fused into the down mat-vec
    (PQ_EPI_F32_COMBINE; fp32 atomic adds, so the summation order of the
    top-k terms is not fixed).  A single token's whole layer is two launches
    (pq_moe_decode1_gate_up_*, which routes and quantizes by itself, then
    the down mat-vec with the fused combine).
Prefill (same section; dequant-per-tile GEMM for large batches):
    route -> group -> fused gate/up GEMM with SwiGLU epilogue (bf16 h)
    -> down GEMM -> weighted combine.
"""
from __future__ import annotations

import torch

from . import (PQ_EPI_F32, PQ_EPI_F32_COMBINE, PQ_EPI_SWIGLU_BF16, PQ_EPI_SWIGLU_Q8,
               GroupBuffers, Grid1Weights, Sign1Weights, TernaryWeights, decode_prep, decode_prep_supported,
               group_tokens_by_expert, moe_combine, moe_decode1_gate_up, moe_gemm_dequant_tile,
               moe_matvec_grid1, moe_matvec_sign1, moe_matvec_ternary, moe_route_topk, quantize_act_q8,
               tile_layout)

# The decode layer's prep (q8, routing, grouping) goes through
# pq_moe_decode_prep, which takes one launch for a few tokens and two above
# (the q8 and the routing side by side, then the grouping), one launch fewer
# than the separate calls.  The combine is fused into the down mat-vec at one
# token only: launch latency dominates there, while above the fp32 atomic
# adds of the fused combine start to contend.
FUSED_COMBINE_MAX_TOKENS = 1


class DecodeLayer:
    """Buffers and call sequence of one decode MoE FFN layer of fixed shape."""

    def __init__(self, fmt: str, n_tokens: int, hidden: int, inter: int, n_experts: int,
                 top_k: int, device="cuda", fused: bool = None, fused_combine: bool = None,
                 decode1: bool = None):
        self.fmt, self.T, self.H, self.I, self.E, self.k = fmt, n_tokens, hidden, inter, n_experts, top_k
        self.device = device
        if fused is None:
            fused = True
        self.fused = bool(fused) and decode_prep_supported(n_tokens, n_experts, top_k)
        if fused_combine is None:
            fused_combine = n_tokens <= FUSED_COMBINE_MAX_TOKENS
        self.fused_combine = self.fused and bool(fused_combine)
        if decode1 is None:
            decode1 = self.fused_combine
        self.decode1 = bool(decode1) and n_tokens == 1
        A = n_tokens * top_k
        f32, i8 = torch.float32, torch.int8
        self.use_state(self.new_route_state())
        self.hq = torch.empty((A, inter), dtype=i8, device=device)
        self.hd = torch.empty((A, inter // 32), dtype=f32, device=device)
        self.out = torch.empty((A, hidden), dtype=f32, device=device)
        self.y = torch.empty((n_tokens, hidden), dtype=f32, device=device)
        self._mv = {"ternary": moe_matvec_ternary, "grid1": moe_matvec_grid1, "sign1": moe_matvec_sign1}[fmt]

    def new_route_state(self) -> dict:
        """A separate set of q8 / routing / grouping buffers."""
        f32, i8, i32 = torch.float32, torch.int8, torch.int32
        T, dev = self.T, self.device
        return {"xq": torch.empty((T, self.H), dtype=i8, device=dev),
                "xd": torch.empty((T, self.H // 32), dtype=f32, device=dev),
                "ids": torch.empty((T, self.k), dtype=i32, device=dev),
                "w": torch.empty((T, self.k), dtype=f32, device=dev),
                "groups": GroupBuffers.empty(T, self.k, self.E, dev)}

    def use_state(self, st: dict):
        self.xq, self.xd, self.ids, self.w, self.groups = st["xq"], st["xd"], st["ids"], st["w"], st["groups"]

    def route(self, x: torch.Tensor, logits: torch.Tensor):
        if self.fused:
            decode_prep(x, logits, self.k, self.xq, self.xd, self.ids, self.w, self.groups,
                        self.y if self.fused_combine else None)
            return
        quantize_act_q8(x, self.xq, self.xd)
        moe_route_topk(logits, self.k, self.ids, self.w)
        group_tokens_by_expert(self.ids, self.E, self.groups)

    def gate_up(self, gate, up, dbg=None):
        self._mv(gate, up, self.groups, self.xq, self.xd, True, PQ_EPI_SWIGLU_Q8, self.hq, self.hd, dbg)

    def down(self, down, dbg=None):
        if self.fused_combine:
            self._mv(down, None, self.groups, self.hq, self.hd, False, PQ_EPI_F32_COMBINE, self.y, self.w, dbg)
        else:
            self._mv(down, None, self.groups, self.hq, self.hd, False, PQ_EPI_F32, self.out, None, dbg)

    def combine(self):
        if not self.fused_combine:   # else the down mat-vec already accumulated y
            moe_combine(self.out, self.w, self.k, self.y)

    def __call__(self, x, logits, gate, up, down):
        if self.decode1:
            moe_decode1_gate_up(gate, up, x, logits, self.k, self.ids, self.w, self.groups,
                                self.hq, self.hd, self.y)
            self.down(down)
            return self.y
        self.route(x, logits)
        self.gate_up(gate, up)
        self.down(down)
        self.combine()
        return self.y


class PrefillLayer:
    """Buffers and call sequence of one prefill MoE FFN layer (grid1 or sub-scaled
    sign weights in the tile layout, bf16 x)."""

    def __init__(self, n_tokens: int, hidden: int, inter: int, n_experts: int, top_k: int,
                 device="cuda", fused_combine: bool = False):
        self.T, self.H, self.I, self.E, self.k = n_tokens, hidden, inter, n_experts, top_k
        self.device = device
        A = n_tokens * top_k
        self.use_state(self.new_route_state())
        self.h = torch.empty((A, inter), dtype=torch.bfloat16, device=device)
        # fused combine: the down GEMM adds w * out into y (fp32 atomics, the
        # order of a token's top_k additions unspecified); otherwise the
        # per-assignment outputs go through memory and the deterministic
        # slot-order combine.  At 2048 tokens x top-8 the 67M atomic adds
        # cost more than the combine pass they replace (step 1.16 ms against
        # 0.94-1.03 ms measured), so the separate combine is the default.
        self.fused_combine = bool(fused_combine)
        self.out = None if self.fused_combine else torch.empty((A, hidden), dtype=torch.float32, device=device)
        self.y = torch.empty((n_tokens, hidden), dtype=torch.float32, device=device)

    def new_route_state(self) -> dict:
        T, dev = self.T, self.device
        return {"ids": torch.empty((T, self.k), dtype=torch.int32, device=dev),
                "w": torch.empty((T, self.k), dtype=torch.float32, device=dev),
                "groups": GroupBuffers.empty(T, self.k, self.E, dev)}

    def use_state(self, st: dict):
        self.ids, self.w, self.groups = st["ids"], st["w"], st["groups"]

    def route(self, logits):
        moe_route_topk(logits, self.k, self.ids, self.w)
        group_tokens_by_expert(self.ids, self.E, self.groups)

    def gate_up(self, x_bf16, gate, up, dbg=None):
        moe_gemm_dequant_tile(gate, up, self.groups, x_bf16, True, PQ_EPI_SWIGLU_BF16, self.h, dbg)

    def down(self, down, dbg=None):
        if self.fused_combine:
            self.y.zero_()
            moe_gemm_dequant_tile(down, None, self.groups, self.h, False, PQ_EPI_F32_COMBINE, self.y, dbg,
                                  out1=self.w)
        else:
            moe_gemm_dequant_tile(down, None, self.groups, self.h, False, PQ_EPI_F32, self.out, dbg)

    def combine(self):
        if not self.fused_combine:
            moe_combine(self.out, self.w, self.k, self.y)

    def __call__(self, x_bf16, logits, gate, up, down):
        self.route(logits)
        self.gate_up(x_bf16, gate, up)
        self.down(down)
        self.combine()
        return self.y


def weights_to_device(fmt: str, planes: dict, grid=None, device="cuda", tiled: bool = False):
    """Host numpy planes (workloads module layout) -> device weight container;
    `tiled`: code planes in the tile layout of the prefill GEMM (grid1, sign1)."""
    import numpy as np

    def t(a):
        a = np.ascontiguousarray(a)
        if a.dtype == np.uint16:
            a = a.view(np.int16)
        return torch.from_numpy(a).to(device)

    if fmt == "ternary":
        if tiled:
            raise ValueError("ternary weights have no tile layout")
        return TernaryWeights(t(planes["qs"]), t(planes["d"]))
    if fmt == "sign1":
        w = Sign1Weights(t(planes["signs"]), t(planes["sc"]), t(planes["d"]))
    else:
        w = Grid1Weights(t(planes["qs"]), t(planes["qh"]), t(planes["d"]), t(grid))
    return tile_layout(w) if tiled else w
