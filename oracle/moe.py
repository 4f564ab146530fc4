"""MoE FFN compositions of the oracle's steps (TEST INFRASTRUCTURE ONLY).

Decode layer (Parakon Runtime README, "How it works"; pxq_llama README,
"Updates - 2026-07-28" for the fused gate/up + SiLU and "What's PXQ?" for the
grouped MoE path):

    xq, xd = q8(x)                               per 32 along hidden
    ids, w = top-k(logits), softmax over the k   no dropping
    offsets, sorted, active = group(ids)         stable by expert id
    g[a] = W_gate[e] . x[t],  u[a] = W_up[e] . x[t]      a = t*k + j, e = ids[a]
    h[a] = silu(g[a]) * u[a]                     fp64, then rounded to fp32
    hq, hd = q8(h)                               per 32 along intermediate
    out[a] = W_down[e] . h[a]
    y[t] = sum_j w[t][j] * out[t*k + j]

Prefill layer (Parakon Runtime README, "How it works": dequant-per-tile GEMM
for large batches): the same with bf16 activations, no q8 of activations,
h rounded to bf16 (nearest even) before the down projection.

Each stage also has a "staged" form that takes the previous stage's values as
inputs (typically the GPU's), so that a discontinuous step (re-quantization of
h) can be checked bit-exactly on the GPU's own inputs.
"""
from __future__ import annotations

import numpy as np

from . import (combine, float_to_bf16, group, matvec_bf16, matvec_q8, quantize_q8, route_topk, unpack_sign1,
               swiglu, unpack_grid1, unpack_ternary)


def unpack_expert(fmt: str, planes: dict, e: int, K: int, grid=None) -> np.ndarray:
    if fmt == "ternary":
        return unpack_ternary(planes["qs"][e], K)
    if fmt == "grid1":
        return unpack_grid1(planes["qs"][e], planes["qh"][e], grid, K)
    if fmt == "sign1":
        return unpack_sign1(planes["signs"][e], planes["sc"][e], K)
    raise ValueError(fmt)


def expert_scales(fmt: str, planes: dict, e: int, K: int) -> np.ndarray:
    """fp16 bits [N][K/256] of expert e: the per-256-block scales, or for the
    sub-scaled sign format its per-row anchor repeated over the row's blocks."""
    if fmt == "sign1":
        return np.repeat(planes["d"][e][:, None], K // 256, axis=1)
    return planes["d"][e]


def grouped_matvec_q8(fmt, planes, grid, ids, xq_rows, xd_rows, row_of_assign, K,
                      want_isums=True, assign_subset=None, rows_subset=None):
    """out[a] = W[ids[a]] . q8row[row_of_assign[a]] for every assignment a.

    Returns (y f64 [A][N], tsum f64 [A][N], isums i32 [A][N][K/32] or None).
    assign_subset / rows_subset restrict the work (others are left NaN / 0).
    """
    ids = np.asarray(ids).ravel()
    A = ids.size
    N = planes["d"].shape[1]
    sel_rows = np.arange(N) if rows_subset is None else np.asarray(rows_subset)
    y = np.full((A, N), np.nan)
    t = np.full((A, N), np.nan)
    isums = np.zeros((A, N, K // 32), np.int32) if want_isums else None
    assigns = np.arange(A) if assign_subset is None else np.asarray(assign_subset)
    for e in np.unique(ids[assigns]):
        W = unpack_expert(fmt, planes, int(e), K, grid)[sel_rows]
        d16 = expert_scales(fmt, planes, int(e), K)[sel_rows]
        for a in assigns[ids[assigns] == e]:
            r = row_of_assign[a]
            ya, ta, ia = matvec_q8(W, d16, xq_rows[r], xd_rows[r], want_isums)
            y[a, sel_rows] = ya
            t[a, sel_rows] = ta
            if want_isums:
                isums[a, sel_rows] = ia
    return y, t, isums


def grouped_matvec_bf16(fmt, planes, grid, ids, x_rows_bf16, row_of_assign, K,
                        assign_subset=None, rows_subset=None):
    ids = np.asarray(ids).ravel()
    A = ids.size
    N = planes["d"].shape[1]
    sel_rows = np.arange(N) if rows_subset is None else np.asarray(rows_subset)
    y = np.full((A, N), np.nan)
    t = np.full((A, N), np.nan)
    assigns = np.arange(A) if assign_subset is None else np.asarray(assign_subset)
    for e in np.unique(ids[assigns]):
        W = unpack_expert(fmt, planes, int(e), K, grid)[sel_rows]
        d16 = expert_scales(fmt, planes, int(e), K)[sel_rows]
        for a in assigns[ids[assigns] == e]:
            ya, ta = matvec_bf16(W, d16, x_rows_bf16[row_of_assign[a]])
            y[a, sel_rows] = ya
            t[a, sel_rows] = ta
    return y, t


def decode_ffn(inp: dict, want_isums: bool = True, assign_subset=None) -> dict:
    """Free-running oracle chain of one decode MoE FFN layer.

    assign_subset restricts the expert work to those assignments (rows of the
    others are left NaN / 0) and skips the combine (y is None)."""
    cfg = inp["cfg"]
    fmt, k, H, I, E = cfg["fmt"], cfg["top_k"], cfg["H"], cfg["I"], cfg["E"]
    grid = inp.get("grid")
    r = {}
    r["xq"], r["xd"] = quantize_q8(inp["x"])
    r["ids"], r["w"] = route_topk(inp["logits"], k)
    r["offsets"], r["sorted"], r["active"] = group(r["ids"], E)
    A = r["ids"].size
    tok = np.arange(A) // k
    sub = assign_subset
    r["g"], r["tg"], r["isum_g"] = grouped_matvec_q8(fmt, inp["gate"], grid, r["ids"], r["xq"], r["xd"], tok, H,
                                                     want_isums, assign_subset=sub)
    r["u"], r["tu"], r["isum_u"] = grouped_matvec_q8(fmt, inp["up"], grid, r["ids"], r["xq"], r["xd"], tok, H,
                                                     want_isums, assign_subset=sub)
    if sub is None:
        h64 = swiglu(r["g"].astype(np.float32), r["u"].astype(np.float32))
        r["hq"], r["hd"] = quantize_q8(h64.astype(np.float32))
    else:
        sub = np.asarray(sub)
        h64 = np.full((A, I), np.nan)
        h64[sub] = swiglu(r["g"][sub].astype(np.float32), r["u"][sub].astype(np.float32))
        r["hq"] = np.zeros((A, I), np.int8)
        r["hd"] = np.zeros((A, I // 32), np.float32)
        r["hq"][sub], r["hd"][sub] = quantize_q8(h64[sub].astype(np.float32))
    r["h"] = h64
    r["out"], r["tout"], r["isum_d"] = grouped_matvec_q8(fmt, inp["down"], grid, r["ids"], r["hq"], r["hd"],
                                                         np.arange(A), I, want_isums, assign_subset=sub)
    if sub is None:
        r["y"], r["ty"] = combine(r["out"].astype(np.float32), r["w"].astype(np.float32), k)
    else:
        r["y"], r["ty"] = None, None
    return r


def tol_ok(got, ref, tsum, rel=1e-5, abs_=1e-6):
    """Elementwise |got - ref| <= rel * tsum + abs_  (the path's fp32 tolerance)."""
    got = np.asarray(got, np.float64)
    return np.abs(got - ref) <= rel * np.asarray(tsum) + abs_


def prefill_ffn(inp: dict, assign_subset=None) -> dict:
    """Free-running oracle chain of one prefill MoE FFN layer (grid1 or
    sub-scaled sign weights, bf16 x), ending in the weighted combine y.

    assign_subset restricts the expert work to those assignments (the other
    rows of g, u, h, out stay NaN) and skips the combine (y is None)."""
    cfg = inp["cfg"]
    fmt, k, H, I, E = cfg["fmt"], cfg["top_k"], cfg["H"], cfg["I"], cfg["E"]
    grid = inp.get("grid")
    r = {}
    r["ids"], r["w"] = route_topk(inp["logits"], k)
    r["offsets"], r["sorted"], r["active"] = group(r["ids"], E)
    A = r["ids"].size
    tok = np.arange(A) // k
    r["g"], r["tg"] = grouped_matvec_bf16(fmt, inp["gate"], grid, r["ids"], inp["x_bf16"], tok, H, assign_subset)
    r["u"], r["tu"] = grouped_matvec_bf16(fmt, inp["up"], grid, r["ids"], inp["x_bf16"], tok, H, assign_subset)
    rows = np.arange(A) if assign_subset is None else np.asarray(assign_subset)
    h = np.full((A, I), np.nan)
    h[rows] = swiglu(r["g"][rows].astype(np.float32), r["u"][rows].astype(np.float32))
    r["h"] = h
    hb = np.zeros((A, I), np.uint16)
    hb[rows] = float_to_bf16(h[rows].astype(np.float32)).reshape(len(rows), I)
    r["h_bf16"] = hb
    r["out"], r["tout"] = grouped_matvec_bf16(fmt, inp["down"], grid, r["ids"], hb, np.arange(A), I, assign_subset)
    if assign_subset is None:
        r["y"], r["ty"] = combine(r["out"].astype(np.float32), r["w"].astype(np.float32), k)
    else:
        r["y"], r["ty"] = None, None
    return r
