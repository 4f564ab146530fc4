"""GPU parity of the decode path (HIP kernels through the C ABI) against the CPU oracle.

Bar: q8 codes/scales, routing ids, grouping and every int32 block sum
bit-exact; fp32 outputs within |got - ref| <= 1e-5 * sum|terms| + 1e-6.
The SwiGLU re-quantization is checked on the GPU's own fp32 h (bit-exact),
because q8 is discontinuous; the free-running chain is checked where no
near-tie flipped a q8 value.
"""
import ctypes
import zlib

import numpy as np
import pytest
import torch

import bit_quantized_moe_q8_amd as pq
from bit_quantized_moe_q8_amd.layer import DecodeLayer, weights_to_device
import oracle
from oracle import moe
import workloads as wl

from gpu_util import (assert_equal, assert_plan, assert_tol, dev, decode_inputs, q8h_check, say, to_dev,
                      to_host)

pytestmark = pytest.mark.gpu


# ------------------------------------------------------------------- q8

@pytest.mark.parametrize("rows,cols,seed", [(1, 1024, 1), (8, 4096, 2), (64, 2048, 3), (3, 32, 4), (513, 768, 5)])
def test_q8_bit_exact(rows, cols, seed):
    say("q8", rows, cols, seed)
    x = wl.activations_f32(seed, rows, cols)
    xq, xd = pq.quantize_act_q8(to_dev(x))
    q_ref, d_ref = oracle.quantize_q8(x)
    assert_equal(to_host(xq), q_ref, "xq")
    assert_equal(to_host(xd), d_ref, "xd")


def test_q8_edge_blocks():
    say("q8 edge blocks")
    x = np.zeros((1, 32 * 8), np.float32)
    x[0, 0:12] = [127.0, 2.5, -2.5, 0.5, -0.5, 1.5, -0.49, 126.5, -126.5, 0.0, 3.0, -1.0]
    # block 1: all zero; block 2: tiny values; block 3: max shared by two elements
    x[0, 64:96] = np.linspace(-1e-30, 1e-30, 32, dtype=np.float32)
    x[0, 96:128] = 0.25
    x[0, 97] = -3.0
    x[0, 100] = 3.0
    x[0, 128:160] = np.float32(1e30) * np.linspace(-1, 1, 32, dtype=np.float32)
    x[0, 160:192] = np.arange(32, dtype=np.float32) - 15.5
    x[0, 192:256] = wl.activations_f32(9, 1, 64)
    xq, xd = pq.quantize_act_q8(to_dev(x))
    q_ref, d_ref = oracle.quantize_q8(x)
    assert_equal(to_host(xq), q_ref, "xq")
    assert_equal(to_host(xd), d_ref, "xd")


def test_q8_subnormal_blocks():
    say("q8 subnormal blocks")
    x = np.zeros((1, 96), np.float32)
    x[0, 0:32] = np.float32(1e-40) * np.linspace(-1, 1, 32, dtype=np.float32)
    x[0, 32:64] = np.float32(3e-39) * np.linspace(-1, 1, 32, dtype=np.float32)
    x[0, 64:96] = np.float32(1.5e-36) * (np.arange(32, dtype=np.float32) - 16)
    xq, xd = pq.quantize_act_q8(to_dev(x))
    q_ref, d_ref = oracle.quantize_q8(x)
    assert_equal(to_host(xq), q_ref, "xq")
    assert_equal(to_host(xd), d_ref, "xd")


# ---------------------------------------------------------------- routing

@pytest.mark.parametrize("T,E,k,kind", [(1, 128, 8, "normal"), (8, 256, 8, "uniform"), (64, 256, 8, "zipf"),
                                        (2048, 256, 8, "uniform"), (5, 1024, 16, "normal"), (3, 7, 7, "normal"),
                                        (9, 64, 1, "normal")])
def test_route_topk(T, E, k, kind):
    say("route", T, E, k, kind)
    logits = wl.router_logits(41, T, E, kind)
    ids, w = pq.moe_route_topk(to_dev(logits), k)
    ids_ref, w_ref = oracle.route_topk(logits, k)
    assert_equal(to_host(ids), ids_ref, "ids")
    assert_tol(to_host(w), w_ref, w_ref, "w")


def test_route_ties():
    say("route ties")
    l = np.zeros((3, 96), np.float32)
    l[1, [5, 70, 71, 90]] = 2.0
    l[2] = np.repeat(np.float32([1.0, 2.0, 3.0]), 32)
    ids, w = pq.moe_route_topk(to_dev(l), 8)
    ids_ref, w_ref = oracle.route_topk(l, 8)
    assert_equal(to_host(ids), ids_ref, "ids")
    assert_tol(to_host(w), w_ref, w_ref, "w")


# --------------------------------------------------------------- grouping

@pytest.mark.parametrize("T,E,k,kind", [(1, 128, 8, "normal"), (8, 256, 8, "uniform"), (64, 256, 8, "zipf"),
                                        (2048, 256, 8, "uniform"), (1000, 1024, 16, "normal"), (1, 1, 1, "normal")])
def test_group_bit_exact(T, E, k, kind):
    say("group", T, E, k, kind)
    ids, _ = oracle.route_topk(wl.router_logits(42, T, E, kind), k)
    g = pq.group_tokens_by_expert(to_dev(ids), E)
    off, srt, act = oracle.group(ids, E)
    assert_equal(to_host(g.expert_offsets), off, "offsets")
    assert_equal(to_host(g.sorted_assign)[: ids.size], srt, "sorted")
    assert int(to_host(g.n_active)[0]) == act.size
    assert_equal(to_host(g.active_experts)[: act.size], act, "active")


def test_group_all_to_one_expert_and_twice_identical():
    say("group skewed")
    E = 64
    ids = np.full((4096, 4), 17, np.int32)
    ids[::7, 2] = 3
    ids[5, 0] = 63
    g1 = pq.group_tokens_by_expert(to_dev(ids), E)
    g2 = pq.group_tokens_by_expert(to_dev(ids), E)
    off, srt, act = oracle.group(ids, E)
    for g in (g1, g2):
        assert_equal(to_host(g.expert_offsets), off, "offsets")
        assert_equal(to_host(g.sorted_assign), srt, "sorted")
        assert_equal(to_host(g.active_experts)[: act.size], act, "active")


# ------------------------------------------------------- single mat-vecs

def _single(fmt, E, N, K, T, k, act_by_token, seed, want_dbg=True, ids=None):
    """Grouped F32 mat-vec on random routing; compare isums exactly and y within tolerance.
    Without debug outputs the production kernels run (at one token: the
    one-token kernel)."""
    rng = np.random.default_rng(seed)
    if ids is None:
        ids = np.stack([rng.choice(E, size=k, replace=False) for _ in range(T)]).astype(np.int32)
    planes = wl.stack_experts(fmt, seed, "w", E, N, K)
    grid = wl.codebook(seed) if fmt == "grid1" else None
    n_rows = T if act_by_token else T * k
    xq, xd = oracle.quantize_q8(wl.activations_f32(seed, n_rows, K))
    g = pq.group_tokens_by_expert(to_dev(ids), E)
    W = weights_to_device(fmt, planes, grid)
    A = T * k
    isums = torch.zeros((A, N, K // 32), dtype=torch.int32, device=dev()) if want_dbg else None
    mv = {"ternary": pq.moe_matvec_ternary, "grid1": pq.moe_matvec_grid1, "sign1": pq.moe_matvec_sign1}[fmt]
    out, _ = mv(W, None, g, to_dev(xq), to_dev(xd), act_by_token, pq.PQ_EPI_F32,
                dbg={"isums": isums} if want_dbg else None)
    rows_of = (np.arange(A) // k) if act_by_token else np.arange(A)
    y_ref, t_ref, i_ref = moe.grouped_matvec_q8(fmt, planes, grid, ids, xq, xd, rows_of, K, want_dbg)
    if want_dbg:
        assert_equal(to_host(isums), i_ref, "isums")
    assert_tol(to_host(out), y_ref, t_ref, "y")
    return to_host(out)


def test_ternary_matvec_1024_single_matrix():
    """One 1024x1024 ternary matrix, one token: E=1, T=1, k=1."""
    say("ternary 1024x1024 single")
    inp = wl.make_workload("ternary_matvec_1024")
    planes = inp["w"]
    xq_d, xd_d = pq.quantize_act_q8(to_dev(inp["x"]))
    xq, xd = oracle.quantize_q8(inp["x"])
    assert_equal(to_host(xq_d), xq, "xq")
    assert_equal(to_host(xd_d), xd, "xd")
    g = pq.group_tokens_by_expert(to_dev(np.zeros((1, 1), np.int32)), 1)
    isums = torch.zeros((1, 1024, 32), dtype=torch.int32, device=dev())
    W = weights_to_device("ternary", planes)
    assert_plan(pq.PQ_PLAN_MATVEC | pq.PQ_PLAN_DEBUG, pq.PQ_CALL_MATVEC, "ternary", 1, 1, 1, 1024, 1024, debug=True)
    assert_plan(pq.PQ_PLAN_MATVEC_TOK1, pq.PQ_CALL_MATVEC, "ternary", 1, 1, 1, 1024, 1024)
    out, _ = pq.moe_matvec_ternary(W, None, g, xq_d, xd_d, True, pq.PQ_EPI_F32, dbg={"isums": isums})
    w = oracle.unpack_ternary(planes["qs"][0], 1024)
    y_ref, t_ref, i_ref = oracle.matvec_q8(w, planes["d"][0], xq[0], xd[0])
    assert_equal(to_host(isums)[0], i_ref, "isums")
    assert_tol(to_host(out)[0], y_ref, t_ref, "y")
    # the production variant (no debug outputs) gives the same bits
    out2, _ = pq.moe_matvec_ternary(W, None, g, xq_d, xd_d, True, pq.PQ_EPI_F32)
    assert_equal(to_host(out2), to_host(out), "debug vs production variant")


@pytest.mark.parametrize("fmt,E,N,K,expert", [
    ("ternary", 1, 1024, 1024, 0),    # the single-matrix workload's shape
    ("ternary", 3, 100, 256, 2),      # smallest K, ragged rows
    ("ternary", 2, 72, 2048, 1),      # K split over four wave groups
    ("ternary", 2, 40, 4096, 0),      # the widest ternary row
    ("ternary", 2, 33, 768, 1),       # 12 lanes per row
    ("grid1", 2, 64, 4096, 1),
    ("grid1", 1, 40, 1536, 0),
    ("grid1", 1, 16, 8192, 0),        # the widest grid1 row
    ("sign1", 2, 72, 2048, 1),
    ("sign1", 1, 40, 6144, 0),
])
def test_matvec_x32_single_launch(fmt, E, N, K, expert):
    """pq_matvec_x32_*: one launch that quantizes the fp32 row itself; y
    bit-identical to pq_quantize_act_q8 + the one-token mat-vec of the same
    expert, and within the stated bound of the oracle (q8 by the oracle's
    rule, then the q8 mat-vec)."""
    say("matvec x32", fmt, E, N, K, expert)
    seed = zlib.crc32(repr((fmt, E, N, K)).encode()) % 1000
    planes = wl.stack_experts(fmt, seed, "w", E, N, K)
    grid = wl.codebook(seed) if fmt == "grid1" else None
    x = wl.activations_f32(seed, 1, K)
    W = weights_to_device(fmt, planes, grid)
    xd_dev = to_dev(x)
    y = pq.matvec_x32(W, xd_dev.view(-1), expert)
    # the two-launch pair: q8, then the one-token kernel for one token routed to `expert`
    xq_d, xdd = pq.quantize_act_q8(xd_dev)
    g = pq.group_tokens_by_expert(to_dev(np.full((1, 1), expert, np.int32)), E)
    mv = {"ternary": pq.moe_matvec_ternary, "grid1": pq.moe_matvec_grid1, "sign1": pq.moe_matvec_sign1}[fmt]
    out, _ = mv(W, None, g, xq_d, xdd, True, pq.PQ_EPI_F32)
    torch.cuda.synchronize()
    assert_equal(to_host(y), to_host(out)[0], "single launch vs q8 + mat-vec")
    xq, xd = oracle.quantize_q8(x)
    y_ref, t_ref, _ = moe.grouped_matvec_q8(fmt, planes, grid, np.full((1, 1), expert, np.int32), xq, xd,
                                            np.zeros(1, np.int64), K, False)
    assert_tol(to_host(y), y_ref[0], t_ref[0], "y")
    # a second call into the same output gives the same bits
    y2 = pq.matvec_x32(W, xd_dev.view(-1), expert, y=torch.full_like(y, 7.0))
    assert_equal(to_host(y2), to_host(y), "repeat")


@pytest.mark.parametrize("fmt,E,N,K,T,k,abt", [
    ("ternary", 4, 96, 256, 1, 2, True),      # smallest K, ragged rows (3 tiles)
    ("ternary", 8, 100, 768, 3, 2, True),     # 12 lanes per row, ragged tail tile
    ("ternary", 8, 64, 1024, 5, 3, False),    # activation row per assignment
    ("ternary", 16, 70, 2048, 9, 4, True),    # 4 tokens per pass, ragged
    ("ternary", 3, 33, 4096, 2, 3, True),     # 64 lanes per row
    ("grid1", 4, 96, 256, 1, 2, True),
    ("grid1", 8, 40, 1536, 3, 2, False),
    ("grid1", 8, 64, 1024, 6, 3, True),
    ("grid1", 16, 50, 4096, 9, 4, True),
    ("ternary", 8, 40, 1536, 3, 2, True),     # 24 chunks per row
    ("ternary", 4, 33, 3072, 2, 2, False),    # 48 chunks per row
    ("grid1", 8, 40, 3072, 3, 2, True),       # 24 chunks per row
    ("grid1", 4, 20, 6144, 2, 2, False),      # 48 chunks per row
    ("sign1", 4, 96, 256, 1, 2, True),        # sub-scaled signs: 2 lanes per row
    ("sign1", 8, 40, 1536, 3, 2, False),
    ("sign1", 16, 50, 4096, 9, 4, True),      # pairs of assignments per pass
    ("sign1", 8, 64, 1024, 40, 3, True),      # split groups of assignments
    ("sign1", 4, 20, 6144, 2, 2, False),      # 48 chunks per row
    ("sign1", 2, 16, 8192, 3, 2, True),       # 64 chunks per row (the widest)
    ("sign1", 1024, 40, 512, 20, 8, True),    # 1024 experts (the limit)
])
def test_grouped_matvec(fmt, E, N, K, T, k, abt):
    say("matvec", fmt, E, N, K, T, k, abt)
    _single(fmt, E, N, K, T, k, abt, seed=zlib.crc32(repr((fmt, E, N, K, T)).encode()) % 1000)


def test_matvec_one_expert_many_tokens():
    """All tokens on one expert (many passes of the token loop)."""
    say("matvec one expert")
    for fmt in ("ternary", "grid1"):
        _single(fmt, 1, 64, 1024, 37, 1, True, seed=7)


@pytest.mark.parametrize("fmt,K,k,abt", [
    ("ternary", 256, 8, True),     # 4 lanes per row
    ("ternary", 768, 8, False),    # 12 lanes per row (down projection shape)
    ("ternary", 2048, 8, True),    # 32 lanes per row (gate/up shape)
    ("ternary", 4096, 2, False),   # 64 lanes per row
    ("ternary", 512, 1, True),
    ("grid1", 256, 4, True),       # 2 lanes per row
    ("grid1", 1536, 8, False),
    ("grid1", 4096, 8, True),
    ("ternary", 1536, 8, True),    # 24 lanes per row
    ("grid1", 3072, 4, False),
    ("grid1", 6144, 2, True),      # 48 lanes per row
    ("sign1", 2048, 8, True),
    ("sign1", 1536, 8, False),     # 12 lanes per row
    ("sign1", 256, 4, True),       # 2 lanes per row
    ("sign1", 6144, 2, False),     # 48 lanes per row
    ("sign1", 8192, 1, True),      # 64 lanes per row
])
def test_matvec_one_token(fmt, K, k, abt):
    """The one-token production kernel (no debug outputs), ragged row tiles."""
    say("matvec one token", fmt, K, k, abt)
    assert_plan(pq.PQ_PLAN_MATVEC_TOK1, pq.PQ_CALL_MATVEC, fmt, 1, k, 16, 72, K)
    _single(fmt, 16, 72, K, 1, k, abt, seed=K + k, want_dbg=False)


@pytest.mark.parametrize("fmt", ["ternary", "grid1", "sign1"])
def test_matvec_one_token_repeated_ids(fmt):
    """One token whose top-k list repeats an expert (fewer active experts than
    assignments): every epilogue of the one-token kernel against the oracle."""
    say("matvec one token repeated ids", fmt)
    E, N, K, k = 8, 256, 512, 5
    ids = np.array([[5, 5, 2, 7, 5]], np.int32)
    for abt in (True, False):
        _single(fmt, E, N, K, 1, k, abt, seed=11, want_dbg=False, ids=ids)
    grid = wl.codebook(3) if fmt == "grid1" else None
    gate = wl.stack_experts(fmt, 3, "gate", E, N, K)
    up = wl.stack_experts(fmt, 3, "up", E, N, K)
    xq, xd = oracle.quantize_q8(wl.activations_f32(3, 1, K))
    g = pq.group_tokens_by_expert(to_dev(ids), E)
    mv = {"ternary": pq.moe_matvec_ternary, "grid1": pq.moe_matvec_grid1, "sign1": pq.moe_matvec_sign1}[fmt]
    hq, hd = mv(weights_to_device(fmt, gate, grid), weights_to_device(fmt, up, grid), g,
                to_dev(xq), to_dev(xd), True, pq.PQ_EPI_SWIGLU_Q8)
    tok = np.zeros(k, np.int64)
    g_ref, tg, _ = moe.grouped_matvec_q8(fmt, gate, grid, ids, xq, xd, tok, K, False)
    u_ref, tu, _ = moe.grouped_matvec_q8(fmt, up, grid, ids, xq, xd, tok, K, False)
    hq_g, hd_g = to_host(hq), to_host(hd)
    q8h_check(hq_g, hd_g, g_ref, u_ref, tg, tu)
    # the repeated assignments (slots 0, 1, 4 of expert 5) are identical
    assert_equal(hq_g[1], hq_g[0], "repeat hq")
    assert_equal(hq_g[4], hq_g[0], "repeat hq")
    # down projection with the fused combine, activation row per assignment
    down = wl.stack_experts(fmt, 3, "down", E, K, N)
    w = np.array([[0.4, 0.1, 0.2, 0.2, 0.1]], np.float32)
    y = torch.zeros((1, K), device=dev())
    mv(weights_to_device(fmt, down, grid), None, g, hq, hd, False, pq.PQ_EPI_F32_COMBINE,
       out0=y, out1=to_dev(w))
    o_ref, to, _ = moe.grouped_matvec_q8(fmt, down, grid, ids, hq_g, hd_g, np.arange(k), N, False)
    y_ref, ty = oracle.combine(o_ref.astype(np.float32), w, k)
    ty_d = np.abs(w.astype(np.float64)) @ to
    assert_tol(to_host(y), y_ref, ty + ty_d, "y")


# ----------------------------------------------------------- decode layers

def _run_layer(name, fused=False, **override):
    inp = decode_inputs(name, **override)
    cfg = inp["cfg"]
    fmt, T, H, I, E, k = cfg["fmt"], cfg["T"], cfg["H"], cfg["I"], cfg["E"], cfg["top_k"]
    A = T * k
    layer = DecodeLayer(fmt, T, H, I, E, k, dev(), fused=fused, fused_combine=fused)
    assert layer.fused == fused and layer.fused_combine == fused
    # the staged check runs the debug variants; the production run after it
    # (whose hq and y must repeat) takes the production kernels
    for debug in (True, False):
        gu = pq.plan(pq.PQ_CALL_MATVEC, fmt, T, k, E, I, H, pq.PQ_EPI_SWIGLU_Q8, debug)
        dn = pq.plan(pq.PQ_CALL_MATVEC, fmt, T, k, E, H, I, pq.PQ_EPI_F32, debug)
        assert gu > 0 and dn > 0 and bool(gu & pq.PQ_PLAN_DEBUG) == debug
        if T == 1 and not debug:
            assert dn == pq.PQ_PLAN_MATVEC_TOK1
    if layer.decode1:
        assert_plan(pq.PQ_PLAN_DECODE1_ROUTED, pq.PQ_CALL_DECODE1_GATE_UP, fmt, T, k, E, I, H, pq.PQ_EPI_SWIGLU_Q8)
    grid = inp.get("grid")
    W = {n: weights_to_device(fmt, inp[n], grid) for n in ("gate", "up", "down")}
    x, logits = to_dev(inp["x"]), to_dev(inp["logits"])
    dbg1 = {"isums": torch.zeros((A, I, H // 32), dtype=torch.int32, device=dev()),
            "isums_up": torch.zeros((A, I, H // 32), dtype=torch.int32, device=dev()),
            "g": torch.zeros((A, I), device=dev()), "u": torch.zeros((A, I), device=dev()),
            "h": torch.zeros((A, I), device=dev())}
    dbg2 = {"isums": torch.zeros((A, H, I // 32), dtype=torch.int32, device=dev())}
    layer.route(x, logits)
    layer.gate_up(W["gate"], W["up"], dbg1)
    layer.down(W["down"], dbg2)
    layer.combine()
    torch.cuda.synchronize()
    gpu = {k2: to_host(v) for k2, v in dict(xq=layer.xq, xd=layer.xd, ids=layer.ids, w=layer.w,
                                            hq=layer.hq, hd=layer.hd, out=layer.out, y=layer.y).items()}
    gpu.update({"dbg_" + k2: to_host(v) for k2, v in dbg1.items()})
    gpu["dbg_isum_d"] = to_host(dbg2["isums"])
    gpu["offsets"] = to_host(layer.groups.expert_offsets)
    gpu["sorted"] = to_host(layer.groups.sorted_assign)[:A]
    # second production run: integer and fp outputs must repeat bit for bit
    layer(x, logits, W["gate"], W["up"], W["down"])
    torch.cuda.synchronize()
    gpu["hq2"], gpu["y2"] = to_host(layer.hq), to_host(layer.y)
    gpu["fused"] = fused
    return inp, gpu


def _check_layer(inp, gpu):
    cfg = inp["cfg"]
    fmt, T, H, I, E, k = cfg["fmt"], cfg["T"], cfg["H"], cfg["I"], cfg["E"], cfg["top_k"]
    A = T * k
    grid = inp.get("grid")
    # stage 1: q8(x), routing, grouping
    xq, xd = oracle.quantize_q8(inp["x"])
    assert_equal(gpu["xq"], xq, "xq")
    assert_equal(gpu["xd"], xd, "xd")
    ids, w = oracle.route_topk(inp["logits"], k)
    assert_equal(gpu["ids"], ids, "ids")
    assert_tol(gpu["w"], w, w, "w")
    off, srt, _ = oracle.group(ids, E)
    assert_equal(gpu["offsets"], off, "offsets")
    assert_equal(gpu["sorted"], srt, "sorted")
    # stage 2: gate/up block sums and outputs
    tok = np.arange(A) // k
    g_ref, tg, ig = moe.grouped_matvec_q8(fmt, inp["gate"], grid, ids, xq, xd, tok, H)
    u_ref, tu, iu = moe.grouped_matvec_q8(fmt, inp["up"], grid, ids, xq, xd, tok, H)
    assert_equal(gpu["dbg_isums"], ig, "gate isums")
    assert_equal(gpu["dbg_isums_up"], iu, "up isums")
    assert_tol(gpu["dbg_g"], g_ref, tg, "g")
    assert_tol(gpu["dbg_u"], u_ref, tu, "u")
    # stage 3: h from the GPU's own g, u; q8 of the GPU's own h bit-exact
    h_ref = oracle.swiglu(gpu["dbg_g"], gpu["dbg_u"])
    assert_tol(gpu["dbg_h"], h_ref, np.abs(h_ref), "h")
    hq_ref, hd_ref = oracle.quantize_q8(gpu["dbg_h"])
    assert_equal(gpu["hq"], hq_ref, "hq")
    assert_equal(gpu["hd"], hd_ref, "hd")
    # stage 4: down on the GPU's own hq/hd
    o_ref, to, io = moe.grouped_matvec_q8(fmt, inp["down"], grid, ids, gpu["hq"], gpu["hd"], np.arange(A), I)
    assert_equal(gpu["dbg_isum_d"], io, "down isums")
    ty_down = np.einsum("tj,tjn->tn", np.abs(gpu["w"].astype(np.float64)), to.reshape(T, k, H))
    if gpu["fused"]:
        # stage 5 fused into the down mat-vec: y against the oracle's combine
        # of the oracle's down outputs (the bound adds the weighted term sums)
        y_ref, ty = oracle.combine(o_ref.astype(np.float32), gpu["w"], k)
        assert_tol(gpu["y"], y_ref, ty + ty_down, "y (fused combine)")
        assert_equal(gpu["hq2"], gpu["hq"], "hq repeat")
        assert_tol(gpu["y2"], y_ref, ty + ty_down, "y repeat (fused combine)")
    else:
        assert_tol(gpu["out"], o_ref, to, "out")
        # stage 5: combine on the GPU's own out and w
        y_ref, ty = oracle.combine(gpu["out"], gpu["w"], k)
        assert_tol(gpu["y"], y_ref, ty, "y (staged)")
        # repeat run is bitwise identical
        assert_equal(gpu["hq2"], gpu["hq"], "hq repeat")
        assert_equal(gpu["y2"], gpu["y"], "y repeat")
    # free-running oracle chain: q8(h) within the bound derived from the
    # tolerance of g and u; tokens whose q8 h rows all agree must match y
    ref = moe.decode_ffn(inp, want_isums=False)
    same = (ref["hq"] == gpu["hq"]).reshape(T, k, I).all(axis=(1, 2))
    flips = q8h_check(gpu["hq"], gpu["hd"], ref["g"], ref["u"], ref["tg"], ref["tu"], "free-running q8(h)")
    say("  free-running q8(h) flips at rounding boundaries: %d of %d" % (flips, ref["hq"].size))
    ty_free = np.einsum("tj,tjn->tn", np.abs(ref["w"]), ref["tout"].reshape(T, k, H))
    assert_tol(gpu["y"][same], ref["y"][same], ty_free[same], "y (free-running)")


@pytest.mark.parametrize("name,override,fused", [
    ("ternary_moe_decode_t1", {}, False),
    ("ternary_moe_decode_t1", {}, True),
    ("grid1_moe_decode_t8", {}, False),
    ("grid1_moe_decode_t8", {}, True),
    ("ternary_moe_decode_t64_zipf", {}, False),
    ("ternary_moe_decode_t1", dict(T=4, E=16, H=768, I=256, top_k=4), False),
    ("ternary_moe_decode_t1", dict(T=4, E=16, H=768, I=256, top_k=4), True),
    ("grid1_moe_decode_t8", dict(T=3, E=8, H=1024, I=512, top_k=2), False),
    ("grid1_moe_decode_t8", dict(T=16, E=256, H=1024, I=256, top_k=16), True),
    ("sign1_moe_decode_t8", {}, False),
    ("sign1_moe_decode_t8", dict(T=1, E=64, H=2048, I=1536, top_k=8), True),
    ("sign1_moe_decode_t8", dict(T=48, E=16, H=1024, I=512, top_k=4), False),
])
def test_decode_layer(name, override, fused):
    say("decode layer", name, override, "fused" if fused else "separate")
    inp, gpu = _run_layer(name, fused, **override)
    _check_layer(inp, gpu)


@pytest.mark.parametrize("name,override", [("ternary_moe_decode_t1", {}),
                                           ("sign1_moe_decode_t8", dict(T=1, E=64, H=2048, I=1536, top_k=8))])
def test_one_token_layer_in_captured_graph(name, override):
    """The one-token layer (two launches: routed gate/up, down with the fused
    combine) captured in a graph and replayed three times, with eager steps
    on other inputs between the replays: routing, q8(h) and y of every replay
    match the oracle (y within tolerance: the fused combine adds the top-k
    terms with atomics, so its last bits can differ between runs)."""
    say("one-token layer in graph", name)
    inp = decode_inputs(name, **override)
    cfg = inp["cfg"]
    fmt, T, H, I, E, k = cfg["fmt"], cfg["T"], cfg["H"], cfg["I"], cfg["E"], cfg["top_k"]
    layer = DecodeLayer(fmt, T, H, I, E, k, dev())
    assert layer.decode1
    W = {n: weights_to_device(fmt, inp[n], inp.get("grid")) for n in ("gate", "up", "down")}
    x, logits = to_dev(inp["x"]), to_dev(inp["logits"])
    other_x = to_dev(wl.activations_f32(77, T, H))
    other_lg = to_dev(wl.router_logits(77, T, E, "normal"))
    ref = moe.decode_ffn(inp, want_isums=False)
    layer(x, logits, W["gate"], W["up"], W["down"])
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        layer(x, logits, W["gate"], W["up"], W["down"])
    for rep in range(3):
        layer(other_x, other_lg, W["gate"], W["up"], W["down"])   # eager step on other inputs
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        assert_equal(to_host(layer.ids), ref["ids"], "ids (replay %d)" % rep)
        hq, hd = to_host(layer.hq), to_host(layer.hd)
        q8h_check(hq, hd, ref["g"], ref["u"], ref["tg"], ref["tu"], "q8(h) (replay %d)" % rep)
        o_ref, to, _ = moe.grouped_matvec_q8(fmt, inp["down"], inp.get("grid"), ref["ids"], hq, hd,
                                             np.arange(T * k), I, want_isums=False)
        w = to_host(layer.w)
        y_ref, ty = oracle.combine(o_ref.astype(np.float32), w, k)
        ty = ty + np.einsum("tj,tjn->tn", np.abs(w.astype(np.float64)), to.reshape(T, k, H))
        assert_tol(to_host(layer.y), y_ref, ty, "y (replay %d)" % rep)


def _prep_case(T, E, H, k, logits=None, seed=0):
    rng = np.random.default_rng(seed)
    x = rng.standard_normal((T, H)).astype(np.float32)
    x[:, :32] = 0.0                              # an all-zero q8 block
    if logits is None:
        logits = rng.standard_normal((T, E)).astype(np.float32)
    xd_, ld = to_dev(x), to_dev(logits)
    sep = {}
    sep["xq"], sep["xd"] = pq.quantize_act_q8(xd_)
    sep["ids"], sep["w"] = pq.moe_route_topk(ld, k)
    g = pq.group_tokens_by_expert(sep["ids"], E)
    fz = pq.GroupBuffers.empty(T, k, E, dev())
    f = {"xq": torch.empty((T, H), dtype=torch.int8, device=dev()),
         "xd": torch.empty((T, H // 32), dtype=torch.float32, device=dev()),
         "ids": torch.empty((T, k), dtype=torch.int32, device=dev()),
         "w": torch.empty((T, k), dtype=torch.float32, device=dev())}
    y = torch.full((T, H), 7.0, device=dev())
    pq.decode_prep(xd_, ld, k, f["xq"], f["xd"], f["ids"], f["w"], fz, y)
    torch.cuda.synchronize()
    for key in ("xq", "xd", "ids", "w"):
        assert_equal(to_host(f[key]), to_host(sep[key]), "prep " + key)
    n = int(to_host(g.n_active)[0])
    assert int(to_host(fz.n_active)[0]) == n
    assert_equal(to_host(fz.expert_offsets), to_host(g.expert_offsets), "prep offsets")
    assert_equal(to_host(fz.sorted_assign)[:T * k], to_host(g.sorted_assign)[:T * k], "prep sorted")
    assert_equal(to_host(fz.active_experts)[:n], to_host(g.active_experts)[:n], "prep active")
    assert not to_host(y).any(), "y not cleared"
    # and against the oracle
    xq, xdq = oracle.quantize_q8(x)
    assert_equal(to_host(f["xq"]), xq, "prep xq vs oracle")
    ids, w = oracle.route_topk(logits, k)
    assert_equal(to_host(f["ids"]), ids, "prep ids vs oracle")
    assert_tol(to_host(f["w"]), w, w, "prep w vs oracle")


@pytest.mark.parametrize("T,E,H,k", [(1, 128, 2048, 8), (8, 128, 4096, 8), (4, 256, 512, 8),
                                     (1, 1024, 64, 16), (3, 5, 64, 5), (1, 1, 32, 1),
                                     # two launches (q8 + routing, then grouping)
                                     (8, 256, 4096, 8), (16, 256, 256, 16), (4, 1024, 512, 8),
                                     (17, 64, 256, 2), (64, 256, 2048, 8), (300, 128, 512, 4),
                                     (2048, 256, 4096, 8)])
def test_decode_prep_matches_separate_calls(T, E, H, k):
    say("decode prep", T, E, H, k, "one launch" if pq.decode_prep_one_launch(T, E, k) else "two launches")
    _prep_case(T, E, H, k, seed=T * 131 + E)


def test_decode_prep_ties():
    say("decode prep ties")
    logits = np.zeros((6, 64), np.float32)
    logits[1, 10:20] = 1.0
    logits[2] = -0.0
    logits[3, ::2] = 2.5
    logits[4] = np.arange(64, dtype=np.float32)[::-1]
    _prep_case(6, 64, 128, 8, logits=logits, seed=3)


def test_decode_prep_no_tokens():
    """Zero tokens: the empty grouping (offsets all 0, no active expert)."""
    E = 64
    g = pq.GroupBuffers.empty(0, 4, E, dev())
    g.expert_offsets.fill_(-1)
    g.n_active.fill_(-1)
    st = pq.lib().pq_moe_decode_prep(None, None, 0, 256, E, 4, None, None, None, None,
                                     ctypes.c_void_p(g.expert_offsets.data_ptr()), None,
                                     ctypes.c_void_p(g.active_experts.data_ptr()),
                                     ctypes.c_void_p(g.n_active.data_ptr()), None, None)
    assert st == pq.PQ_OK
    torch.cuda.synchronize()
    assert not to_host(g.expert_offsets).any()
    assert int(to_host(g.n_active)[0]) == 0


def test_decode_prep_limits():
    """Any batch within the general limits is accepted (checked before any
    pointer); assignments beyond 1<<20 are a shape error."""
    st = pq.lib().pq_moe_decode_prep(None, None, 17, 64, 8, 2, *([None] * 9), None)
    assert st == pq.PQ_ERR_NULL
    st = pq.lib().pq_moe_decode_prep(None, None, (1 << 20) // 2 + 1, 64, 8, 2, *([None] * 9), None)
    assert st == pq.PQ_ERR_SHAPE


@pytest.mark.parametrize("T,k,rows,offset", [
    (7, 3, 100, 0),       # rows % 4 == 0: 16-byte path
    (7, 3, 101, 0),       # ragged rows: one output per thread
    (5, 2, 100, 1),       # out not 16-byte aligned: one output per thread
    (33000, 2, 12, 0),    # more tokens than one grid column holds
])
def test_combine(T, k, rows, offset):
    say("combine", T, k, rows, offset)
    rng = np.random.default_rng(5 + rows + T)
    out = rng.standard_normal((T * k, rows)).astype(np.float32)
    w = rng.random((T, k)).astype(np.float32)
    out_d = to_dev(np.concatenate([np.zeros(offset, np.float32), out.ravel()]))[offset:]
    y = pq.moe_combine(out_d.view(T * k, rows), to_dev(w), k)
    y_ref, ty = oracle.combine(out, w, k)
    assert_tol(to_host(y), y_ref, ty, "y")


# ------------------------------------------- one-token gate/up with routing

@pytest.mark.parametrize("fmt,E,H,I,k,kind", [
    ("ternary", 128, 2048, 768, 8, "normal"),    # the one-token layer shape
    ("grid1", 256, 4096, 1536, 8, "uniform"),
    ("ternary", 16, 256, 96, 4, "normal"),        # smallest rows, ragged q8 pass
    ("grid1", 8, 1536, 64, 8, "ties"),            # k == E, equal logits
    ("ternary", 1024, 512, 32, 16, "normal"),     # most experts, top-16
    ("ternary", 5, 4096, 256, 1, "ties"),
    ("ternary", 300, 1536, 64, 6, "normal"),     # rank over 300 keys, 24 lanes per row
    ("sign1", 64, 2048, 1536, 8, "normal"),       # sub-scaled signs
    ("sign1", 512, 4096, 96, 4, "ties"),          # ranking by wave maxima, equal logits
    ("sign1", 8, 256, 32, 2, "uniform"),          # smallest shapes
])
def test_decode1_gate_up(fmt, E, H, I, k, kind):
    """The routed one-token gate/up against the oracle, and bit for bit
    against the staged prep + gate/up mat-vec on the same inputs."""
    say("decode1 gate/up", fmt, E, H, I, k, kind)
    assert_plan(pq.PQ_PLAN_DECODE1_ROUTED, pq.PQ_CALL_DECODE1_GATE_UP, fmt, 1, k, E, I, H, pq.PQ_EPI_SWIGLU_Q8)
    seed = E + H + k
    x = wl.activations_f32(seed, 1, H)
    if kind == "ties":
        logits = np.zeros((1, E), np.float32)
        logits[0, ::2] = 1.5
        logits[0, 1] = -0.0
    else:
        logits = wl.router_logits(seed, 1, E, kind)
    grid = wl.codebook(seed) if fmt == "grid1" else None
    gate = wl.stack_experts(fmt, seed, "gate", E, I, H)
    up = wl.stack_experts(fmt, seed, "up", E, I, H)
    Wg, Wu = weights_to_device(fmt, gate, grid), weights_to_device(fmt, up, grid)
    xd_, lg_ = to_dev(x), to_dev(logits)
    i32 = torch.int32
    ids = torch.empty((1, k), dtype=i32, device=dev())
    w = torch.empty((1, k), device=dev())
    g = pq.GroupBuffers.empty(1, k, E, dev())
    hq = torch.empty((k, I), dtype=torch.int8, device=dev())
    hd = torch.empty((k, I // 32), device=dev())
    y = torch.full((1, H), 7.0, device=dev())
    pq.moe_decode1_gate_up(Wg, Wu, xd_, lg_, k, ids, w, g, hq, hd, y)
    # staged path
    ids2 = torch.empty_like(ids)
    w2 = torch.empty_like(w)
    g2 = pq.GroupBuffers.empty(1, k, E, dev())
    xq2 = torch.empty((1, H), dtype=torch.int8, device=dev())
    xs2 = torch.empty((1, H // 32), device=dev())
    pq.decode_prep(xd_, lg_, k, xq2, xs2, ids2, w2, g2)
    mv = {"ternary": pq.moe_matvec_ternary, "grid1": pq.moe_matvec_grid1, "sign1": pq.moe_matvec_sign1}[fmt]
    hq2, hd2 = mv(Wg, Wu, g2, xq2, xs2, True, pq.PQ_EPI_SWIGLU_Q8)
    torch.cuda.synchronize()
    na = int(to_host(g.n_active)[0])
    assert na == k
    for got, ref, what in ((ids, ids2, "ids"), (w, w2, "w"), (g.expert_offsets, g2.expert_offsets, "offsets"),
                           (g.sorted_assign[:k], g2.sorted_assign[:k], "sorted"),
                           (g.active_experts[:k], g2.active_experts[:k], "active"), (hq, hq2, "hq"),
                           (hd, hd2, "hd")):
        assert_equal(to_host(got), to_host(ref), what + " vs staged")
    assert_equal(to_host(y), np.zeros((1, H), np.float32), "y zeroed")
    # the oracle
    ids_ref, w_ref = oracle.route_topk(logits, k)
    assert_equal(to_host(ids), ids_ref, "ids")
    assert_tol(to_host(w), w_ref, w_ref, "w")
    off, srt, act = oracle.group(ids_ref, E)
    assert_equal(to_host(g.expert_offsets), off, "offsets")
    assert_equal(to_host(g.sorted_assign)[:k], srt, "sorted")
    assert_equal(to_host(g.active_experts)[:k], act, "active")
    xq, xs = oracle.quantize_q8(x)
    tok = np.zeros(k, np.int64)
    g_ref, tg, _ = moe.grouped_matvec_q8(fmt, gate, grid, ids_ref, xq, xs, tok, H, False)
    u_ref, tu, _ = moe.grouped_matvec_q8(fmt, up, grid, ids_ref, xq, xs, tok, H, False)
    q8h_check(to_host(hq), to_host(hd), g_ref, u_ref, tg, tu)


# ------------------------------------------------------- load-time helpers

@pytest.mark.parametrize("E,N,K,n_plant,seed", [(4, 96, 512, 0, 1), (4, 96, 512, 37, 2),
                                                (1, 1, 256, 5, 3), (3, 65, 1280, 1000, 4)])
def test_validate_ternary_counts(E, N, K, n_plant, seed):
    say("validate ternary", E, N, K, n_plant, seed)
    planes = wl.stack_experts("ternary", seed, "w", E, N, K)
    qs = planes["qs"].copy()
    rng = np.random.default_rng(seed)
    flat = qs.reshape(-1)
    pos = rng.integers(0, flat.size, size=n_plant)
    field = rng.integers(0, 4, size=n_plant)
    for p_, f_ in zip(pos, field):   # set one 2-bit field of the byte to 3
        flat[p_] |= np.uint8(3 << (2 * int(f_)))
    want = oracle.count_invalid_ternary(qs.reshape(E * N, K // 4), K)
    assert (want > 0) == (n_plant > 0)
    w = pq.TernaryWeights(to_dev(qs), to_dev(planes["d"]))
    n_bad = pq.validate_ternary(w)
    assert int(to_host(n_bad)[0]) == want


def test_selftest_known_answers():
    say("selftest")
    st = pq.selftest()
    assert st == pq.PQ_OK, pq.status_str(st)
