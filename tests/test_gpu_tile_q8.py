"""GPU parity of the int8-MFMA tile over q8 activations (pq_moe_tile_q8_*),
and of the mat-vec entry points when they hand heavily loaded experts to it,
against the CPU oracle.

Bar (as for the mat-vec): every int32 block sum bit-exact; fp32 outputs within
|got - ref| <= 1e-5 * sum|terms| + 1e-6; the SwiGLU q8 codes and scales
bit-exact against the oracle's q8 of the GPU's own fp32 h.
"""
import zlib

import numpy as np
import pytest
import torch

import bit_quantized_moe_q8_amd as pq
from bit_quantized_moe_q8_amd.layer import weights_to_device
import oracle
from oracle import moe
import workloads as wl

from gpu_util import assert_equal, assert_plan, assert_tol, dev, say, to_dev, to_host

pytestmark = pytest.mark.gpu


def _seed(*key):
    return zlib.crc32(repr(key).encode()) % 1000


def _ids(rng, E, T, k):
    return np.stack([rng.choice(E, size=k, replace=False) for _ in range(T)]).astype(np.int32)


def _tile_fn(fmt):
    return {"ternary": pq.moe_tile_q8_ternary, "grid1": pq.moe_tile_q8_grid1, "sign1": pq.moe_tile_q8_sign1}[fmt]


def _mv_fn(fmt):
    return {"ternary": pq.moe_matvec_ternary, "grid1": pq.moe_matvec_grid1, "sign1": pq.moe_matvec_sign1}[fmt]


@pytest.mark.parametrize("fmt,E,N,K,T,k,abt", [
    ("ternary", 2, 64, 256, 40, 1, True),      # ~20 per expert: both column subtiles
    ("ternary", 1, 100, 768, 70, 1, True),     # 3 chunks (32, 32, 6), ragged row tile
    ("ternary", 4, 33, 2048, 17, 2, False),    # activation row per assignment
    ("ternary", 3, 200, 4096, 33, 1, True),    # 16 slabs
    ("ternary", 16, 64, 512, 5, 3, True),      # single assignments, empty experts
    ("ternary", 2, 40, 3072, 20, 1, True),     # 12 slabs
    ("grid1", 2, 64, 256, 40, 1, True),
    ("grid1", 1, 100, 1536, 70, 1, True),
    ("grid1", 4, 40, 4096, 17, 2, False),
    ("grid1", 8, 130, 1024, 20, 3, True),      # 3 row tiles, ragged
    ("grid1", 2, 40, 6144, 20, 1, True),       # 24 slabs
    ("ternary", 2, 64, 8192, 40, 1, True),     # 32 slabs (the widest rows of the mat-vec)
    ("grid1", 1024, 32, 256, 24, 8, True),     # 1024 experts (the limit), most with one assignment
    ("ternary", 3, 100, 512, 2100, 1, True),   # > 2048 assignments: chunks of 64, ragged
    ("grid1", 5, 64, 768, 1100, 2, False),     # > 2048 assignments, activation row per assignment
    ("sign1", 2, 64, 256, 40, 1, True),        # sub-scaled signs as int8 sign * sc
    ("sign1", 4, 40, 4096, 17, 2, False),
    ("sign1", 8, 130, 768, 20, 3, True),       # a width the mat-vec has no variant for
    ("sign1", 2, 64, 8192, 40, 1, True),       # 32 slabs
    ("sign1", 3, 100, 512, 2100, 1, True),     # > 2048 assignments: chunks of 64
    ("sign1", 1024, 32, 256, 24, 8, True),     # 1024 experts
])
def test_tile_q8_f32(fmt, E, N, K, T, k, abt):
    say("tile q8 f32", fmt, E, N, K, T, k, abt)
    seed = _seed(fmt, E, N, K, T)
    rng = np.random.default_rng(seed)
    ids = _ids(rng, E, T, k)
    planes = wl.stack_experts(fmt, seed, "w", E, N, K)
    grid = wl.codebook(seed) if fmt == "grid1" else None
    n_rows = T if abt else T * k
    xq, xd = oracle.quantize_q8(wl.activations_f32(seed, n_rows, K))
    g = pq.group_tokens_by_expert(to_dev(ids), E)
    W = weights_to_device(fmt, planes, grid)
    A = T * k
    isums = torch.zeros((A, N, K // 32), dtype=torch.int32, device=dev())
    out, _ = _tile_fn(fmt)(W, None, g, to_dev(xq), to_dev(xd), abt, pq.PQ_EPI_F32, dbg={"isums": isums})
    out_prod, _ = _tile_fn(fmt)(W, None, g, to_dev(xq), to_dev(xd), abt, pq.PQ_EPI_F32)
    torch.cuda.synchronize()
    rows_of = (np.arange(A) // k) if abt else np.arange(A)
    y_ref, t_ref, i_ref = moe.grouped_matvec_q8(fmt, planes, grid, ids, xq, xd, rows_of, K)
    assert_equal(to_host(isums), i_ref, "isums")
    assert_tol(to_host(out), y_ref, t_ref, "y")
    assert_equal(to_host(out_prod), to_host(out), "debug vs production variant")


@pytest.mark.parametrize("fmt,E,I,H,T,k", [
    ("ternary", 4, 96, 512, 30, 2),
    ("ternary", 1, 32, 256, 33, 1),
    ("grid1", 2, 256, 1024, 70, 1),
    ("grid1", 8, 64, 2048, 24, 3),
    ("ternary", 4, 64, 256, 1040, 2),         # > 2048 assignments: chunks of 64
    ("sign1", 2, 256, 1024, 70, 1),
    ("sign1", 4, 64, 256, 1040, 2),
])
def test_tile_q8_swiglu(fmt, E, I, H, T, k):
    """Gate/up with the SwiGLU + q8 epilogue (rows = I, cols = H)."""
    say("tile q8 swiglu", fmt, E, I, H, T, k)
    seed = _seed("swiglu", fmt, E, I, H, T)
    rng = np.random.default_rng(seed)
    ids = _ids(rng, E, T, k)
    gate = wl.stack_experts(fmt, seed, "gate", E, I, H)
    up = wl.stack_experts(fmt, seed, "up", E, I, H)
    grid = wl.codebook(seed) if fmt == "grid1" else None
    xq, xd = oracle.quantize_q8(wl.activations_f32(seed, T, H))
    g = pq.group_tokens_by_expert(to_dev(ids), E)
    Wg, Wu = weights_to_device(fmt, gate, grid), weights_to_device(fmt, up, grid)
    A = T * k
    dbg = {"isums": torch.zeros((A, I, H // 32), dtype=torch.int32, device=dev()),
           "isums_up": torch.zeros((A, I, H // 32), dtype=torch.int32, device=dev()),
           "g": torch.zeros((A, I), device=dev()), "u": torch.zeros((A, I), device=dev()),
           "h": torch.zeros((A, I), device=dev())}
    hq, hd = _tile_fn(fmt)(Wg, Wu, g, to_dev(xq), to_dev(xd), True, pq.PQ_EPI_SWIGLU_Q8, dbg=dbg)
    hq2, hd2 = _tile_fn(fmt)(Wg, Wu, g, to_dev(xq), to_dev(xd), True, pq.PQ_EPI_SWIGLU_Q8)
    torch.cuda.synchronize()
    tok = np.arange(A) // k
    g_ref, tg, ig = moe.grouped_matvec_q8(fmt, gate, grid, ids, xq, xd, tok, H)
    u_ref, tu, iu = moe.grouped_matvec_q8(fmt, up, grid, ids, xq, xd, tok, H)
    assert_equal(to_host(dbg["isums"]), ig, "gate isums")
    assert_equal(to_host(dbg["isums_up"]), iu, "up isums")
    gg, uu, hh = to_host(dbg["g"]), to_host(dbg["u"]), to_host(dbg["h"])
    assert_tol(gg, g_ref, tg, "g")
    assert_tol(uu, u_ref, tu, "u")
    h_ref = oracle.swiglu(gg, uu)
    assert_tol(hh, h_ref, np.abs(h_ref), "h")
    hq_ref, hd_ref = oracle.quantize_q8(hh)
    assert_equal(to_host(hq), hq_ref, "hq")
    assert_equal(to_host(hd), hd_ref, "hd")
    assert_equal(to_host(hq2), to_host(hq), "hq debug vs production")
    assert_equal(to_host(hd2), to_host(hd), "hd debug vs production")


@pytest.mark.parametrize("fmt,E,H,I,T,k", [("ternary", 4, 200, 512, 20, 2), ("grid1", 2, 64, 1536, 40, 1),
                                             ("sign1", 2, 64, 1536, 40, 1)])
def test_tile_q8_combine(fmt, E, H, I, T, k):
    """Down projection with the weighted combine fused in (rows = H, cols = I)."""
    say("tile q8 combine", fmt, E, H, I, T, k)
    seed = _seed("combine", fmt, E, H, I, T)
    rng = np.random.default_rng(seed)
    ids = _ids(rng, E, T, k)
    down = wl.stack_experts(fmt, seed, "down", E, H, I)
    grid = wl.codebook(seed) if fmt == "grid1" else None
    A = T * k
    hq, hd = oracle.quantize_q8(wl.activations_f32(seed, A, I))
    w = rng.uniform(0.05, 1.0, size=(T, k)).astype(np.float32)
    g = pq.group_tokens_by_expert(to_dev(ids), E)
    Wd = weights_to_device(fmt, down, grid)
    y = torch.zeros((T, H), device=dev())
    _tile_fn(fmt)(Wd, None, g, to_dev(hq), to_dev(hd), False, pq.PQ_EPI_F32_COMBINE, out0=y, out1=to_dev(w))
    torch.cuda.synchronize()
    o_ref, to, _ = moe.grouped_matvec_q8(fmt, down, grid, ids, hq, hd, np.arange(A), I, want_isums=False)
    y_ref = np.einsum("tj,tjn->tn", w.astype(np.float64), o_ref.reshape(T, k, H))
    ty = np.einsum("tj,tjn->tn", np.abs(w.astype(np.float64)), to.reshape(T, k, H))
    # the fused combine rounds each w * out product and each of the k atomic
    # adds in fp32: (k + 1) * 2^-24 * sum|w * out|, far inside 1e-5 * ty
    assert_tol(to_host(y), y_ref, ty, "y")


@pytest.mark.parametrize("fmt,K,E,T", [("ternary", 768, 16, 40), ("grid1", 1024, 16, 40), ("ternary", 512, 1024, 600),
                                       ("sign1", 1024, 16, 40), ("sign1", 2048, 256, 300),
                                       ("ternary", 2048, 64, 1024),    # 2048 assignments: the one-launch limit
                                       ("ternary", 768, 64, 1100)])    # 2200: tile (chunks of 64) then mat-vec
def test_matvec_hands_heavy_experts_to_tile(fmt, K, E, T):
    """Through pq_moe_matvec_*: T tokens, top-2 of E experts (more
    assignments than experts, so the split grouping runs), every token's
    first choice expert 0 (T assignments) and the second spread over the
    others (a few each).  Block sums and outputs match the oracle for all;
    expert 0's outputs are the tile kernel's own bits."""
    say("matvec dispatch", fmt, K, E, T)
    N, k = 96, 2
    assert T * k > E
    # ternary rows of 768 or 2048: the tile and the mat-vec items in one launch
    mixed = pq.PQ_PLAN_MIXED if fmt == "ternary" and K in (768, 2048) and T * k <= 2048 else 0
    assert_plan(pq.PQ_PLAN_MATVEC_PAIRS | pq.PQ_PLAN_TILE_Q8 | mixed, pq.PQ_CALL_MATVEC, fmt, T, k, E, N, K)
    seed = _seed("dispatch", fmt, K, E)
    rng = np.random.default_rng(seed)
    ids = np.stack([np.zeros(T, np.int32), rng.integers(1, E, size=T).astype(np.int32)], axis=1)
    planes = wl.stack_experts(fmt, seed, "w", E, N, K)
    grid = wl.codebook(seed) if fmt == "grid1" else None
    xq, xd = oracle.quantize_q8(wl.activations_f32(seed, T, K))
    g = pq.group_tokens_by_expert(to_dev(ids), E)
    W = weights_to_device(fmt, planes, grid)
    A = T * k
    isums = torch.zeros((A, N, K // 32), dtype=torch.int32, device=dev())
    out, _ = _mv_fn(fmt)(W, None, g, to_dev(xq), to_dev(xd), True, pq.PQ_EPI_F32, dbg={"isums": isums})
    out_prod, _ = _mv_fn(fmt)(W, None, g, to_dev(xq), to_dev(xd), True, pq.PQ_EPI_F32)
    tile, _ = _tile_fn(fmt)(W, None, g, to_dev(xq), to_dev(xd), True, pq.PQ_EPI_F32)
    torch.cuda.synchronize()
    y_ref, t_ref, i_ref = moe.grouped_matvec_q8(fmt, planes, grid, ids, xq, xd, np.arange(A) // k, K)
    assert_equal(to_host(isums), i_ref, "isums")
    assert_tol(to_host(out), y_ref, t_ref, "y")
    assert_tol(to_host(out_prod), y_ref, t_ref, "y (production)")
    heavy = ids.ravel() == 0
    assert_equal(to_host(out_prod)[heavy], to_host(tile)[heavy], "heavy expert rows vs tile kernel")


def test_tile_q8_single_assignment():
    """One token on one expert of two (one chunk with one live column)."""
    say("tile q8 single")
    for fmt in ("ternary", "grid1", "sign1"):
        E, N, K = 2, 64, 512
        planes = wl.stack_experts(fmt, 3, "w", E, N, K)
        grid = wl.codebook(3) if fmt == "grid1" else None
        W = weights_to_device(fmt, planes, grid)
        ids = np.array([[1]], np.int32)
        xq, xd = oracle.quantize_q8(wl.activations_f32(3, 1, K))
        g = pq.group_tokens_by_expert(to_dev(ids), E)
        out, _ = _tile_fn(fmt)(W, None, g, to_dev(xq), to_dev(xd), True, pq.PQ_EPI_F32)
        torch.cuda.synchronize()
        y_ref, t_ref, _ = moe.grouped_matvec_q8(fmt, planes, grid, ids, xq, xd, np.arange(1), K, want_isums=False)
        assert_tol(to_host(out), y_ref, t_ref, "y")


@pytest.mark.parametrize("name", ["ternary_moe_prefill_q8_t2048", "grid1_moe_prefill_q8_t2048",
                                  "sign1_moe_prefill_q8_t2048"])
def test_q8_prefill_full_size_sampled(name):
    """2048 tokens through all 256 experts with q8 activations, in the layer
    sequence the benchmark times (the mat-vec entry points hand every expert
    with 8+ assignments to the tile kernel).  Six tokens (48 assignments) are
    checked: routing exactly, q8(h) against the free-running oracle (up to
    rounding ties), the down outputs on the GPU's own q8(h), and y."""
    from bit_quantized_moe_q8_amd.layer import DecodeLayer
    from gpu_util import q8h_check
    say("q8 prefill full size", name)
    inp = wl.make_workload(name)
    cfg = inp["cfg"]
    fmt, T, H, I, E, k = cfg["fmt"], cfg["T"], cfg["H"], cfg["I"], cfg["E"], cfg["top_k"]
    grid = inp.get("grid")
    layer = DecodeLayer(fmt, T, H, I, E, k, dev())
    assert layer.fused and not layer.fused_combine   # prep in two launches, separate combine
    W = {n: weights_to_device(fmt, inp[n], grid) for n in ("gate", "up", "down")}
    layer(to_dev(inp["x"]), to_dev(inp["logits"]), W["gate"], W["up"], W["down"])
    torch.cuda.synchronize()
    toks = np.array([0, 1, 511, 1024, 1500, T - 1])
    sub = (toks[:, None] * k + np.arange(k)).ravel()
    ref = moe.decode_ffn(inp, want_isums=False, assign_subset=sub)
    assert_equal(to_host(layer.ids), ref["ids"], "ids")
    hq, hd = to_host(layer.hq), to_host(layer.hd)
    q8h_check(hq[sub], hd[sub], ref["g"][sub], ref["u"][sub], ref["tg"][sub], ref["tu"][sub])
    o_ref, to, _ = moe.grouped_matvec_q8(fmt, inp["down"], grid, ref["ids"], hq, hd, np.arange(T * k), I,
                                         want_isums=False, assign_subset=sub)
    out = to_host(layer.out)
    assert_tol(out[sub], o_ref[sub], to[sub], "out")
    w = to_host(layer.w)
    y_ref, ty = oracle.combine(out[sub], w[toks], k)
    assert_tol(to_host(layer.y)[toks], y_ref, ty, "y")


@pytest.mark.parametrize("H,I", [(512, 256), (2048, 768)])
def test_heavy_split_layer_in_captured_graph(H, I):
    """A layer step whose mat-vec entry points launch the tile kernel for a
    heavy expert and the mat-vec for the rest (rows of 2048 and 768: both in
    one launch), captured in a graph, replays to the eager step's bits,
    three times, with eager work on the same buffers between the replays."""
    from bit_quantized_moe_q8_amd.layer import DecodeLayer
    say("heavy split layer in graph", H, I)
    fmt, T, E, k = "ternary", 16, 8, 2
    mixed = pq.PQ_PLAN_MIXED if (H, I) == (2048, 768) else 0
    assert_plan(pq.PQ_PLAN_MATVEC_PAIRS | pq.PQ_PLAN_TILE_Q8 | mixed, pq.PQ_CALL_MATVEC, fmt, T, k, E, I, H,
                pq.PQ_EPI_SWIGLU_Q8)
    assert_plan(pq.PQ_PLAN_MATVEC_PAIRS | pq.PQ_PLAN_TILE_Q8 | mixed, pq.PQ_CALL_MATVEC, fmt, T, k, E, H, I)
    rng = np.random.default_rng(5)
    logits = rng.standard_normal((T, E)).astype(np.float32)
    logits[:, 0] += 8.0          # expert 0 in every token's top-2: 16 assignments
    planes = {n: wl.stack_experts(fmt, 5, n, E, *((I, H) if n != "down" else (H, I))) for n in ("gate", "up", "down")}
    W = {n: weights_to_device(fmt, planes[n]) for n in planes}
    x = to_dev(wl.activations_f32(5, T, H))
    lg = to_dev(logits)
    layer = DecodeLayer(fmt, T, H, I, E, k, dev())
    layer(x, lg, W["gate"], W["up"], W["down"])
    torch.cuda.synchronize()
    ref_hq, ref_y = to_host(layer.hq), to_host(layer.y)
    assert (to_host(layer.ids)[:, 0] == 0).all()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        layer(x, lg, W["gate"], W["up"], W["down"])
    for rep in range(3):
        layer.hq.zero_()
        layer.y.zero_()
        layer(x, lg, W["gate"], W["up"], W["down"])   # eager work between replays
        layer.hq.zero_()
        layer.y.zero_()
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        assert_equal(to_host(layer.hq), ref_hq, "hq (replay %d)" % rep)
        assert_equal(to_host(layer.y), ref_y, "y (replay %d)" % rep)
