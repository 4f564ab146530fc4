"""GPU parity of the prefill dequant-per-tile GEMM (grid1 weights, bf16 x, MFMA) against the oracle.

fp32 G, U and down outputs: |got - ref| <= 1e-5 * sum|terms| + 1e-6, with the
terms the individual products x * w * d.  h = silu(G) * U is checked against
the fp64 value from the GPU's own G, U, and its bf16 rounding (nearest even)
bit-exactly against the oracle's rounding of the GPU's own fp32 h.  The down
GEMM is checked on the GPU's own bf16 h.
"""
import numpy as np
import pytest
import torch

import bit_quantized_moe_q8_amd as pq
from bit_quantized_moe_q8_amd.layer import PrefillLayer, weights_to_device
import oracle
from oracle import moe
import workloads as wl

from gpu_util import assert_equal, assert_tol, dev, say, to_dev, to_host

pytestmark = pytest.mark.gpu

# rows of one expert's group that one GEMM work item takes (its chunk)
CHUNK = 96


def _run(inp, sample=None, fused=False):
    cfg = inp["cfg"]
    T, H, I, E, k = cfg["T"], cfg["H"], cfg["I"], cfg["E"], cfg["top_k"]
    A = T * k
    layer = PrefillLayer(T, H, I, E, k, dev(), fused_combine=fused)
    W = {n: weights_to_device(cfg["fmt"], inp[n], inp.get("grid"), tiled=True) for n in ("gate", "up", "down")}
    x = to_dev(inp["x_bf16"])
    dbg = {"g": torch.zeros((A, I), device=dev()), "u": torch.zeros((A, I), device=dev()),
           "h": torch.zeros((A, I), device=dev())}
    layer.route(to_dev(inp["logits"]))
    layer.gate_up(x, W["gate"], W["up"], dbg)
    # fused combine: the per-assignment outputs come from the debug output
    out = torch.zeros((A, H), device=dev()) if fused else layer.out
    layer.down(W["down"], {"g": out} if fused else None)
    layer.combine()
    torch.cuda.synchronize()
    idx = None if sample is None else torch.as_tensor(sample, device=dev())
    pick = (lambda t: to_host(t)) if idx is None else (lambda t: to_host(t.index_select(0, idx)))
    gpu = {"ids": to_host(layer.ids), "w": to_host(layer.w), "g": pick(dbg["g"]), "u": pick(dbg["u"]),
           "h": pick(dbg["h"]), "hb": pick(layer.h), "hb_all": to_host(layer.h), "out": pick(out),
           "y": to_host(layer.y), "out_all": to_host(out)}
    # production launches (no debug outputs): the same h bits; y again within
    # tolerance (the fused combine's atomic order may differ)
    layer.gate_up(x, W["gate"], W["up"])
    layer.down(W["down"])
    layer.combine()
    torch.cuda.synchronize()
    gpu["hb_prod"] = pick(layer.h)
    gpu["y_prod"] = to_host(layer.y)
    return gpu


def _check(inp, gpu, sample=None):
    cfg = inp["cfg"]
    T, H, I, E, k = cfg["T"], cfg["H"], cfg["I"], cfg["E"], cfg["top_k"]
    A = T * k
    ids, w = oracle.route_topk(inp["logits"], k)
    assert_equal(gpu["ids"], ids, "ids")
    rows = np.arange(A) if sample is None else np.asarray(sample)
    tok = np.arange(A) // k
    fmt, grid = cfg["fmt"], inp.get("grid")
    g_ref, tg = moe.grouped_matvec_bf16(fmt, inp["gate"], grid, ids, inp["x_bf16"], tok, H, rows)
    u_ref, tu = moe.grouped_matvec_bf16(fmt, inp["up"], grid, ids, inp["x_bf16"], tok, H, rows)
    assert_tol(gpu["g"], g_ref[rows], tg[rows], "G")
    assert_tol(gpu["u"], u_ref[rows], tu[rows], "U")
    h_ref = oracle.swiglu(gpu["g"], gpu["u"])
    assert_tol(gpu["h"], h_ref, np.abs(h_ref), "h (fp32)")
    hb_ref = oracle.float_to_bf16(gpu["h"]).reshape(gpu["h"].shape)
    assert_equal(gpu["hb"], hb_ref, "h (bf16 rounding)")
    assert_equal(gpu["hb_prod"], gpu["hb"], "debug vs production variant")
    o_ref, to = moe.grouped_matvec_bf16(fmt, inp["down"], grid, ids, gpu["hb_all"], np.arange(A), I, rows)
    assert_tol(gpu["out"], o_ref[rows], to[rows], "out")
    # the combine (fused or not) of the GPU's own per-assignment outputs, for
    # every token: fp32 products and k fp32 additions in any order stay far
    # inside 1e-5 * sum|w * out|
    y_ref, ty = oracle.combine(gpu["out_all"], gpu["w"], k)
    assert_tol(gpu["y"], y_ref, ty, "y")
    assert_tol(gpu["y_prod"], y_ref, ty, "y (production launches)")


@pytest.mark.parametrize("T,E,H,I,k,seed", [
    (48, 8, 512, 256, 2, 1),      # every expert ~12 rows
    (200, 4, 256, 256, 2, 2),     # ~100 rows per expert: two chunks, ragged second
    (37, 16, 768, 512, 4, 3),     # K = 3 blocks for gate/up, 2 for down
    (5, 64, 1024, 256, 3, 4),     # most experts empty, single rows
    (130, 1, 512, 256, 1, 5),     # one expert takes every token (two chunks)
    (200, 1, 512, 256, 1, 6),     # one expert, three chunks (96 + 96 + 8 rows)
])
@pytest.mark.parametrize("name", ["grid1_moe_prefill_t2048", "sign1_moe_prefill_t2048"])
@pytest.mark.parametrize("fused", [True, False])
def test_prefill_layer_small(T, E, H, I, k, seed, name, fused):
    if name.startswith("sign1") and (H % 512 or I % 512):
        I = 512   # sub-scaled signs need row lengths that are multiples of 512
        H = max(512, H // 512 * 512)
    say("prefill small", name, T, E, H, I, k, "fused combine" if fused else "separate combine")
    inp = wl.make_workload(name, seed=seed, T=T, E=E, H=H, I=I, top_k=k)
    gpu = _run(inp, fused=fused)
    _check(inp, gpu)
    if not fused:
        assert_equal(gpu["y_prod"], gpu["y"], "slot-order combine is deterministic")


def _every_expert_sample(inp):
    """Assignments that cover every expert with rows: the first row of its
    last chunk (the GEMM's work unit), its last row, and one row drawn at
    random from its group; sorted, unique."""
    cfg = inp["cfg"]
    ids, _ = oracle.route_topk(inp["logits"], cfg["top_k"])
    off, srt, act = oracle.group(ids, cfg["E"])
    rng = np.random.default_rng(0)
    pick = []
    for e in act:
        b, n = int(off[e]), int(off[e + 1] - off[e])
        pick += [srt[b + (n - 1) // CHUNK * CHUNK], srt[b + n - 1], srt[b + int(rng.integers(n))]]
    return np.unique(np.asarray(pick)), act


@pytest.mark.parametrize("name", ["grid1_moe_prefill_t2048", "sign1_moe_prefill_t2048"])
def test_prefill_layer_full_size_sampled(name):
    """2048 tokens, hidden 4096, intermediate 1536, 256 experts, top-8: all
    experts run on the GPU; for every expert the first row of its last chunk,
    its last row and a random row are checked in every column (G, U,
    h, out), so an expert-index or chunk-offset error anywhere shows."""
    say("prefill full size", name)
    inp = wl.make_workload(name)
    sample, act = _every_expert_sample(inp)
    assert act.size == inp["cfg"]["E"]
    say("  %d assignments over %d experts" % (sample.size, act.size))
    gpu = _run(inp, sample)
    _check(inp, gpu, sample)


@pytest.mark.parametrize("N,K,T,E,k", [(104, 256, 40, 3, 2), (296, 512, 9, 5, 2), (8, 256, 3, 2, 1)])
def test_gemm_partial_column_tiles(N, K, T, E, k):
    """F32 epilogue with N not a multiple of the 256-column tile (tail columns
    dropped; N a multiple of the tile layout's 8-row groups)."""
    say("gemm partial tiles", N, K, T, E, k)
    seed = 11
    planes = wl.stack_experts("grid1", seed, "w", E, N, K)
    grid = wl.codebook(seed)
    rng = np.random.default_rng(seed)
    ids = np.stack([rng.choice(E, size=k, replace=False) for _ in range(T)]).astype(np.int32)
    x = wl.activations_bf16(seed, T, K)
    g = pq.group_tokens_by_expert(to_dev(ids), E)
    W = weights_to_device("grid1", planes, grid, tiled=True)
    out = pq.moe_gemm_dequant_tile(W, None, g, to_dev(x), True, pq.PQ_EPI_F32)
    torch.cuda.synchronize()
    A = T * k
    y_ref, t_ref = moe.grouped_matvec_bf16("grid1", planes, grid, ids, x, np.arange(A) // k, K)
    assert_tol(to_host(out), y_ref, t_ref, "out")


@pytest.mark.parametrize("pattern", ["zeros", "equal", "wide"])
def test_gemm_grid1_scale_patterns(pattern):
    """The GEMM applies each 256-weight block's scale to one running
    accumulator (rescaled by the ratio of consecutive nonzero scales, weights
    of zero-scale blocks masked): block scales of zero (first block, runs of
    zeros, whole rows), equal consecutive scales, and scales spread over the
    fp16 range, against the oracle at the stated bound."""
    say("gemm grid1 scales", pattern)
    N, K, T, E, k, seed = 48, 2048, 120, 3, 2, 31
    planes = wl.stack_experts("grid1", seed, "w", E, N, K)
    rng = np.random.default_rng(seed)
    d = planes["d"].view(np.float16).astype(np.float32).reshape(E, N, K // 256)
    if pattern == "zeros":
        d[rng.random(d.shape) < 0.3] = 0.0
        d[:, 0:4, 0] = 0.0          # the first block
        d[:, 4:8, 2:6] = 0.0        # a run of blocks
        d[:, 8:16, :] = 0.0         # whole rows
        d[:, 16:20, 1:] = 0.0       # only the first block nonzero
    elif pattern == "equal":
        d[:, :24, :] = d[:, :24, :1]           # one scale per row
        d[:, 24:, 2::2] = d[:, 24:, 1:-1:2]    # pairs of equal neighbours
    else:
        d = (2.0 ** rng.integers(-20, 12, size=d.shape) * rng.uniform(1, 2, size=d.shape)).astype(np.float32)
        d *= np.where(rng.random(d.shape) < 0.2, -1.0, 1.0)
    planes["d"] = d.astype(np.float16).reshape(planes["d"].shape).view(planes["d"].dtype)
    grid = wl.codebook(seed)
    ids = np.stack([rng.choice(E, size=k, replace=False) for _ in range(T)]).astype(np.int32)
    x = wl.activations_bf16(seed, T, K)
    g = pq.group_tokens_by_expert(to_dev(ids), E)
    W = weights_to_device("grid1", planes, grid, tiled=True)
    out = pq.moe_gemm_dequant_tile(W, None, g, to_dev(x), True, pq.PQ_EPI_F32)
    torch.cuda.synchronize()
    A = T * k
    y_ref, t_ref = moe.grouped_matvec_bf16("grid1", planes, grid, ids, x, np.arange(A) // k, K)
    got = to_host(out)
    assert_tol(got, y_ref, t_ref, "out")
    if pattern == "zeros":
        rows_zero = np.zeros((A, N), bool)
        rows_zero[:, 8:16] = True
        assert np.all(got[rows_zero] == 0.0)


@pytest.mark.parametrize("N,K,T,E,k", [(104, 512, 40, 3, 2), (296, 1024, 9, 5, 2), (8, 512, 3, 2, 1),
                                       (64, 4096, 70, 2, 1),
                                       (48, 512, 100, 1024, 8)])   # 1024 experts, most empty or single rows
def test_gemm_sign1_f32(N, K, T, E, k):
    """Sub-scaled sign weights through the GEMM (bf16 of sign * sc, the row
    anchor per block), F32 epilogue, partial column tiles; debug and
    production launches give the same bits."""
    say("gemm sign1 f32", N, K, T, E, k)
    seed = N + K + T
    planes = wl.stack_experts("sign1", seed, "w", E, N, K)
    rng = np.random.default_rng(seed)
    ids = np.stack([rng.choice(E, size=k, replace=False) for _ in range(T)]).astype(np.int32)
    x = wl.activations_bf16(seed, T, K)
    g = pq.group_tokens_by_expert(to_dev(ids), E)
    W = weights_to_device("sign1", planes, None, tiled=True)
    A = T * k
    dbg = {"g": torch.zeros((A, N), device=dev())}
    out = pq.moe_gemm_dequant_tile(W, None, g, to_dev(x), True, pq.PQ_EPI_F32, dbg=dbg)
    out2 = pq.moe_gemm_dequant_tile(W, None, g, to_dev(x), True, pq.PQ_EPI_F32)
    torch.cuda.synchronize()
    y_ref, t_ref = moe.grouped_matvec_bf16("sign1", planes, None, ids, x, np.arange(A) // k, K)
    assert_tol(to_host(out), y_ref, t_ref, "out")
    assert_equal(to_host(out2), to_host(out), "debug vs production variant")


@pytest.mark.parametrize("I,H,T,E,k", [(96, 1024, 50, 4, 2), (256, 512, 20, 2, 1)])
def test_gemm_sign1_swiglu(I, H, T, E, k):
    """Gate/up with the SwiGLU bf16 epilogue over sub-scaled signs: G and U
    against the oracle, h against the GPU's own G and U, its bf16 rounding
    bit-exact, production bits equal to the debug launch's."""
    say("gemm sign1 swiglu", I, H, T, E, k)
    seed = I + H + T
    gate = wl.stack_experts("sign1", seed, "gate", E, I, H)
    up = wl.stack_experts("sign1", seed, "up", E, I, H)
    rng = np.random.default_rng(seed)
    ids = np.stack([rng.choice(E, size=k, replace=False) for _ in range(T)]).astype(np.int32)
    x = wl.activations_bf16(seed, T, H)
    g = pq.group_tokens_by_expert(to_dev(ids), E)
    Wg, Wu = weights_to_device("sign1", gate, None, tiled=True), weights_to_device("sign1", up, None, tiled=True)
    A = T * k
    dbg = {"g": torch.zeros((A, I), device=dev()), "u": torch.zeros((A, I), device=dev()),
           "h": torch.zeros((A, I), device=dev())}
    hb = pq.moe_gemm_dequant_tile(Wg, Wu, g, to_dev(x), True, pq.PQ_EPI_SWIGLU_BF16, dbg=dbg)
    hb2 = pq.moe_gemm_dequant_tile(Wg, Wu, g, to_dev(x), True, pq.PQ_EPI_SWIGLU_BF16)
    torch.cuda.synchronize()
    tok = np.arange(A) // k
    g_ref, tg = moe.grouped_matvec_bf16("sign1", gate, None, ids, x, tok, H)
    u_ref, tu = moe.grouped_matvec_bf16("sign1", up, None, ids, x, tok, H)
    gg, uu, hh = to_host(dbg["g"]), to_host(dbg["u"]), to_host(dbg["h"])
    assert_tol(gg, g_ref, tg, "G")
    assert_tol(uu, u_ref, tu, "U")
    h_ref = oracle.swiglu(gg, uu)
    assert_tol(hh, h_ref, np.abs(h_ref), "h (fp32)")
    hb_host = to_host(hb).view(np.uint16) if to_host(hb).dtype != np.uint16 else to_host(hb)
    assert_equal(hb_host.reshape(hh.shape), oracle.float_to_bf16(hh).reshape(hh.shape), "h (bf16 rounding)")
    assert_equal(to_host(hb2), to_host(hb), "debug vs production variant")


@pytest.mark.parametrize("fmt,E,N,K", [("grid1", 3, 24, 1024), ("grid1", 1, 8, 256), ("sign1", 2, 40, 1536),
                                       ("sign1", 1, 8, 512)])
def test_tile_layout_is_the_stated_permutation(fmt, E, N, K):
    """pq_tile_layout_{grid1,sign1} against the layout written out with numpy
    reshapes (groups of 4 rows x 32 bytes per block for qs/signs, 8 rows x 16
    bytes per block for qh and per block pair for sc): bit-exact; d and the
    grid are shared, not copied."""
    say("tile layout", fmt, E, N, K)
    planes = wl.stack_experts(fmt, 3 + N, "w", E, N, K)
    grid = wl.codebook(3) if fmt == "grid1" else None
    W = weights_to_device(fmt, planes, grid)
    T = pq.tile_layout(W)
    torch.cuda.synchronize()
    KB = K // 256

    def regroup(a, R, nb, unit):
        b = np.ascontiguousarray(a).view(np.uint8).reshape(E, N // R, R, nb, unit)
        return b.transpose(0, 1, 3, 2, 4).reshape(-1)

    if fmt == "grid1":
        pairs = [(T.qs, regroup(planes["qs"], 4, KB, 32)), (T.qh, regroup(planes["qh"], 8, KB, 16))]
        assert T.d.data_ptr() == W.d.data_ptr() and T.grid.data_ptr() == W.grid.data_ptr()
    else:
        pairs = [(T.signs, regroup(planes["signs"], 4, KB, 32)), (T.sc, regroup(planes["sc"], 8, KB // 2, 16))]
        assert T.d.data_ptr() == W.d.data_ptr()
    for got, want in pairs:
        assert_equal(to_host(got).view(np.uint8).reshape(-1), want, "tile layout")
    assert T.tiled and not W.tiled


@pytest.mark.parametrize("name", ["grid1_moe_prefill_t2048", "sign1_moe_prefill_t2048"])
def test_prefill_layer_in_captured_graph(name):
    """The prefill layer (route, group, gate/up GEMM, down GEMM, combine: the
    step the benchmark replays) captured in a graph and replayed three times
    with eager steps on other inputs between the replays: every replay gives
    the eager run's ids, h and y bit for bit (no atomics on this path), and
    the eager run matches the oracle."""
    say("prefill layer in graph", name)
    T, E, H, I, k = 200, 8, 512, 512, 2
    inp = wl.make_workload(name, seed=21, T=T, E=E, H=H, I=I, top_k=k)
    layer = PrefillLayer(T, H, I, E, k, dev())
    W = {n: weights_to_device(inp["cfg"]["fmt"], inp[n], inp.get("grid"), tiled=True) for n in ("gate", "up", "down")}
    x, logits = to_dev(inp["x_bf16"]), to_dev(inp["logits"])
    other = wl.make_workload(name, seed=22, T=T, E=E, H=H, I=I, top_k=k)
    ox, olg = to_dev(other["x_bf16"]), to_dev(other["logits"])
    layer(x, logits, W["gate"], W["up"], W["down"])
    torch.cuda.synchronize()
    ref = {"ids": to_host(layer.ids), "h": to_host(layer.h.view(torch.int16)), "y": to_host(layer.y)}
    gpu = _run(inp)          # the staged check of the same inputs against the oracle
    _check(inp, gpu)
    assert_equal(gpu["y_prod"], ref["y"], "eager layer call vs staged run")
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        layer(x, logits, W["gate"], W["up"], W["down"])
    for rep in range(3):
        layer(ox, olg, W["gate"], W["up"], W["down"])   # eager step on other inputs
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        assert_equal(to_host(layer.ids), ref["ids"], "ids (replay %d)" % rep)
        assert_equal(to_host(layer.h.view(torch.int16)), ref["h"], "h (replay %d)" % rep)
        assert_equal(to_host(layer.y), ref["y"], "y (replay %d)" % rep)
