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


def _run(inp, sample=None):
    cfg = inp["cfg"]
    T, H, I, E, k = cfg["T"], cfg["H"], cfg["I"], cfg["E"], cfg["top_k"]
    A = T * k
    layer = PrefillLayer(T, H, I, E, k, dev())
    W = {n: weights_to_device(cfg["fmt"], inp[n], inp.get("grid")) for n in ("gate", "up", "down")}
    x = to_dev(inp["x_bf16"])
    dbg = {"g": torch.zeros((A, I), device=dev()), "u": torch.zeros((A, I), device=dev()),
           "h": torch.zeros((A, I), device=dev())}
    layer.route(to_dev(inp["logits"]))
    layer.gate_up(x, W["gate"], W["up"], dbg)
    layer.down(W["down"])
    layer.combine()
    torch.cuda.synchronize()
    idx = None if sample is None else torch.as_tensor(sample, device=dev())
    pick = (lambda t: to_host(t)) if idx is None else (lambda t: to_host(t.index_select(0, idx)))
    gpu = {"ids": to_host(layer.ids), "w": to_host(layer.w), "g": pick(dbg["g"]), "u": pick(dbg["u"]),
           "h": pick(dbg["h"]), "hb": pick(layer.h), "hb_all": to_host(layer.h), "out": pick(layer.out),
           "y": to_host(layer.y), "out_all": to_host(layer.out)}
    # production launch (no debug outputs) gives the same bits
    layer.gate_up(x, W["gate"], W["up"])
    torch.cuda.synchronize()
    gpu["hb_prod"] = pick(layer.h)
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
    if sample is None:
        y_ref, ty = oracle.combine(gpu["out_all"], gpu["w"], k)
        assert_tol(gpu["y"], y_ref, ty, "y")


@pytest.mark.parametrize("T,E,H,I,k,seed", [
    (48, 8, 512, 256, 2, 1),      # every expert ~12 rows
    (200, 4, 256, 256, 2, 2),     # ~100 rows per expert: two 64-row chunks, ragged second
    (37, 16, 768, 512, 4, 3),     # K = 3 blocks for gate/up, 2 for down
    (5, 64, 1024, 256, 3, 4),     # most experts empty, single rows
    (130, 1, 512, 256, 1, 5),     # one expert takes every token (3 chunks)
])
@pytest.mark.parametrize("name", ["grid1_moe_prefill_t2048", "sign1_moe_prefill_t2048"])
def test_prefill_layer_small(T, E, H, I, k, seed, name):
    if name.startswith("sign1") and (H % 512 or I % 512):
        I = 512   # sub-scaled signs need row lengths that are multiples of 512
        H = max(512, H // 512 * 512)
    say("prefill small", name, T, E, H, I, k)
    inp = wl.make_workload(name, seed=seed, T=T, E=E, H=H, I=I, top_k=k)
    gpu = _run(inp)
    _check(inp, gpu)


@pytest.mark.parametrize("name", ["grid1_moe_prefill_t2048", "sign1_moe_prefill_t2048"])
def test_prefill_layer_full_size_sampled(name):
    """2048 tokens, hidden 4096, intermediate 1536, 256 experts, top-8: all
    experts run on the GPU; 48 assignments (every column) are checked."""
    say("prefill full size", name)
    inp = wl.make_workload(name)
    rng = np.random.default_rng(0)
    A = 2048 * 8
    sample = np.sort(rng.choice(A, size=48, replace=False))
    gpu = _run(inp, sample)
    _check(inp, gpu, sample)


@pytest.mark.parametrize("N,K,T,E,k", [(100, 256, 40, 3, 2), (300, 512, 9, 5, 2), (1, 256, 3, 2, 1)])
def test_gemm_partial_column_tiles(N, K, T, E, k):
    """F32 epilogue with N not a multiple of the 256-column tile (tail columns dropped)."""
    say("gemm partial tiles", N, K, T, E, k)
    seed = 11
    planes = wl.stack_experts("grid1", seed, "w", E, N, K)
    grid = wl.codebook(seed)
    rng = np.random.default_rng(seed)
    ids = np.stack([rng.choice(E, size=k, replace=False) for _ in range(T)]).astype(np.int32)
    x = wl.activations_bf16(seed, T, K)
    g = pq.group_tokens_by_expert(to_dev(ids), E)
    W = weights_to_device("grid1", planes, grid)
    out = pq.moe_gemm_dequant_tile(W, None, g, to_dev(x), True, pq.PQ_EPI_F32)
    torch.cuda.synchronize()
    A = T * k
    y_ref, t_ref = moe.grouped_matvec_bf16("grid1", planes, grid, ids, x, np.arange(A) // k, K)
    assert_tol(to_host(out), y_ref, t_ref, "out")


@pytest.mark.parametrize("N,K,T,E,k", [(100, 512, 40, 3, 2), (300, 1024, 9, 5, 2), (1, 512, 3, 2, 1),
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
    W = weights_to_device("sign1", planes, None)
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
    Wg, Wu = weights_to_device("sign1", gate, None), weights_to_device("sign1", up, None)
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
