"""Benchmark of the packed 1-bit-class MoE expert path on one MI355X.

By default every workload of the five-shape suite runs in one process and one
JSON line reports them all:

  ternary_matvec_1024          one 1024x1024 ternary mat-vec, one token
  ternary_moe_decode_t1        ternary MoE FFN decode, 1 token (E 128, H 2048, I 768)
  grid1_moe_decode_t8          grid1 MoE FFN decode, 8 tokens (E 256, H 4096, I 1536)
  ternary_moe_decode_t64_zipf  ternary MoE decode, 64 Zipf-routed tokens (E 256)
  grid1_moe_prefill_t2048      prefill: 2048 tokens through the grid1 experts (bf16 MFMA GEMM)

The headline (the top-level metric/value/roofline) is the largest of them, the
2048-token prefill; the others sit under "configs" with the same fields.

A step is one pass of the whole hot path over one batch of synthetic input:
decode: q8(x) -> top-k route -> group -> fused gate/up mat-vec (SwiGLU + q8)
-> down mat-vec -> weighted combine; prefill: route -> group -> gate/up GEMM
(SwiGLU, bf16 h) -> down GEMM -> combine; the single matrix: q8(x) and
the mat-vec in one launch.  Prefill weights are held in the GEMM's tile layout, built once
on the device when the pool is made (as a model loader would), outside every
timed region.  Each step uses the weights of a different layer from a rotating
pool sized so that the packed bytes touched between two visits of a layer
exceed the 256 MB last-level cache several times over: weights come from
HBM, not from cache.  Steps are captured in HIP graphs of --graph-steps layer
steps (as a model's decode step would be) and replayed; the K timed steps are
exactly K (whole graphs plus one shorter graph for the remainder), and so are
the W warmup steps.

value (per workload): decode: packed weight bytes of the experts touched per
step / step time (GB/s); prefill: the algorithmic GEMM flops of a step /
step time (TFLOP/s).
roofline: the dominant kernel (the fused gate/up), its algorithmic bytes
(decode) or flops (prefill) per launch over its average launch time,
measured with HIP events around a graph of launches on the launch stream,
against the nominal peak (8 TB/s, 2.5 PFLOP/s bf16) and against the rates
measured on the same device in the same run (a read stream, an MFMA loop).
For the single matrix the roofline kernel is the mat-vec over stacked pools
of 1024 matrices per launch (the streaming rate); its step is one call.
cpu_baseline: the CPU oracle on a bounded sample of the same steps.

Usage: python bench.py [--gpus 1] [--steps K] [--warmup W] [--workload all|NAME]
"""
from __future__ import annotations

import argparse
import json
import math
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

HBM_PEAK_GBS = 8000.0
BF16_PEAK_TFLOPS = 2500.0
INT8_PEAK_TOPS = 5000.0
MALL_BYTES = 256 << 20

SUITE = ["ternary_matvec_1024", "ternary_moe_decode_t1", "grid1_moe_decode_t8",
         "ternary_moe_decode_t64_zipf", "grid1_moe_prefill_t2048"]
HEADLINE = "grid1_moe_prefill_t2048"
METRIC = "decode expert mat-vec GB/s (packed bytes) & % HBM peak; prefill GEMM % MFMA peak"


def parse():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=64)
    ap.add_argument("--warmup", type=int, default=16)
    ap.add_argument("--workload", default="all", help="'all' (the five-shape suite) or one workload name")
    ap.add_argument("--seed", type=int, default=None)
    ap.add_argument("--graph-steps", type=int, default=8, help="layer steps per captured graph")
    ap.add_argument("--kernel-launches", type=int, default=64,
                    help="launches of the dominant kernel timed with HIP events")
    ap.add_argument("--cpu-seconds", type=float, default=4.0,
                    help="oracle sample budget per workload (0 = skip)")
    ap.add_argument("--no-graph", action="store_true", help="launch steps eagerly")
    ap.add_argument("--no-peaks", action="store_true", help="skip the measured read / MFMA peaks")
    ap.add_argument("--copy-calibration", action="store_true",
                    help="only run a plain device copy of known size (counter calibration)")
    return ap.parse_args()


COPY_BYTES = 512 << 20
COPY_REPS = 8


def copy_calibration():
    """A plain device-to-device copy of COPY_BYTES, COPY_REPS times: the
    reference that scales the HBM byte counters (FETCH_SIZE, WRITE_SIZE)."""
    import torch
    src = torch.empty(COPY_BYTES, dtype=torch.uint8, device="cuda:0").fill_(1)
    dst = torch.empty_like(src)
    torch.cuda.synchronize()
    for _ in range(COPY_REPS):
        dst.copy_(src)
    torch.cuda.synchronize()
    print(json.dumps({"copy_bytes": COPY_BYTES, "reps": COPY_REPS}), flush=True)


def kernel_sources_sha256(names):
    import hashlib
    h = hashlib.sha256()
    for n in names:
        with open(os.path.join(ROOT, "bit_quantized_moe_q8_amd", "csrc", n), "rb") as f:
            h.update(f.read())
    return h.hexdigest()


def measured_traffic(workload, sources):
    """HBM bytes per launch of the dominant kernel from the committed counter
    record, or None when there is none or the kernel sources changed since."""
    path = os.path.join(ROOT, "profiles", "traffic.json")
    try:
        with open(path) as f:
            rec = json.load(f).get(workload)
    except (OSError, ValueError):
        return None
    if not rec or rec.get("sources_sha256") != kernel_sources_sha256(sources):
        return None
    return rec.get("hbm_bytes_per_launch")


def log(*a):
    print(*a, file=sys.stderr, flush=True)


# --------------------------------------------------------------------- timing

class StepRunner:
    """Runs the steps of a rotating pool of L layers, M steps per captured
    graph: warmup(W) and timed(K) each run exactly that many steps, in whole
    graphs of M consecutive layers plus one graph for the remainder."""

    def __init__(self, step, L, M, use_graph):
        import torch
        self.torch = torch
        self.step, self.L, self.M, self.use_graph = step, L, M, use_graph
        self.graphs = {}
        self.cursor = 0

    def _chunks(self, n):
        out, c = [], self.cursor
        while n > 0:
            r = min(self.M, n)
            out.append((c % self.L, r))
            c += r
            n -= r
        return out, c

    def prepare(self, *counts):
        """Capture every graph the given sequence of step counts will replay."""
        if not self.use_graph:
            return
        torch = self.torch
        c0 = self.cursor
        for _ in range(2):   # warm the kernels before capture
            self.step(0)
        torch.cuda.synchronize()
        for n in counts:
            chunks, self.cursor = self._chunks(n)
            for key in chunks:
                if key not in self.graphs:
                    g = torch.cuda.CUDAGraph()
                    with torch.cuda.graph(g):
                        for i in range(key[1]):
                            self.step((key[0] + i) % self.L)
                    self.graphs[key] = g
        self.cursor = c0
        torch.cuda.synchronize()

    def run(self, n):
        chunks, self.cursor = self._chunks(n)
        for start, r in chunks:
            if self.use_graph:
                self.graphs[(start, r)].replay()
            else:
                for i in range(r):
                    self.step((start + i) % self.L)
        return chunks


def time_steps(runner, K, W):
    """(ms_total, layers of the timed steps) for K steps after W warmup steps."""
    torch = runner.torch
    runner.prepare(W, K)
    runner.run(W)
    torch.cuda.synchronize()
    ev0, ev1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    ev0.record()
    chunks = runner.run(K)
    ev1.record()
    torch.cuda.synchronize()
    layers = [(s + i) % runner.L for s, r in chunks for i in range(r)]
    return ev0.elapsed_time(ev1), layers


def time_launches(fn, R, use_graph):
    """Average ms of fn(i), i = 0..R-1, replayed from one graph (or eagerly),
    between two HIP events on the current stream."""
    import torch
    if use_graph:
        g = torch.cuda.CUDAGraph()
        with torch.cuda.graph(g):
            for i in range(R):
                fn(i)
        g.replay()
        torch.cuda.synchronize()
    k0, k1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    torch.cuda._sleep(50_000_000)
    k0.record()
    if use_graph:
        g.replay()
    else:
        for i in range(R):
            fn(i)
    k1.record()
    torch.cuda.synchronize()
    return k0.elapsed_time(k1) / R


# ---------------------------------------------------------------- measured peaks

def measure_peaks():
    """Achievable rates on this device: a 4 GiB read stream (GB/s) and a
    bf16 MFMA loop (TFLOP/s), best of 5 after a warmup."""
    import torch
    import bit_quantized_moe_q8_amd as pq
    dev = torch.device("cuda:0")
    buf = torch.empty(4 << 30, dtype=torch.uint8, device=dev).fill_(3)
    isink = torch.zeros(1024, dtype=torch.int32, device=dev)
    fsink = torch.zeros(1024, dtype=torch.float32, device=dev)
    best_r, best_m = 0.0, 0.0
    wgs = 4 * 256      # four waves per SIMD
    iters = 8000
    for rep in range(6):
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record()
        nb = pq.peak_read(buf, isink)
        e1.record()
        torch.cuda.synchronize()
        if rep:
            best_r = max(best_r, nb / (e0.elapsed_time(e1) * 1e-3) / 1e9)
        e0.record()
        fl = pq.peak_mfma_bf16(wgs, iters, fsink)
        e1.record()
        torch.cuda.synchronize()
        if rep:
            best_m = max(best_m, fl / (e0.elapsed_time(e1) * 1e-3) / 1e12)
    del buf
    torch.cuda.empty_cache()
    log("measured peaks: read %.0f GB/s, bf16 MFMA loop %.0f TFLOP/s" % (best_r, best_m))
    return {"read_gbs": round(best_r, 1), "mfma_bf16_tflops": round(best_m, 1),
            "how": "best of 5: a 4 GiB read stream with 16-byte loads (pq_peak_read); "
                   "1024 workgroups x 4 waves x 8000 x 8 back-to-back v_mfma_f32_16x16x32_bf16 "
                   "on register operands (pq_peak_mfma_bf16)"}


# ------------------------------------------------------------------ workloads

def make_pool(fmt, E, rows_cols, L, seed, dev, grid_seed, tiled=False):
    """L layers of random packed weights on the device; `tiled`: code planes in
    the tile layout of the prefill GEMM (built on the device, outside any
    timed region, as a model loader would)."""
    import torch
    import bit_quantized_moe_q8_amd as pq
    import workloads as wl
    gen = torch.Generator(device=dev)
    gen.manual_seed(seed)
    grid = torch.from_numpy(wl.codebook(grid_seed)).to(dev) if fmt == "grid1" else None
    layers = []
    for _ in range(L):
        lay = {}
        for name, (n, kk) in rows_cols.items():
            if fmt == "ternary":
                w = pq.TernaryWeights(**wl.torch_ternary_planes(gen, E, n, kk, dev))
            elif fmt == "sign1":
                w = pq.Sign1Weights(**wl.torch_sign1_planes(gen, E, n, kk, dev))
            else:
                w = pq.Grid1Weights(grid=grid, **wl.torch_grid1_planes(gen, E, n, kk, dev))
            lay[name] = pq.tile_layout(w) if tiled else w
            del w
        layers.append(lay)
    return layers


# the tile layout's (rows per group, 16-byte..32-byte unit, 256-column blocks
# per unit) of each code plane
TILE_PLANES = {"qs": (4, 32, 1), "signs": (4, 32, 1), "qh": (8, 16, 1), "sc": (8, 16, 2)}


def untile(a, f):
    """Host copy of a tile-layout plane [E][rows][bytes per row] back in row order."""
    import numpy as np
    R, unit, per = TILE_PLANES[f]
    E, N = a.shape[0], a.shape[1]
    b = np.ascontiguousarray(a).view(np.uint8).reshape(E, N, -1)
    nb = b.shape[2] // unit
    out = b.reshape(E, N // R, nb, R, unit).transpose(0, 1, 3, 2, 4).reshape(E, N, nb * unit)
    return np.ascontiguousarray(out).view(a.dtype).reshape(a.shape)


def bench_layer_workload(name, args, peaks):
    import numpy as np
    import torch

    import bit_quantized_moe_q8_amd as pq
    from bit_quantized_moe_q8_amd.layer import DecodeLayer, PrefillLayer
    import workloads as wl

    cfg = dict(wl.WORKLOADS[name])
    seed = cfg["seed"] if args.seed is None else args.seed
    fmt, T, H, I, E, k = cfg["fmt"], cfg["T"], cfg["H"], cfg["I"], cfg["E"], cfg["top_k"]
    prefill = cfg["kind"] == "prefill"
    q8_prefill = cfg["kind"] == "prefill_q8"
    dev = torch.device("cuda:0")

    per_matrix = wl.packed_bytes_per_matrix(fmt, I, H)      # gate or up ([I][H])
    # down is [H][I]: the same size for per-256 scales, larger by its extra
    # rows' anchors for the sub-scaled signs (one anchor per row)
    per_expert = 2 * per_matrix + wl.packed_bytes_per_matrix(fmt, H, I)
    touched_est = min(E, T * k) * per_expert
    M = max(1, args.graph_steps)
    L = max(8, int(math.ceil(4 * MALL_BYTES / max(touched_est, 1))))
    L = min(int(math.ceil(L / M) * M), 256)
    log("workload %s: %d layers in the pool (%.2f GB packed), %d steps per graph" % (
        name, L, L * E * per_expert / 1e9, M))

    layers = make_pool(fmt, E, {"gate": (I, H), "up": (I, H), "down": (H, I)}, L, seed, dev, seed, tiled=prefill)
    xs, lg = [], []
    for l in range(L):
        if prefill:
            xs.append(torch.from_numpy(wl.activations_bf16(seed, T, H, index=l).view(np.int16)).to(dev))
        else:
            xs.append(torch.from_numpy(wl.activations_f32(seed, T, H, index=l)).to(dev))
        lg.append(torch.from_numpy(wl.router_logits(seed, T, E, cfg["logits"], index=l)).to(dev))

    layer = PrefillLayer(T, H, I, E, k, dev) if prefill else DecodeLayer(fmt, T, H, I, E, k, dev)
    step = lambda l: layer(xs[l], lg[l], layers[l]["gate"], layers[l]["up"], layers[l]["down"])

    # experts touched per layer input (the library's own routing + grouping);
    # every layer input also gets its own routing buffers for the kernel timing
    n_active, states = [], []
    for l in range(L):
        st = layer.new_route_state()
        layer.use_state(st)
        if prefill:
            layer.route(lg[l])
        else:
            layer.route(xs[l], lg[l])
        states.append(st)
    torch.cuda.synchronize()
    n_active = [int(st["groups"].n_active.item()) for st in states]
    layer.use_state(layer.new_route_state())

    K, W = args.steps, args.warmup
    runner = StepRunner(step, L, M, not args.no_graph)
    ms_total, step_layers = time_steps(runner, K, W)
    ms_step = ms_total / K
    bytes_steps = sum(n_active[l] * per_expert for l in step_layers)
    gbs = bytes_steps / (ms_total * 1e-3) / 1e9
    tokens_s = K * T / (ms_total * 1e-3)
    step_flops = 2.0 * T * k * 3 * I * H   # gate, up and down GEMMs
    log("  step: %.4f ms, %.1f GB/s packed, %.0f tokens/s" % (ms_step, gbs, tokens_s))

    # ---- dominant kernel: the fused gate/up, one launch per pool layer (cycling)
    decode1 = (not prefill) and layer.decode1

    def dominant(i):
        l = i % L
        layer.use_state(states[l])
        if prefill:
            layer.gate_up(xs[l], layers[l]["gate"], layers[l]["up"])
        elif q8_prefill:
            tile = {"ternary": pq.moe_tile_q8_ternary, "grid1": pq.moe_tile_q8_grid1,
                    "sign1": pq.moe_tile_q8_sign1}[fmt]
            tile(layers[l]["gate"], layers[l]["up"], layer.groups, layer.xq, layer.xd, True,
                 pq.PQ_EPI_SWIGLU_Q8, layer.hq, layer.hd)
        elif decode1:
            st = states[l]
            pq.moe_decode1_gate_up(layers[l]["gate"], layers[l]["up"], xs[l], lg[l], k, st["ids"],
                                   st["w"], st["groups"], layer.hq, layer.hd, layer.y)
        else:
            layer.gate_up(layers[l]["gate"], layers[l]["up"])

    R = max(1, min(args.kernel_launches, 4 * L))
    avg_ms = time_launches(dominant, R, not args.no_graph)
    plan = pq.plan(pq.PQ_CALL_GEMM if prefill else pq.PQ_CALL_TILE_Q8 if q8_prefill
                   else pq.PQ_CALL_DECODE1_GATE_UP if decode1 else pq.PQ_CALL_MATVEC,
                   fmt, T, k, E, I, H, pq.PQ_EPI_SWIGLU_BF16 if prefill else pq.PQ_EPI_SWIGLU_Q8)
    kfiles = (["k_gemm.hip"] if plan & pq.PQ_PLAN_GEMM else
              ["k_matvec1.hip"] if plan & pq.PQ_PLAN_DECODE1_ROUTED else
              (["k_matvec.hip"] if plan & (pq.PQ_PLAN_MATVEC | pq.PQ_PLAN_MATVEC_PAIRS) else []) +
              (["k_tile_q8.hip", "k_tile_q8.hpp"] if plan & pq.PQ_PLAN_TILE_Q8 else []))
    traffic = measured_traffic(name, kfiles + ["pq_device.hpp", "pq_internal.hpp"])
    if prefill or q8_prefill:
        ops = 2.0 * T * k * 2 * I * H
        ach = ops / (avg_ms * 1e-3) / 1e12
        peak = BF16_PEAK_TFLOPS if prefill else INT8_PEAK_TOPS
        roofline = {"bound": "mfma",
                    "kernel": ("k_gemm (gate/up, bf16 MFMA, SwiGLU epilogue)" if prefill
                               else "k_tile_q8 (gate/up, int8 MFMA, SwiGLU+q8 epilogue)"),
                    "achieved": round(ach, 2), "peak": peak, "unit": "TFLOP/s" if prefill else "TOP/s",
                    "frac": round(ach / peak, 4), "traffic": traffic,
                    "avg_launch_us": round(avg_ms * 1e3, 3), "ops_per_launch": ops}
        if prefill and peaks:
            roofline["frac_of_measured_mfma_loop"] = round(ach / peaks["mfma_bf16_tflops"], 4)
    else:
        kbytes = sum(n_active[i % L] * 2 * per_matrix for i in range(R)) / R
        ach = kbytes / (avg_ms * 1e-3) / 1e9
        kname = ("k_matvec_tok1 (one token: routing, q8, gate/up, SwiGLU+q8 epilogue)" if decode1
                 else "k_matvec_mixed (gate/up in one launch, SwiGLU+q8 epilogue: experts with 8+ "
                      "assignments on the int8-MFMA tile, the rest on the mat-vec)"
                 if plan & pq.PQ_PLAN_MIXED
                 else "k_tile_q8 + k_matvec (gate/up, SwiGLU+q8 epilogue; experts with 8+ "
                      "assignments on the int8-MFMA tile, the rest on the mat-vec)"
                 if plan & pq.PQ_PLAN_TILE_Q8 else "k_matvec (gate/up, SwiGLU+q8 epilogue)")
        roofline = {"bound": "hbm", "kernel": kname, "achieved": round(ach, 1), "peak": HBM_PEAK_GBS,
                    "unit": "GB/s", "frac": round(ach / HBM_PEAK_GBS, 4), "traffic": traffic,
                    "avg_launch_us": round(avg_ms * 1e3, 3), "bytes_per_launch": round(kbytes)}
        if peaks:
            roofline["frac_of_measured_read"] = round(ach / peaks["read_gbs"], 4)
    log("  dominant kernel: %.2f us per launch, %s %s" % (avg_ms * 1e3, roofline["achieved"], roofline["unit"]))

    cpu = None
    if args.cpu_seconds > 0:
        cpu = cpu_baseline_layers(args, cfg, layers, xs, lg, n_active, per_expert, L, prefill, q8_prefill)

    res = {"workload": name, "format": fmt, "tokens": T, "hidden": H, "intermediate": I, "experts": E,
           "top_k": k, "layers_in_pool": L, "steps_per_graph": M if not args.no_graph else 0,
           "step_us": round(ms_step * 1e3, 3), "ms_per_step": round(ms_step, 6),
           "packed_gbs": round(gbs, 2), "hbm_frac_step": round(gbs / HBM_PEAK_GBS, 4),
           "packed_bytes_per_step": round(bytes_steps / K), "tokens_per_s": round(tokens_s, 1),
           "dispatch": plan, "roofline": roofline, "cpu_baseline": cpu}
    if prefill:
        tf = step_flops / (ms_step * 1e-3) / 1e12
        res.update(value=round(tf, 2), unit="TFLOP/s", dtype="bf16", step_flops=step_flops)
    else:
        res.update(value=round(gbs, 2), unit="GB/s", dtype="int8")
    del layers, xs, lg, states, layer, runner
    torch.cuda.synchronize()
    torch.cuda.empty_cache()
    return res


def bench_single_matrix(name, args, peaks):
    """The single 1024x1024 ternary mat-vec: per call (q8 and the mat-vec in
    one launch, pq_matvec_x32_ternary; one distinct matrix per step from a
    1.1 GB pool) and the streaming rate of
    the mat-vec over stacked launches of 1024 matrices each (1024 tokens, one
    matrix per token)."""
    import numpy as np
    import torch

    import bit_quantized_moe_q8_amd as pq
    import workloads as wl

    cfg = dict(wl.WORKLOADS[name])
    seed = cfg["seed"] if args.seed is None else args.seed
    N, K = cfg["N"], cfg["K"]
    dev = torch.device("cuda:0")
    per_matrix = wl.packed_bytes_per_matrix("ternary", N, K)
    P, S = 4096, 1024   # matrices in the pool, matrices per stacked launch
    M = max(1, args.graph_steps)
    log("workload %s: %d matrices in the pool (%.2f GB packed), %d steps per graph" % (
        name, P, P * per_matrix / 1e9, M))
    gen = torch.Generator(device=dev)
    gen.manual_seed(seed)
    pool = pq.TernaryWeights(**wl.torch_ternary_planes(gen, P, N, K, dev))
    xs = [torch.from_numpy(wl.activations_f32(seed, 1, K, index=i)).to(dev).view(-1) for i in range(64)]
    y = torch.empty((N,), dtype=torch.float32, device=dev)

    def step(i):
        # matrix i of the pool, q8 of x inside the same launch
        pq.matvec_x32(pool, xs[i % 64], i, y)

    K_, W = args.steps, args.warmup
    runner = StepRunner(step, P, M, not args.no_graph)
    ms_total, _ = time_steps(runner, K_, W)
    ms_step = ms_total / K_
    gbs = K_ * per_matrix / (ms_total * 1e-3) / 1e9
    log("  per call: %.2f us (q8 and mat-vec in one launch), %.1f GB/s packed" % (ms_step * 1e3, gbs))

    # stacked: launch j runs matrices [j*S, (j+1)*S), token t on matrix t
    stacks = [pq.TernaryWeights(pool.qs[j * S:(j + 1) * S], pool.d[j * S:(j + 1) * S]) for j in range(P // S)]
    ids = torch.arange(S, dtype=torch.int32, device=dev).view(S, 1)
    gS = pq.group_tokens_by_expert(ids, S)
    xqS, xdS = pq.quantize_act_q8(torch.from_numpy(wl.activations_f32(seed, S, K, index=99)).to(dev))
    yS = torch.empty((S, N), dtype=torch.float32, device=dev)
    stacked = lambda i: pq.moe_matvec_ternary(stacks[i % len(stacks)], None, gS, xqS, xdS, True,
                                              pq.PQ_EPI_F32, yS)
    R = max(4, min(args.kernel_launches, 32))
    avg_ms = time_launches(stacked, R, not args.no_graph)
    kbytes = S * per_matrix
    ach = kbytes / (avg_ms * 1e-3) / 1e9
    plan = pq.plan(pq.PQ_CALL_MATVEC, "ternary", S, 1, S, N, K)
    traffic = measured_traffic(name, ["k_matvec.hip", "pq_device.hpp", "pq_internal.hpp"])
    roofline = {"bound": "hbm", "kernel": "k_matvec (1024 stacked 1024x1024 matrices per launch, one token each)",
                "achieved": round(ach, 1), "peak": HBM_PEAK_GBS, "unit": "GB/s",
                "frac": round(ach / HBM_PEAK_GBS, 4), "traffic": traffic,
                "avg_launch_us": round(avg_ms * 1e3, 3), "bytes_per_launch": kbytes}
    if peaks:
        roofline["frac_of_measured_read"] = round(ach / peaks["read_gbs"], 4)
    log("  stacked: %.1f us per launch of %d matrices, %.1f GB/s" % (avg_ms * 1e3, S, ach))

    cpu = None
    if args.cpu_seconds > 0:
        import oracle
        done, spent = 0, 0.0
        while spent < args.cpu_seconds and done < P:
            qs = pool.qs[done].cpu().numpy()
            d = pool.d[done].cpu().numpy().view(np.uint16)
            x = xs[done % 64].cpu().numpy()
            t0 = time.perf_counter()
            w = oracle.unpack_ternary(qs, K)
            q, dq = oracle.quantize_q8(x)
            oracle.matvec_q8(w, d, q[0], dq[0], want_isums=False)
            spent += time.perf_counter() - t0
            done += 1
        cpu = {"value": round(done * per_matrix / spent / 1e9, 6), "unit": "GB/s", "cores": oracle.num_threads(),
               "kind": "oracle", "sample": "%d single-matrix calls (unpack, q8, mat-vec), %.1f s" % (done, spent),
               "us_per_call": round(spent / done * 1e6, 1)}
        log("  cpu oracle: %d calls in %.1f s" % (done, spent))
    res = {"workload": name, "format": "ternary", "tokens": 1, "rows": N, "cols": K,
           "matrices_in_pool": P, "matrices_per_stacked_launch": S,
           "steps_per_graph": M if not args.no_graph else 0,
           "step_us": round(ms_step * 1e3, 3), "ms_per_step": round(ms_step, 6), "us_per_call": round(ms_step * 1e3, 3),
           "value": round(gbs, 2), "unit": "GB/s", "dtype": "int8", "packed_gbs": round(gbs, 2),
           "stacked_gbs": round(ach, 1), "hbm_frac_step": round(gbs / HBM_PEAK_GBS, 4),
           "packed_bytes_per_step": per_matrix, "tokens_per_s": round(1.0 / (ms_step * 1e-3), 1),
           "dispatch": {"call": "pq_matvec_x32_ternary (one launch)", "stacked": plan},
           "roofline": roofline, "cpu_baseline": cpu}
    del pool, stacks, runner
    torch.cuda.synchronize()
    torch.cuda.empty_cache()
    return res


def cpu_baseline_layers(args, cfg, layers, xs, lg, n_active, per_expert, L, prefill, q8_prefill):
    """The oracle, as it stands, on whole steps of the same workload until the
    budget is spent (prefill: a fixed sample of assignments per step, time
    scaled to the whole step, the oracle's work being linear in them)."""
    import numpy as np
    import torch

    import oracle
    from oracle import moe

    fmt = cfg["fmt"]
    T, k = cfg["T"], cfg["top_k"]
    done_bytes, done_steps, spent = 0, 0, 0.0
    for l in range(L):
        if spent >= args.cpu_seconds and done_steps > 0:
            break
        logits = lg[l].cpu().numpy()
        ids, _ = oracle.route_topk(logits, k)
        A = T * k
        sub = None
        if prefill or q8_prefill:
            sub = np.linspace(0, A - 1, min(A, 16)).astype(np.int64)
            touched = np.unique(ids.ravel()[sub])
        else:
            touched = np.unique(ids)
        inp = {"cfg": dict(cfg), "logits": logits}
        sel = torch.as_tensor(touched, dtype=torch.long, device=layers[l]["gate"].d.device)
        for name in ("gate", "up", "down"):
            Wt = layers[l][name]
            planes = {}
            for f in ("qs", "qh", "signs", "sc", "d"):
                if not hasattr(Wt, f):
                    continue
                src = getattr(Wt, f)
                host = np.zeros(tuple(src.shape), dtype=np.uint8 if f in ("qs", "signs", "sc") else np.uint16)
                host[touched] = src.index_select(0, sel).cpu().numpy().view(host.dtype)
                planes[f] = untile(host, f) if getattr(Wt, "tiled", False) and f in TILE_PLANES else host
            inp[name] = planes
            if fmt == "grid1":
                inp["grid"] = Wt.grid.cpu().numpy()
        if prefill:
            inp["x_bf16"] = xs[l].cpu().numpy().view(np.uint16)
        else:
            inp["x"] = xs[l].cpu().numpy()
        t0 = time.perf_counter()
        if prefill:
            moe.prefill_ffn(inp, assign_subset=sub)
        else:
            moe.decode_ffn(inp, want_isums=False, assign_subset=sub)
        dt = time.perf_counter() - t0
        spent += dt * (A / len(sub) if sub is not None else 1.0)
        done_bytes += n_active[l] * per_expert
        done_steps += 1
    gbs = done_bytes / spent / 1e9
    log("  cpu oracle: %d steps in %.1f s (scaled), %.4f GB/s, %d threads" % (
        done_steps, spent, gbs, oracle.num_threads()))
    what = ("%d steps, 16 of %d assignments each, time scaled to the whole step" % (done_steps, T * k)
            if (prefill or q8_prefill) else "%d whole steps" % done_steps)
    return {"value": round(gbs, 6), "unit": "GB/s", "cores": oracle.num_threads(), "kind": "oracle",
            "sample": "%s (layers 0..%d of the pool), %.1f s" % (what, done_steps - 1, spent),
            "tokens_per_s": round(done_steps * T / spent, 3)}


def main():
    args = parse()
    if args.copy_calibration:
        copy_calibration()
        return
    if args.gpus != 1:
        print("bench.py runs on one GPU only: this path has no multi-GPU mode "
              "(expert-parallel sharding is a design note only, not built).", file=sys.stderr)
        sys.exit(2)
    import torch
    import workloads as wl

    names = SUITE if args.workload == "all" else [args.workload]
    for n in names:
        if n not in wl.WORKLOADS:
            raise SystemExit("unknown workload %s" % n)
    torch.cuda.set_device(0)
    t_start = time.perf_counter()
    peaks = None if args.no_peaks else measure_peaks()
    results = {}
    for n in names:
        if wl.WORKLOADS[n]["kind"] == "matvec":
            results[n] = bench_single_matrix(n, args, peaks)
        else:
            results[n] = bench_layer_workload(n, args, peaks)
    head_name = HEADLINE if HEADLINE in results else names[-1]
    h = results[head_name]
    config = {k: h[k] for k in ("workload", "format", "tokens", "hidden", "intermediate", "experts", "top_k",
                                "layers_in_pool", "steps_per_graph", "packed_bytes_per_step",
                                "rows", "cols", "matrices_in_pool") if k in h}
    config["parallelism"] = "single GPU"
    out = {
        "metric": METRIC, "value": h["value"], "unit": h["unit"], "n_gpus": 1,
        "steps": args.steps, "warmup": args.warmup, "ms_per_step": h["ms_per_step"],
        "higher_is_better": True, "scaling": "weak", "vs_baseline": None, "dtype": h["dtype"],
        "data": "synthetic", "config": config,
        "tokens_per_s": h["tokens_per_s"], "packed_gbs": h["packed_gbs"],
        "roofline": h["roofline"], "cpu_baseline": h["cpu_baseline"],
        "peaks_measured": peaks,
        "configs": {n: {k: v for k, v in r.items() if k != "workload"} for n, r in results.items()},
        "wall_s": round(time.perf_counter() - t_start, 1),
    }
    print(json.dumps(out), flush=True)


if __name__ == "__main__":
    main()
