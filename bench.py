"""Benchmark of the packed 1-bit-class MoE expert path on one MI355X.

A step is one pass of the whole hot path over one batch of synthetic input:
decode: q8(x) -> top-k route -> group -> fused gate/up mat-vec (SwiGLU + q8)
-> down mat-vec -> weighted combine; prefill: route -> group -> gate/up GEMM
(SwiGLU, bf16 h) -> down GEMM -> combine; q8 prefill: the decode sequence at
2048 tokens, where the mat-vec entry points hand every expert with 8 or more
assignments to the int8-MFMA tile kernel.  Each step uses the weights of a
different layer from a rotating pool sized so that the packed bytes touched
between two visits of a layer exceed the 256 MB last-level cache several
times over: the weights are read from HBM, not from cache.  Steps are
captured in HIP graphs (several layers per graph, as a model's decode step
would be) and replayed.

value: packed weight bytes of the experts touched per step / step time (GB/s).
roofline: the dominant kernel (fused gate/up), its algorithmic bytes (decode)
or operations (prefill) per launch over its average launch time, measured
with HIP events around the launches on the launch stream.
cpu_baseline: the CPU oracle on a bounded sample of the same steps.

Usage: python bench.py [--gpus 1] [--steps K] [--warmup W] [--workload NAME]
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


def parse():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=400)
    ap.add_argument("--warmup", type=int, default=48)
    ap.add_argument("--workload", default="ternary_moe_decode_t1")
    ap.add_argument("--seed", type=int, default=None)
    ap.add_argument("--graph-steps", type=int, default=8, help="layer steps per captured graph")
    ap.add_argument("--kernel-launches", type=int, default=200,
                    help="eager launches of the dominant kernel timed with HIP events")
    ap.add_argument("--cpu-seconds", type=float, default=12.0, help="oracle sample budget (0 = skip)")
    ap.add_argument("--no-graph", action="store_true", help="launch steps eagerly")
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


def main():
    args = parse()
    if args.copy_calibration:
        copy_calibration()
        return
    if args.gpus != 1:
        print("bench.py runs on one GPU only: this path has no multi-GPU mode "
              "(expert-parallel sharding is a design note only, not built).", file=sys.stderr)
        sys.exit(2)

    import numpy as np
    import torch

    import bit_quantized_moe_q8_amd as pq
    from bit_quantized_moe_q8_amd.layer import DecodeLayer, PrefillLayer
    import workloads as wl

    cfg = dict(wl.WORKLOADS[args.workload])
    if cfg["kind"] == "matvec":
        raise SystemExit("the single-matrix workload is a parity case, not a bench line")
    seed = cfg["seed"] if args.seed is None else args.seed
    fmt, T, H, I, E, k = cfg["fmt"], cfg["T"], cfg["H"], cfg["I"], cfg["E"], cfg["top_k"]
    prefill = cfg["kind"] == "prefill"
    q8_prefill = cfg["kind"] == "prefill_q8"
    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)

    per_matrix = wl.packed_bytes_per_matrix(fmt, I, H)      # gate or up ([I][H])
    # down is [H][I]: the same size for per-256 scales, larger by its extra
    # rows' anchors for the sub-scaled signs (one anchor per row)
    per_expert = 2 * per_matrix + wl.packed_bytes_per_matrix(fmt, H, I)
    expect_touched = min(E, T * k)
    touched_est = expect_touched * per_expert
    M = max(1, args.graph_steps)
    L = max(8, int(math.ceil(4 * MALL_BYTES / max(touched_est, 1))))
    L = int(math.ceil(L / M) * M)
    L = min(L, 256)
    log("workload %s: %d layers in the pool (%.2f GB packed), %d steps per graph" % (
        args.workload, L, L * E * per_expert / 1e9, M))

    # ---- rotating pool of packed layers, generated on the device
    gen = torch.Generator(device=dev)
    gen.manual_seed(seed)
    layers = []
    for _ in range(L):
        if fmt == "ternary":
            mk = lambda n, kk: pq.TernaryWeights(**wl.torch_ternary_planes(gen, E, n, kk, dev))
        elif fmt == "sign1":
            mk = lambda n, kk: pq.Sign1Weights(**wl.torch_sign1_planes(gen, E, n, kk, dev))
        else:
            grid = torch.from_numpy(wl.codebook(seed)).to(dev)
            mk = lambda n, kk: pq.Grid1Weights(grid=grid, **wl.torch_grid1_planes(gen, E, n, kk, dev))
        layers.append({"gate": mk(I, H), "up": mk(I, H), "down": mk(H, I)})

    # ---- one input batch per layer (distinct tokens)
    xs, lg = [], []
    for l in range(L):
        if prefill:
            xs.append(torch.from_numpy(wl.activations_bf16(seed, T, H, index=l).view(np.int16)).to(dev))
        else:
            xs.append(torch.from_numpy(wl.activations_f32(seed, T, H, index=l)).to(dev))
        lg.append(torch.from_numpy(wl.router_logits(seed, T, E, cfg["logits"], index=l)).to(dev))

    if prefill:
        layer = PrefillLayer(T, H, I, E, k, dev)
        step = lambda l: layer(xs[l], lg[l], layers[l]["gate"], layers[l]["up"], layers[l]["down"])
    else:
        layer = DecodeLayer(fmt, T, H, I, E, k, dev)
        step = lambda l: layer(xs[l], lg[l], layers[l]["gate"], layers[l]["up"], layers[l]["down"])

    # ---- experts touched per layer input (the library's own routing + grouping)
    n_active = []
    for l in range(L):
        if prefill:
            layer.route(lg[l])
        else:
            layer.route(xs[l], lg[l])
        n_active.append(int(layer.groups.n_active.item()))
    torch.cuda.synchronize()

    K, W = args.steps, args.warmup
    if K % M or W % M or L % M:
        M = math.gcd(math.gcd(K, W if W else K), L)
    n_graph = L // M
    graphs = []
    use_graph = not args.no_graph
    if use_graph:
        for _ in range(2):   # warm the kernels before capture
            step(0)
        torch.cuda.synchronize()
        for j in range(n_graph):
            g = torch.cuda.CUDAGraph()
            with torch.cuda.graph(g):
                for l in range(j * M, (j + 1) * M):
                    step(l)
            graphs.append(g)
        torch.cuda.synchronize()

    def run(nsteps, start):
        if use_graph:
            for i in range(nsteps // M):
                graphs[((start // M) + i) % n_graph].replay()
        else:
            for i in range(nsteps):
                step((start + i) % L)

    run(W, 0)
    torch.cuda.synchronize()
    ev0, ev1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    ev0.record()
    run(K, W)
    ev1.record()
    torch.cuda.synchronize()
    ms_total = ev0.elapsed_time(ev1)
    ms_step = ms_total / K
    step_layers = [((W + i) % L) for i in range(K)]
    bytes_steps = sum(n_active[l] * per_expert for l in step_layers)
    value = bytes_steps / (ms_total * 1e-3) / 1e9
    tokens_s = K * T / (ms_total * 1e-3)
    log("step: %.4f ms, %.1f GB/s packed, %.0f tokens/s" % (ms_step, value, tokens_s))

    # ---- dominant kernel: fused gate/up.  Every layer input gets its own
    # routing buffers; R launches (one per layer, cycling) are captured in one
    # HIP graph like the steps, replayed once to warm up, then timed between
    # two HIP events on the launch stream.  Back to back, a long MFMA-bound
    # launch runs at a lower sustained clock than between the lighter kernels
    # of a step (see the profile summaries).
    R = min(args.kernel_launches, 4 * L) if args.kernel_launches > 0 else 0
    states = []
    for l in range(L):
        st = layer.new_route_state()
        layer.use_state(st)
        if prefill:
            layer.route(lg[l])
        else:
            layer.route(xs[l], lg[l])
        states.append(st)
    torch.cuda.synchronize()

    decode1 = (not prefill) and layer.decode1

    def dominant(i):
        l = i % L
        layer.use_state(states[l])
        if prefill:
            layer.gate_up(xs[l], layers[l]["gate"], layers[l]["up"])
        elif q8_prefill:
            # the int8-MFMA tile alone (the mat-vec entry point adds a launch
            # for the experts under 8 assignments; at 2048 tokens it has none)
            tile = {"ternary": pq.moe_tile_q8_ternary, "grid1": pq.moe_tile_q8_grid1,
                    "sign1": pq.moe_tile_q8_sign1}[fmt]
            tile(layers[l]["gate"], layers[l]["up"], layer.groups, layer.xq, layer.xd, True,
                 pq.PQ_EPI_SWIGLU_Q8, layer.hq, layer.hd)
        elif decode1:
            # one token: the gate/up launch that routes and quantizes itself
            st = states[l]
            pq.moe_decode1_gate_up(layers[l]["gate"], layers[l]["up"], xs[l], lg[l], k, st["ids"],
                                   st["w"], st["groups"], layer.hq, layer.hd, layer.y)
        else:
            layer.gate_up(layers[l]["gate"], layers[l]["up"])

    kbytes = [n_active[i % L] * 2 * per_matrix for i in range(R)]
    kms = []
    if R:
        if use_graph:
            kg = torch.cuda.CUDAGraph()
            with torch.cuda.graph(kg):
                for i in range(R):
                    dominant(i)
            kg.replay()
            torch.cuda.synchronize()
        k0, k1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        torch.cuda._sleep(100_000_000)
        k0.record()
        if use_graph:
            kg.replay()
        else:
            for i in range(R):
                dominant(i)
        k1.record()
        torch.cuda.synchronize()
        kms = [k0.elapsed_time(k1) / R] * R
    roofline = None
    # the mat-vec entry point hands experts with 8+ assignments to the tile
    # kernel when a batch of 8+ tokens has more assignments than experts
    heavy_split = (not prefill and not q8_prefill and not decode1 and T >= 8 and T * k > E)
    kfiles = (["k_gemm.hip"] if prefill else ["k_tile_q8.hip"] if q8_prefill
              else ["k_matvec1.hip"] if decode1
              else ["k_matvec.hip", "k_tile_q8.hip"] if heavy_split else ["k_matvec.hip"])
    srcs = kfiles + ["pq_device.hpp", "pq_internal.hpp"]
    traffic = measured_traffic(args.workload, srcs)
    if R:
        avg_ms = sum(kms) / R
        avg_bytes = sum(kbytes) / R
        if prefill:
            # algorithmic flops of the gate/up GEMM: 2 * A * (2 * I) * H
            flops = 2.0 * T * k * 2 * I * H
            ach = flops / (avg_ms * 1e-3) / 1e12
            roofline = {"bound": "mfma", "kernel": "k_gemm (gate/up, SwiGLU epilogue)",
                        "achieved": round(ach, 2), "peak": BF16_PEAK_TFLOPS, "unit": "TFLOP/s",
                        "frac": round(ach / BF16_PEAK_TFLOPS, 4), "traffic": traffic,
                        "avg_launch_us": round(avg_ms * 1e3, 3), "flop_per_launch": flops}
        elif q8_prefill:
            # algorithmic int8 operations of the gate/up tile: 2 * A * (2 * I) * H
            ops = 2.0 * T * k * 2 * I * H
            ach = ops / (avg_ms * 1e-3) / 1e12
            roofline = {"bound": "mfma", "kernel": "k_tile_q8 (gate/up, int8 MFMA, SwiGLU+q8 epilogue)",
                        "achieved": round(ach, 2), "peak": INT8_PEAK_TOPS, "unit": "TOP/s",
                        "frac": round(ach / INT8_PEAK_TOPS, 4), "traffic": traffic,
                        "avg_launch_us": round(avg_ms * 1e3, 3), "op_per_launch": ops}
        else:
            ach = avg_bytes / (avg_ms * 1e-3) / 1e9
            kname = ("k_matvec_tok1 (one token: routing, q8, gate/up, SwiGLU+q8 epilogue)" if decode1
                     else "k_tile_q8 + k_matvec (gate/up, SwiGLU+q8 epilogue; experts with 8+ "
                          "assignments on the int8-MFMA tile, the rest on the mat-vec)" if heavy_split
                     else "k_matvec (gate/up, SwiGLU+q8 epilogue)")
            roofline = {"bound": "hbm", "kernel": kname,
                        "achieved": round(ach, 1), "peak": HBM_PEAK_GBS, "unit": "GB/s",
                        "frac": round(ach / HBM_PEAK_GBS, 4), "traffic": traffic,
                        "avg_launch_us": round(avg_ms * 1e3, 3),
                        "bytes_per_launch": round(avg_bytes)}
        log("dominant kernel: %.2f us per launch, %s" % (avg_ms * 1e3, roofline["achieved"]))

    # ---- CPU oracle baseline on a bounded sample of the same steps
    cpu = None
    if args.cpu_seconds > 0:
        cpu = cpu_baseline(args, cfg, layers, xs, lg, n_active, per_expert, fmt, prefill, q8_prefill, L, log)

    out = {
        "metric": "decode expert mat-vec GB/s (packed bytes) & % HBM peak; prefill GEMM % MFMA peak",
        "value": round(value, 2), "unit": "GB/s", "n_gpus": 1, "steps": K, "warmup": W,
        "ms_per_step": round(ms_step, 6), "higher_is_better": True, "scaling": "weak",
        "vs_baseline": None, "dtype": "bf16" if prefill else "int8", "data": "synthetic",
        "config": {"workload": args.workload, "format": fmt, "tokens": T, "hidden": H,
                   "intermediate": I, "experts": E, "top_k": k, "layers_in_pool": L,
                   "steps_per_graph": M if use_graph else 0,
                   "packed_bytes_per_step": round(bytes_steps / K),
                   "parallelism": "single GPU"},
        "hbm_frac_step": round(value / HBM_PEAK_GBS, 4),
        "tokens_per_s": round(tokens_s, 1),
        "roofline": roofline,
        "cpu_baseline": cpu,
    }
    print(json.dumps(out), flush=True)


def cpu_baseline(args, cfg, layers, xs, lg, n_active, per_expert, fmt, prefill, q8_prefill, L, log):
    """The oracle, as it stands, on whole steps of the same workload until the budget is spent."""
    import numpy as np

    import oracle
    from oracle import moe

    T, H, I, E, k = cfg["T"], cfg["H"], cfg["I"], cfg["E"], cfg["top_k"]
    done_bytes, done_steps, spent = 0, 0, 0.0
    for l in range(L):
        if spent >= args.cpu_seconds and done_steps > 0:
            break
        logits = lg[l].cpu().numpy()
        ids, _ = oracle.route_topk(logits, k)
        touched = np.unique(ids)
        inp = {"cfg": dict(cfg), "logits": logits}
        for name in ("gate", "up", "down"):
            Wt = layers[l][name]
            planes = {}
            for f in ("qs", "qh", "signs", "sc", "d"):
                if not hasattr(Wt, f):
                    continue
                src = getattr(Wt, f)
                host = np.zeros(tuple(src.shape), dtype=np.uint8 if f in ("qs", "signs", "sc") else np.uint16)
                sel = src[torch_index(touched)].cpu().numpy()
                host[touched] = sel.view(host.dtype)
                planes[f] = host
            inp[name] = planes
            if fmt == "grid1":
                inp["grid"] = Wt.grid.cpu().numpy()
        if prefill:
            inp["x_bf16"] = xs[l].cpu().numpy().view(np.uint16)
        else:
            inp["x"] = xs[l].cpu().numpy()
        if prefill or q8_prefill:
            # a fixed sample of assignments per step; the step time is scaled
            # up by A / sample (the oracle's work is linear in assignments)
            A = T * k
            ns = min(A, 16)
            sub = np.linspace(0, A - 1, ns).astype(np.int64)
            t0 = time.perf_counter()
            if prefill:
                moe.prefill_ffn(inp, assign_subset=sub)
            else:
                moe.decode_ffn(inp, want_isums=False, assign_subset=sub)
            spent += (time.perf_counter() - t0) * (A / ns)
        else:
            t0 = time.perf_counter()
            moe.decode_ffn(inp, want_isums=False)
            spent += time.perf_counter() - t0
        done_bytes += n_active[l] * per_expert
        done_steps += 1
    if done_steps == 0:
        return None
    gbs = done_bytes / spent / 1e9
    log("cpu oracle: %d steps in %.1f s, %.3f GB/s, %d threads" % (done_steps, spent, gbs, oracle.num_threads()))
    what = ("%d steps, 16 of %d assignments each, time scaled to the whole step" % (done_steps, T * k)
            if prefill or q8_prefill else "%d whole steps" % done_steps)
    return {"value": round(gbs, 6), "unit": "GB/s", "cores": oracle.num_threads(), "kind": "oracle",
            "sample": "%s (layers 0..%d of the pool), %.1f s" % (what, done_steps - 1, spent),
            "tokens_per_s": round(done_steps * T / spent, 3)}


def torch_index(idx):
    import torch
    return torch.as_tensor(idx, dtype=torch.long)


if __name__ == "__main__":
    main()
