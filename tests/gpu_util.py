"""Helpers shared by the GPU parity tests (HIP path through the C ABI vs the CPU oracle)."""
from __future__ import annotations

import sys

import numpy as np
import torch

import bit_quantized_moe_q8_amd as pq
import oracle
from oracle import moe
import workloads as wl

RTOL = 1e-5   # |got - ref| <= RTOL * sum|terms| + ATOL  (fp32 outputs)
ATOL = 1e-6


def say(*a):
    print(*a, flush=True)
    sys.stdout.flush()


def dev():
    return torch.device("cuda:0")


def to_dev(a: np.ndarray) -> torch.Tensor:
    a = np.ascontiguousarray(a)
    if a.dtype == np.uint16:
        a = a.view(np.int16)
    return torch.from_numpy(a).to(dev())


def to_host(t: torch.Tensor) -> np.ndarray:
    t = t.detach().cpu()
    if t.dtype == torch.bfloat16:
        return t.view(torch.int16).numpy().view(np.uint16)
    return t.numpy()


def assert_tol(got, ref, tsum, what, rtol=RTOL, atol=ATOL):
    got = np.asarray(got, np.float64)
    ok = np.abs(got - ref) <= rtol * np.asarray(tsum) + atol
    if not ok.all():
        bad = np.argwhere(~ok)[:5]
        idx = tuple(bad[0])
        raise AssertionError("%s: %d/%d outside tolerance, first at %s: got %r ref %r tsum %r" % (
            what, int((~ok).sum()), ok.size, idx, got[idx], ref[idx], np.asarray(tsum)[idx]))


def assert_equal(got, ref, what):
    got, ref = np.asarray(got), np.asarray(ref)
    if got.shape != ref.shape or not np.array_equal(got, ref):
        if got.shape != ref.shape:
            raise AssertionError("%s: shape %s vs %s" % (what, got.shape, ref.shape))
        bad = np.argwhere(got != ref)
        raise AssertionError("%s: %d mismatches, first at %s: got %r ref %r" % (
            what, len(bad), tuple(bad[0]), got[tuple(bad[0])], ref[tuple(bad[0])]))


def touched_experts(cfg, logits):
    ids, _ = oracle.route_topk(logits, cfg["top_k"])
    return np.unique(ids)


def decode_inputs(name, **override):
    """Workload inputs with only the experts the router selects filled."""
    cfg = dict(wl.WORKLOADS[name])
    cfg.update(override)
    logits = wl.router_logits(cfg["seed"], cfg["T"], cfg["E"], cfg["logits"])
    return wl.make_workload(name, experts=touched_experts(cfg, logits), **override)


def q8h_check(hq_gpu, hd_gpu, g_ref, u_ref, tg, tu, what="q8(h)"):
    """q8(h) of a GPU path against the oracle's, where the GPU's h was formed
    from its own fp32 g, u (not observable here).  The bounds follow from the
    fp32 tolerance of g and u alone:
      dg = RTOL*tg + ATOL + 2^-24|g|  (the last term: g_ref rounded to fp32),
      dh = 1.1 |u| dg + |silu(g)| du + 1.1 dg du + 0.25 |u| dg^2 + 2^-21 |h|
    (|silu'| <= 1.1, |silu''| <= 0.5; the last term: the GPU's fp32 rounding
    of silu(g) * u), then per 32-block d = max|h| / 127 moves by at most
      dd = max(dh) / 127 + 2^-23 d,
    and a code q = round(h / d) can differ from the oracle's only where h / d
    lies within  dh / d + |h| dd / d^2 + 2^-22 |h / d|  of a rounding boundary
    (there it may move by one).  Checks hd within dd and the codes under that
    rule; everything else must be bit-exact."""
    g = np.asarray(g_ref, np.float64)
    u = np.asarray(u_ref, np.float64)
    g32, u32 = g.astype(np.float32), u.astype(np.float32)
    h = oracle.swiglu(g32, u32)
    hq_ref, hd_ref = oracle.quantize_q8(h.astype(np.float32))
    eps = 2.0 ** -24
    dg = RTOL * np.asarray(tg) + ATOL + eps * np.abs(g)
    du = RTOL * np.asarray(tu) + ATOL + eps * np.abs(u)
    sig = 1.0 / (1.0 + np.exp(-g))
    dh = 1.1 * np.abs(u) * dg + np.abs(g * sig) * du + 1.1 * dg * du + 0.25 * np.abs(u) * dg ** 2 + 8 * eps * np.abs(h)
    shp = h.shape[:-1] + (h.shape[-1] // 32, 32)
    dd = dh.reshape(shp).max(-1) / 127.0 + 2 * eps * hd_ref
    bad_d = np.abs(np.asarray(hd_gpu, np.float64) - hd_ref) > dd
    if bad_d.any():
        i = tuple(np.argwhere(bad_d)[0])
        raise AssertionError("%s: %d block scales outside the derived bound, first at %s: got %r ref %r bound %r" % (
            what, int(bad_d.sum()), i, hd_gpu[i], hd_ref[i], dd[i]))
    d = np.repeat(hd_ref, 32, axis=-1)
    ddf = np.repeat(dd, 32, axis=-1)
    safe = np.where(d == 0, 1.0, d)
    v = h / safe
    delta = dh / safe + np.abs(h) * ddf / safe ** 2 + 4 * eps * np.abs(v)
    near = np.abs(np.abs(v) - np.floor(np.abs(v)) - 0.5) <= delta
    hq_gpu = np.asarray(hq_gpu)
    diff = hq_gpu.astype(np.int32) - hq_ref.astype(np.int32)
    ok = (diff == 0) | (near & (np.abs(diff) <= 1))
    if not ok.all():
        i = tuple(np.argwhere(~ok)[0])
        raise AssertionError("%s: %d of %d codes differ away from a rounding boundary, first at %s: got %d ref %d" % (
            what, int((~ok).sum()), ok.size, i, hq_gpu[i], hq_ref[i]))
    return int((diff != 0).sum())


_PLAN_NAMES = {pq.PQ_PLAN_MATVEC: "matvec", pq.PQ_PLAN_MATVEC_PAIRS: "matvec-pairs",
               pq.PQ_PLAN_MATVEC_TOK1: "matvec-tok1", pq.PQ_PLAN_TILE_Q8: "tile-q8",
               pq.PQ_PLAN_GEMM: "gemm", pq.PQ_PLAN_DECODE1_ROUTED: "decode1-routed",
               pq.PQ_PLAN_DEBUG: "debug", pq.PQ_PLAN_MIXED: "mixed"}


def plan_str(flags):
    if flags <= 0:
        return "status %d" % -flags
    return "+".join(n for f, n in _PLAN_NAMES.items() if flags & f) or "nothing"


def assert_plan(want, call, fmt, T, k, E, rows, cols, epi=0, debug=False):
    """The kernels the entry point dispatches to for these sizes are the ones
    the test means to check (a silently different kernel would otherwise pass
    the parity check in its place)."""
    got = pq.plan(call, fmt, T, k, E, rows, cols, epi, debug)
    assert got == want, "dispatch: the call launches %s, the test checks %s" % (plan_str(got), plan_str(want))
