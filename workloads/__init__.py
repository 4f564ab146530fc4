"""Seeded synthetic inputs for the packed 1-bit-class MoE expert path.

This module only draws random numbers and lays them out in the storage planes
the kernels and the oracle both consume.  It holds none of the method's
arithmetic: no activation quantization, no code decoding, no dot products,
no routing.  Both the HIP path and the CPU oracle take their inputs from here
and from nowhere else.

Storage planes (structure of arrays, one contiguous plane per field):

* ternary: ``qs`` uint8 [E][N][K/4] (4 two-bit codes per byte, weight 4i+j in
  bits 2j..2j+1 of byte i; codes 0, 1, 2), ``d`` uint16 [E][N][K/256]
  (IEEE half bits, one scale per 256-weight row block).
* grid1: ``qs`` uint8 [E][N][K/8] (low 8 bits of each 8-weight group index),
  ``qh`` uint16 [E][N][K/32] (bits 3j..3j+2 hold the high 3 index bits of group
  4i+j; bits 12..15 zero), ``d`` as above; codebook int8 [2048][8].
* sign1 (sub-scaled sign codes): ``signs`` uint8 [E][N][K/8] (bit j of byte i
  is the sign of weight 8i+j, 1 = negative), ``sc`` uint8 [E][N][K/32] (the
  4-bit sub-scales of 16-weight blocks 2i and 2i+1 in the low and high nibble
  of byte i), ``d`` uint16 [E][N] (IEEE half bits, one anchor per row).

The pages (Parakon Runtime README, "How it works"; pxq_llama README, "What's
PXQ?") describe 1-bit-class codebook and ternary expert formats without a byte
layout; the layout above is this library's.

Distributions:

* weight codes i.i.d. uniform over {0, 1, 2} (each weight -1/0/+1 with p=1/3);
  grid indices i.i.d. uniform over [0, 2048); codebook entries i.i.d. uniform
  over {-1, 0, +1};
* weight scales fp32 U(0.005, 0.05) rounded to fp16 (round to nearest even);
  sign1: sign bits i.i.d. fair, sub-scales i.i.d. uniform over 0..15, row
  anchors fp32 U(0.001, 0.006) rounded to fp16;
* decode activations fp32 N(0,1), each entry independently multiplied by 20
  with probability 0.01; prefill activations bf16 = RNE(fp32 N(0,1));
* router logits: fp32 N(0,1), fp32 U(0,1), or Zipf(1.1) with Gumbel noise
  (log p_{pi(e)} + Gumbel(0,1) for a random expert permutation pi, so that the
  top-k of a token's logits is a draw without replacement from Zipf(1.1)).

Every tensor gets its own numpy PCG64 stream from SeedSequence([seed, tag,
index...]); expert weights get one stream per (tensor, expert), so a subset of
experts can be generated without generating the rest.
"""
from __future__ import annotations

import numpy as np

GRID_ENTRIES = 2048
GRID_DIM = 8

# Stable tags for the per-tensor streams.
_TAGS = {
    "x": 1, "logits": 2, "codebook": 3, "zipf_perm": 4,
    "gate": 10, "up": 11, "down": 12, "w": 13,
}

# Workloads: shapes, formats and distributions.
WORKLOADS = {
    # one 1024x1024 ternary matrix, one token
    "ternary_matvec_1024": dict(kind="matvec", fmt="ternary", E=1, N=1024, K=1024,
                                T=1, top_k=1, logits=None, seed=100),
    # ternary MoE FFN decode, 1 token, hidden 2048, intermediate 768, 128 experts, top-8
    "ternary_moe_decode_t1": dict(kind="decode", fmt="ternary", E=128, H=2048, I=768,
                                  T=1, top_k=8, logits="normal", seed=101),
    # grid-codebook MoE FFN decode, 8 tokens, hidden 4096, intermediate 1536, 256 experts
    "grid1_moe_decode_t8": dict(kind="decode", fmt="grid1", E=256, H=4096, I=1536,
                                T=8, top_k=8, logits="uniform", seed=102),
    # batched ternary MoE decode, 64 tokens, 256 experts, Zipf(1.1)-skewed routing
    "ternary_moe_decode_t64_zipf": dict(kind="decode", fmt="ternary", E=256, H=2048, I=768,
                                        T=64, top_k=8, logits="zipf", seed=103),
    # prefill: 2048 tokens through 256 grid-codebook experts, bf16 activations
    "grid1_moe_prefill_t2048": dict(kind="prefill", fmt="grid1", E=256, H=4096, I=1536,
                                    T=2048, top_k=8, logits="uniform", seed=104),
    # sub-scaled sign codes at the 8-token grid1 decode shapes (the cost of
    # the second, per-16 scale against grid1's single per-256 scale)
    "sign1_moe_decode_t8": dict(kind="decode", fmt="sign1", E=256, H=4096, I=1536,
                                T=8, top_k=8, logits="uniform", seed=107),
    # the same 2048-token batches with q8 activations (fp32 x as for decode),
    # for the exact-block-sum int8-MFMA tile path: grid1 with the prefill
    # shapes, ternary with the 64-token decode shapes and uniform routing
    "grid1_moe_prefill_q8_t2048": dict(kind="prefill_q8", fmt="grid1", E=256, H=4096, I=1536,
                                       T=2048, top_k=8, logits="uniform", seed=105),
    "ternary_moe_prefill_q8_t2048": dict(kind="prefill_q8", fmt="ternary", E=256, H=2048, I=768,
                                         T=2048, top_k=8, logits="uniform", seed=106),
    # sub-scaled signs through the bf16 GEMM at the grid1 prefill shapes
    "sign1_moe_prefill_t2048": dict(kind="prefill", fmt="sign1", E=256, H=4096, I=1536,
                                    T=2048, top_k=8, logits="uniform", seed=109),
    # sub-scaled signs through the same tile at the grid1 prefill shapes
    "sign1_moe_prefill_q8_t2048": dict(kind="prefill_q8", fmt="sign1", E=256, H=4096, I=1536,
                                       T=2048, top_k=8, logits="uniform", seed=108),
}

# The 81 byte values whose four 2-bit fields all lie in {0, 1, 2}; a uniform
# draw over them is four i.i.d. uniform codes.
_VALID_TERNARY_BYTES = np.array(
    [b for b in range(256) if all(((b >> (2 * j)) & 3) != 3 for j in range(4))],
    dtype=np.uint8)
assert _VALID_TERNARY_BYTES.size == 81


def rng_for(seed: int, tag: str, *index: int) -> np.random.Generator:
    """Independent PCG64 stream for (seed, tensor tag, index...)."""
    return np.random.Generator(np.random.PCG64(
        np.random.SeedSequence([int(seed), _TAGS[tag]] + [int(i) for i in index])))


def scales_f16(rng: np.random.Generator, shape) -> np.ndarray:
    """fp32 U(0.005, 0.05) rounded to fp16; returned as the uint16 bit pattern."""
    v = rng.uniform(0.005, 0.05, size=shape).astype(np.float32)
    return v.astype(np.float16).view(np.uint16)


def ternary_expert(seed: int, tag: str, e: int, N: int, K: int):
    """Packed ternary planes of one expert matrix [N][K]: (qs [N][K/4], d [N][K/256])."""
    assert K % 256 == 0
    rng = rng_for(seed, tag, e)
    qs = _VALID_TERNARY_BYTES[rng.integers(0, 81, size=(N, K // 4), dtype=np.uint8)]
    d = scales_f16(rng, (N, K // 256))
    return qs, d


def grid1_expert(seed: int, tag: str, e: int, N: int, K: int):
    """Packed grid1 planes of one expert matrix [N][K]: (qs [N][K/8], qh [N][K/32], d)."""
    assert K % 256 == 0
    rng = rng_for(seed, tag, e)
    qs = rng.integers(0, 256, size=(N, K // 8), dtype=np.uint8)
    qh = rng.integers(0, 4096, size=(N, K // 32), dtype=np.uint16)
    d = scales_f16(rng, (N, K // 256))
    return qs, qh, d


def sign1_expert(seed: int, tag: str, e: int, N: int, K: int):
    """Sub-scaled sign planes of one expert matrix [N][K]: (signs [N][K/8], sc [N][K/32], d [N])."""
    assert K % 256 == 0
    rng = rng_for(seed, tag, e)
    signs = rng.integers(0, 256, size=(N, K // 8), dtype=np.uint8)
    sc = rng.integers(0, 256, size=(N, K // 32), dtype=np.uint8)
    d = rng.uniform(0.001, 0.006, size=N).astype(np.float32).astype(np.float16).view(np.uint16)
    return signs, sc, d


def stack_experts(fmt: str, seed: int, tag: str, E: int, N: int, K: int,
                  experts=None) -> dict:
    """All planes of an [E][N][K] expert tensor.

    experts: optional iterable of expert ids to fill; the others stay zero
    (all-zero ternary bytes and grid indices are valid inputs).
    """
    ids = range(E) if experts is None else sorted(set(int(e) for e in experts))
    if fmt == "ternary":
        qs = np.zeros((E, N, K // 4), np.uint8)
        d = np.zeros((E, N, K // 256), np.uint16)
        for e in ids:
            qs[e], d[e] = ternary_expert(seed, tag, e, N, K)
        return dict(qs=qs, d=d)
    if fmt == "grid1":
        qs = np.zeros((E, N, K // 8), np.uint8)
        qh = np.zeros((E, N, K // 32), np.uint16)
        d = np.zeros((E, N, K // 256), np.uint16)
        for e in ids:
            qs[e], qh[e], d[e] = grid1_expert(seed, tag, e, N, K)
        return dict(qs=qs, qh=qh, d=d)
    if fmt == "sign1":
        signs = np.zeros((E, N, K // 8), np.uint8)
        sc = np.zeros((E, N, K // 32), np.uint8)
        d = np.zeros((E, N), np.uint16)
        for e in ids:
            signs[e], sc[e], d[e] = sign1_expert(seed, tag, e, N, K)
        return dict(signs=signs, sc=sc, d=d)
    raise ValueError(fmt)


def codebook(seed: int) -> np.ndarray:
    """2048 x 8 int8 codebook, entries i.i.d. uniform over {-1, 0, +1}."""
    rng = rng_for(seed, "codebook")
    return (rng.integers(0, 3, size=(GRID_ENTRIES, GRID_DIM), dtype=np.int8) - 1).astype(np.int8)


def activations_f32(seed: int, T: int, H: int, outliers: bool = True, index: int = 0) -> np.ndarray:
    """fp32 N(0,1) [T][H]; with outliers, each entry x20 with probability 0.01."""
    rng = rng_for(seed, "x", index)
    x = rng.standard_normal(size=(T, H), dtype=np.float32)
    if outliers:
        x = np.where(rng.random(size=(T, H)) < 0.01, x * np.float32(20.0), x).astype(np.float32)
    return x


def f32_to_bf16_bits(x: np.ndarray) -> np.ndarray:
    """Round finite fp32 to bf16 (nearest, ties to even); uint16 bit pattern."""
    u = np.ascontiguousarray(x, dtype=np.float32).view(np.uint32).astype(np.uint64)
    r = (u + 0x7FFF + ((u >> 16) & 1)) >> 16
    return r.astype(np.uint16)


def activations_bf16(seed: int, T: int, H: int, index: int = 0) -> np.ndarray:
    """bf16 bits [T][H] of RNE(fp32 N(0,1))."""
    rng = rng_for(seed, "x", index)
    return f32_to_bf16_bits(rng.standard_normal(size=(T, H), dtype=np.float32))


def router_logits(seed: int, T: int, E: int, kind: str, index: int = 0) -> np.ndarray:
    """fp32 router logits [T][E]."""
    rng = rng_for(seed, "logits", index)
    if kind == "normal":
        return rng.standard_normal(size=(T, E), dtype=np.float32)
    if kind == "uniform":
        return rng.random(size=(T, E), dtype=np.float32)
    if kind == "zipf":
        perm = rng_for(seed, "zipf_perm", index).permutation(E)
        ranks = np.arange(1, E + 1, dtype=np.float64)
        logp = -1.1 * np.log(ranks)
        logp -= np.log(np.exp(logp).sum())
        gumbel = -np.log(-np.log(rng.random(size=(T, E))))
        return (logp[perm][None, :] + gumbel).astype(np.float32)
    raise ValueError(kind)


def make_workload(name: str, seed: int | None = None, experts="all", **override) -> dict:
    """Inputs of one workload as host numpy arrays.

    experts: "all" fills every expert; "touched" fills only the experts that
    the router logits can select (computed by the caller and passed as a
    list); or an explicit list of expert ids.
    Keyword overrides replace shape fields (for shrunken test shapes).
    """
    cfg = dict(WORKLOADS[name])
    cfg.update(override)
    if seed is None:
        seed = cfg["seed"]
    cfg["seed"] = seed
    fill = None if (isinstance(experts, str) and experts == "all") else experts
    out = dict(cfg=cfg)
    fmt = cfg["fmt"]
    if cfg["kind"] == "matvec":
        out["w"] = stack_experts(fmt, seed, "w", cfg["E"], cfg["N"], cfg["K"], fill)
        out["x"] = activations_f32(seed, cfg["T"], cfg["K"])
        if fmt == "grid1":
            out["grid"] = codebook(seed)
        return out
    E, H, I, T = cfg["E"], cfg["H"], cfg["I"], cfg["T"]
    out["logits"] = router_logits(seed, T, E, cfg["logits"])
    out["gate"] = stack_experts(fmt, seed, "gate", E, I, H, fill)
    out["up"] = stack_experts(fmt, seed, "up", E, I, H, fill)
    out["down"] = stack_experts(fmt, seed, "down", E, H, I, fill)
    if fmt == "grid1":
        out["grid"] = codebook(seed)
    if cfg["kind"] == "prefill":
        out["x_bf16"] = activations_bf16(seed, T, H)
    else:
        out["x"] = activations_f32(seed, T, H)
    return out


def packed_bytes_per_matrix(fmt: str, N: int, K: int) -> int:
    """Packed weight bytes of one [N][K] matrix (codes + indices + scales)."""
    if fmt == "ternary":
        return N * K // 4 + N * (K // 256) * 2
    if fmt == "grid1":
        return N * K // 8 + N * (K // 32) * 2 + N * (K // 256) * 2
    if fmt == "sign1":
        return N * K // 8 + N * (K // 32) + N * 2
    raise ValueError(fmt)


# ---------------------------------------------------------------------------
# Device-side generators for large rotating pools (benchmark only).  Same
# distributions as above, drawn with torch's device RNG.
# ---------------------------------------------------------------------------

def torch_ternary_planes(gen, E: int, N: int, K: int, device):
    import torch
    lut = torch.as_tensor(_VALID_TERNARY_BYTES, device=device)
    qs = lut[torch.randint(0, 81, (E, N, K // 4), generator=gen, device=device)]
    d = torch_scales_f16(gen, (E, N, K // 256), device)
    return dict(qs=qs.contiguous(), d=d)


def torch_grid1_planes(gen, E: int, N: int, K: int, device):
    import torch
    qs = torch.randint(0, 256, (E, N, K // 8), generator=gen, device=device, dtype=torch.int32).to(torch.uint8)
    qh = torch.randint(0, 4096, (E, N, K // 32), generator=gen, device=device, dtype=torch.int32).to(torch.int16)
    d = torch_scales_f16(gen, (E, N, K // 256), device)
    return dict(qs=qs.contiguous(), qh=qh.contiguous(), d=d)


def torch_sign1_planes(gen, E: int, N: int, K: int, device):
    import torch
    signs = torch.randint(0, 256, (E, N, K // 8), generator=gen, device=device, dtype=torch.int32).to(torch.uint8)
    sc = torch.randint(0, 256, (E, N, K // 32), generator=gen, device=device, dtype=torch.int32).to(torch.uint8)
    v = torch.rand((E, N), generator=gen, device=device, dtype=torch.float32) * 0.005 + 0.001
    d = v.to(torch.float16).view(torch.int16).contiguous()
    return dict(signs=signs.contiguous(), sc=sc.contiguous(), d=d)


def torch_scales_f16(gen, shape, device):
    import torch
    v = torch.rand(shape, generator=gen, device=device, dtype=torch.float32) * 0.045 + 0.005
    return v.to(torch.float16).view(torch.int16).contiguous()
