"""Pins of the CPU oracle against things other than itself.

Each oracle function is checked against hand-derived fixtures (tests/golden),
closed forms, invariants, numpy/scipy/torch library routines, or brute force,
chosen so that a dropped term, a wrong sign or index, or a transposed operand
fails at least one test.
"""
import json
import os

import numpy as np
import pytest
import scipy.special

import oracle
from oracle import moe
import workloads as wl

from conftest import GOLDEN


def _load(name):
    with open(os.path.join(GOLDEN, name)) as f:
        return json.load(f)


def _codes_numpy(qs, K):
    """Independent numpy extraction of ternary 2-bit codes, [N][K]."""
    qs = np.asarray(qs, np.uint8)
    sh = np.array([0, 2, 4, 6], np.uint8)
    return ((qs[..., None] >> sh) & 3).reshape(qs.shape[0], K)


def _deq_scales(d16, K):
    return np.repeat(np.asarray(d16, np.uint16).view(np.float16).astype(np.float64), 256, axis=-1)


# ----------------------------------------------------------------- scalars

def test_half_to_float_all_patterns():
    # every fp16 bit pattern against numpy's float16 (library conversion)
    pats = np.arange(65536, dtype=np.uint32).astype(np.uint16)
    ref = pats.view(np.float16).astype(np.float64)
    got = oracle.halves_to_f64(pats)
    nan = np.isnan(ref)
    assert np.array_equal(np.isnan(got), nan)
    assert np.array_equal(got[~nan], ref[~nan])


def test_bf16_roundtrip_and_rne_vs_torch():
    import torch
    rng = np.random.default_rng(0)
    x = np.concatenate([rng.standard_normal(20000).astype(np.float32),
                        np.float32([0.0, -0.0, 1.0, -1.0, 3.0e38, 1e-40, 1.00390625, 1.01171875])])
    # exact ties: 1 + 2^-8 (tie, even -> 1.0) and 1 + 3*2^-8 (tie, odd -> round up)
    ref = torch.from_numpy(x).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    got = oracle.float_to_bf16(x)
    assert np.array_equal(got, ref)
    back = np.array([oracle.bf16_to_float(b) for b in got[:100]], np.float32)
    assert np.array_equal(back, torch.from_numpy(ref[:100].view(np.int16)).view(torch.bfloat16).float().numpy())
    assert oracle.float_to_bf16(np.float32([1.00390625]))[0] == 0x3F80
    assert oracle.float_to_bf16(np.float32([1.01171875]))[0] == 0x3F82


# --------------------------------------------------------------------- q8

def test_q8_golden_blocks():
    for case in _load("q8_cases.json")["cases"]:
        x = np.zeros(32, np.float32)
        x[: len(case["x"])] = case["x"]
        q, d = oracle.quantize_q8(x)
        want = np.zeros(32, np.int8)
        want[: len(case["q"])] = case["q"]
        assert np.array_equal(q[0], want), case["name"]
        assert d[0, 0] == np.float32(case["d"]), case["name"]


def test_q8_invariants_random():
    x = wl.activations_f32(7, 16, 4096)
    q, d = oracle.quantize_q8(x)
    xb = x.reshape(16, -1, 32)
    qb = q.reshape(16, -1, 32).astype(np.int32)
    db = d.reshape(16, -1, 1).astype(np.float64)
    assert np.abs(qb).max() <= 127
    # the element of largest magnitude maps to +-127 with its sign
    am = np.abs(xb).argmax(axis=-1)
    top_q = np.take_along_axis(qb, am[..., None], -1)[..., 0]
    top_x = np.take_along_axis(xb, am[..., None], -1)[..., 0]
    assert np.array_equal(top_q, np.sign(top_x).astype(np.int32) * 127)
    # reconstruction error at most half a step (plus the two fp32 roundings)
    err = np.abs(xb.astype(np.float64) - qb * db)
    assert np.all(err <= db * (0.5 + 2.0 ** -16))
    # scale is the fp32 quotient max|x| / 127
    amax = np.abs(xb).max(axis=-1)
    assert np.array_equal(d, (amax / np.float32(127)).astype(np.float32))


def test_q8_against_numpy_definition():
    # same definition through numpy's correctly rounded fp32 division and an
    # exact half-away rounding done in fp64
    x = wl.activations_f32(8, 4, 2048)
    q, d = oracle.quantize_q8(x)
    xb = x.reshape(4, -1, 32)
    dd = (np.abs(xb).max(-1) / np.float32(127)).astype(np.float32)
    with np.errstate(divide="ignore", invalid="ignore"):
        v = (xb / dd[..., None]).astype(np.float32).astype(np.float64)
    r = np.trunc(v + np.copysign(0.5, v))
    r = np.where(dd[..., None] == 0, 0, np.clip(r, -127, 127))
    assert np.array_equal(q.reshape(4, -1, 32), r.astype(np.int8))


def test_q8_rejects_nonfinite():
    x = np.zeros(32, np.float32)
    x[3] = np.inf
    with pytest.raises(oracle.OracleError):
        oracle.quantize_q8(x)


# ----------------------------------------------------------------- unpack

def test_ternary_golden_bytes():
    g = _load("ternary_bytes.json")
    for case in g["cases"]:
        w = oracle.unpack_ternary(np.array([[case["byte"]] * 64], np.uint8), 256)
        assert list(w[0, :4]) == case["w"], case
    for b in g["invalid_bytes"]:
        with pytest.raises(oracle.OracleError):
            oracle.unpack_ternary(np.array([[b] * 64], np.uint8), 256)


def test_ternary_all_81_valid_bytes_exhaustive():
    # every byte whose four fields avoid 3 decodes to base-3 digits (value = digit - 3*(digit==2))
    for b in range(256):
        fields = [(b >> (2 * j)) & 3 for j in range(4)]
        arr = np.full((1, 64), b, np.uint8)
        if 3 in fields:
            with pytest.raises(oracle.OracleError):
                oracle.unpack_ternary(arr, 256)
            continue
        w = oracle.unpack_ternary(arr, 256)
        assert list(w[0, :4]) == [{0: 0, 1: 1, 2: -1}[f] for f in fields]


def test_ternary_invalid_count_brute_force():
    # per byte: the number of its four 2-bit fields that equal 3, summed
    rng = np.random.default_rng(17)
    qs = rng.integers(0, 256, size=(3, 64), dtype=np.uint8)
    want = sum(((int(b) >> (2 * j)) & 3) == 3 for b in qs.ravel() for j in range(4))
    assert oracle.count_invalid_ternary(qs, 256) == want
    assert oracle.count_invalid_ternary(np.full((2, 64), 0xFF, np.uint8), 256) == 512
    assert oracle.count_invalid_ternary(np.full((2, 64), 0x0F, np.uint8), 256) == 256
    assert oracle.count_invalid_ternary(wl.ternary_expert(3, "w", 0, 8, 256)[0], 256) == 0


def test_ternary_unpack_vs_numpy_codes():
    qs, _ = wl.ternary_expert(3, "w", 0, 64, 1024)
    w = oracle.unpack_ternary(qs, 1024)
    c = _codes_numpy(qs, 1024).astype(np.int8)
    assert np.array_equal(w, np.where(c == 2, -1, c).astype(np.int8))


def _base3_codebook():
    # entry i: 8 base-3 digits of i, minus 1 -> unique {-1,0,1} vector per index
    idx = np.arange(2048)
    digits = (idx[:, None] // (3 ** np.arange(8))[None, :]) % 3
    return (digits - 1).astype(np.int8)


def test_grid1_golden_indices():
    g = _load("grid1_block.json")
    grid = _base3_codebook()
    qs = np.zeros((1, 32), np.uint8)
    qh = np.zeros((1, 8), np.uint16)
    qs[0, :8] = g["qs"]
    qh[0, :2] = g["qh"]
    w = oracle.unpack_grid1(qs, qh, grid, 256)
    for gi, idx in enumerate(g["idx"]):
        assert np.array_equal(w[0, 8 * gi: 8 * gi + 8], grid[idx]), gi
    # groups 8..31 have index 0
    assert np.array_equal(w[0, 64:].reshape(24, 8), np.repeat(grid[:1], 24, axis=0))


def test_grid1_exhaustive_index_positions():
    # every 11-bit index at every group position of a qh word, across two blocks
    grid = _base3_codebook()
    for pos in range(4):
        for blk in range(2):
            idx = np.arange(2048)
            qs = np.zeros((2048, 64), np.uint8)
            qh = np.zeros((2048, 16), np.uint16)
            g = 4 + pos  # group 4..7 -> qh word 1 of the block
            qs[:, 32 * blk + g] = idx & 0xFF
            qh[:, 8 * blk + 1] = ((idx >> 8) << (3 * pos)) | 0xF000
            w = oracle.unpack_grid1(qs, qh, grid, 512)
            assert np.array_equal(w[:, 256 * blk + 8 * g: 256 * blk + 8 * g + 8], grid[idx])


def test_sign1_golden_rows():
    g = _load("sign1_rows.json")
    for row in g["rows"]:
        w = oracle.unpack_sign1(np.array([row["signs"]], np.uint8), np.array([row["sc"]], np.uint8), 32)
        assert list(w[0]) == row["w"], row


def test_sign1_exhaustive_bytes():
    # every sign byte at every byte position of a 32-weight block, against
    # numpy's little-endian bit unpacking; every sub-scale byte likewise
    for pos in range(4):
        signs = np.zeros((256, 8), np.uint8)
        signs[:, 4 + pos] = np.arange(256)                   # second 32-block of a 64-weight row
        sc = np.full((256, 2), 0x57, np.uint8)               # 7 for weights 0..15 of a block, 5 for 16..31
        w = oracle.unpack_sign1(signs, sc, 64)
        bits = np.unpackbits(np.arange(256, dtype=np.uint8)[:, None], axis=1, bitorder="little")
        mag = 7 if pos < 2 else 5
        assert np.array_equal(w[:, 32 + 8 * pos: 40 + 8 * pos], np.where(bits == 1, -mag, mag))
        assert np.array_equal(w[:, :32], np.where(np.arange(32) < 16, 7, 5)[None, :].repeat(256, 0))
    sc = np.arange(256, dtype=np.uint8)[:, None]
    w = oracle.unpack_sign1(np.zeros((256, 4), np.uint8), sc, 32)
    assert np.array_equal(w[:, 0], np.arange(256) & 15) and np.array_equal(w[:, 31], np.arange(256) >> 4)
    assert np.abs(oracle.unpack_sign1(np.full((4, 32), 255, np.uint8), np.full((4, 8), 255, np.uint8), 256)).max() == 15


def test_sign1_matvec_closed_forms_and_dequant():
    K = 512
    rng = np.random.default_rng(21)
    xq, xd = oracle.quantize_q8(wl.activations_f32(21, 1, K))
    x = xq[0].astype(np.float64) * np.repeat(xd[0].astype(np.float64), 32)
    one = np.full((3, K // 256), 0x3C00, np.uint16)          # anchor 1.0 in every block
    # all signs positive, sub-scale 15: y = 15 * sum(xq * xd); all negative: the negation; sub-scale 0: 0
    for sgn, scb, want in ((0, 0xFF, 15 * x.sum()), (255, 0xFF, -15 * x.sum()), (0x5A, 0x00, 0.0)):
        w = oracle.unpack_sign1(np.full((3, K // 8), sgn, np.uint8), np.full((3, K // 32), scb, np.uint8), K)
        y, t, _ = oracle.matvec_q8(w, one, xq[0], xd[0])
        assert np.allclose(y, want, rtol=1e-12, atol=1e-12)
    # random planes through the MoE helper against a numpy dequantization with the row anchors
    planes = wl.stack_experts("sign1", 21, "w", 2, 40, K)
    ids = np.array([[1]], np.int32)
    y, t, _ = moe.grouped_matvec_q8("sign1", planes, None, ids, xq, xd, np.array([0]), K)
    W = oracle.unpack_sign1(planes["signs"][1], planes["sc"][1], K).astype(np.float64)
    Wd = W * planes["d"][1].view(np.float16).astype(np.float64)[:, None]
    assert np.all(np.abs(y[0] - Wd @ x) <= 1e-12 * t[0] + 1e-300)


def test_packed_sizes_and_bpw():
    # sub-scaled signs: 1 + 4/16 bits per weight plus one fp16 per row
    assert abs(wl.packed_bytes_per_matrix("sign1", 768, 2048) * 8 / (768 * 2048) - 1.26) < 0.005
    assert wl.packed_bytes_per_matrix("ternary", 1024, 1024) == 270336
    assert wl.packed_bytes_per_matrix("ternary", 768, 2048) == 405504
    assert wl.packed_bytes_per_matrix("grid1", 1536, 4096) == 1228800
    assert wl.packed_bytes_per_matrix("ternary", 256, 256) * 8 / (256 * 256) == 2.0625
    assert wl.packed_bytes_per_matrix("grid1", 256, 256) * 8 / (256 * 256) == 1.5625


def test_generator_distributions():
    qs, d = wl.ternary_expert(5, "w", 0, 512, 2048)
    c = _codes_numpy(qs, 2048)
    assert c.max() <= 2
    frac = np.bincount(c.ravel(), minlength=3) / c.size
    assert np.all(np.abs(frac - 1 / 3) < 0.01)
    dv = d.view(np.float16).astype(np.float64)
    assert dv.min() >= 0.00499 and dv.max() <= 0.0501
    grid = wl.codebook(5)
    assert set(np.unique(grid)) == {-1, 0, 1}
    qs, qh, _ = wl.grid1_expert(5, "w", 0, 64, 4096)
    assert int(qh.max()) < 4096


# ----------------------------------------------------------------- mat-vec

def _numpy_matvec(w_int8, d16, xq, xd):
    """Textbook dequantize-then-matmul in fp64 (numpy BLAS)."""
    K = w_int8.shape[1]
    Wd = w_int8.astype(np.float64) * _deq_scales(d16, K)
    xdq = xq.astype(np.float64) * np.repeat(xd.astype(np.float64), 32)
    return Wd @ xdq


@pytest.mark.parametrize("K", [256, 768, 2048])
def test_matvec_q8_vs_numpy_dequant(K):
    qs, d = wl.ternary_expert(11, "w", 0, 96, K)
    w = oracle.unpack_ternary(qs, K)
    xq, xd = oracle.quantize_q8(wl.activations_f32(11, 1, K))
    y, t, isums = oracle.matvec_q8(w, d, xq[0], xd[0])
    ref = _numpy_matvec(w, d, xq[0], xd[0])
    assert np.all(np.abs(y - ref) <= 1e-12 * t + 1e-300)
    # tsum is at least |y| and equals it when all terms have one sign
    assert np.all(t >= np.abs(y) * (1 - 1e-12))
    # tsum exactly: the sum of |d_w * xd * isum| over the 32-weight blocks,
    # with the block sums from a numpy brute force (an over-estimate such as
    # |.| inside the block sum, or a dropped scale, fails here)
    assert np.allclose(t, _numpy_term_sums(w, d, xq[0], xd[0]), rtol=1e-12, atol=0)


def _numpy_term_sums(w_int8, d16, xq, xd):
    K = w_int8.shape[1]
    isum = (w_int8.astype(np.int64).reshape(w_int8.shape[0], K // 32, 32) *
            xq.astype(np.int64).reshape(1, K // 32, 32)).sum(-1)
    dw = np.repeat(np.asarray(d16, np.uint16).view(np.float16).astype(np.float64), 8, axis=-1)
    return np.abs(dw * xd.astype(np.float64)[None, :] * isum).sum(-1)


def test_matvec_q8_term_sums_distinguish_overestimates():
    """A case where |isum| < sum|w*q| inside a block: the pinned term sum
    is the smaller value, so the tolerance is not silently loosened."""
    K = 256
    w = np.zeros((1, K), np.int8)
    w[0, :2] = [1, -1]
    xq = np.zeros(K, np.int8)
    xq[:2] = [5, 5]                        # isum of block 0 = 0, sum|w*q| = 10
    xq[32:34] = [3, 4]
    w[0, 32:34] = [1, 1]                   # isum of block 1 = 7
    xd = np.full(K // 32, 0.5, np.float32)
    d16 = np.full((1, 1), 0x4000, np.uint16)   # 2.0
    y, t, isums = oracle.matvec_q8(w, d16, xq, xd)
    assert isums[0, 0] == 0 and isums[0, 1] == 7
    assert y[0] == 7.0 and t[0] == 7.0


def test_isums_three_formulas_and_brute_force():
    K = 512
    qs, d = wl.ternary_expert(12, "w", 0, 32, K)
    w = oracle.unpack_ternary(qs, K)
    xq, xd = oracle.quantize_q8(wl.activations_f32(12, 1, K))
    _, _, isums = oracle.matvec_q8(w, d, xq[0], xd[0])
    q = xq[0].astype(np.int64).reshape(-1, 32)
    wb = w.astype(np.int64).reshape(32, -1, 32)
    a = (wb * q[None]).sum(-1)
    b = np.where(wb == 1, q[None], 0).sum(-1) - np.where(wb == -1, q[None], 0).sum(-1)
    c = _codes_numpy(qs, K).astype(np.int64).reshape(32, -1, 32)
    c3 = (c * q[None]).sum(-1) - 3 * ((c >> 1) * q[None]).sum(-1)
    assert np.array_equal(isums, a) and np.array_equal(a, b) and np.array_equal(a, c3)
    assert np.abs(isums).max() <= 32 * 127


def test_matvec_closed_forms():
    K = 256
    one = np.full((K, K // 256), 0x3C00, np.uint16)  # fp16 1.0
    xq, xd = oracle.quantize_q8(wl.activations_f32(13, 1, K))
    # identity weights, scale 1: y = dequantized x
    eye = np.eye(K, dtype=np.int8)
    y, _, _ = oracle.matvec_q8(eye, one, xq[0], xd[0])
    assert np.array_equal(y, xq[0].astype(np.float64) * np.repeat(xd[0].astype(np.float64), 32))
    # all +1 -> per-32 sums of q; all -1 -> negated; all 0 -> 0
    for val in (1, -1, 0):
        w = np.full((4, K), val, np.int8)
        _, _, isums = oracle.matvec_q8(w, one[:4], xq[0], xd[0])
        assert np.array_equal(isums[0], val * xq[0].astype(np.int32).reshape(-1, 32).sum(-1))
    # scale enters linearly: scale 2.0 doubles y exactly
    two = np.full((8, 1), 0x4000, np.uint16)
    w = oracle.unpack_ternary(wl.ternary_expert(13, "w", 0, 8, K)[0], K)
    y1, _, _ = oracle.matvec_q8(w, one[:8], xq[0], xd[0])
    y2, _, _ = oracle.matvec_q8(w, two, xq[0], xd[0])
    assert np.array_equal(y2, 2 * y1)
    # a scale in one block only touches that block: per-block additivity
    K2 = 512
    w2 = oracle.unpack_ternary(wl.ternary_expert(14, "w", 0, 8, K2)[0], K2)
    xq2, xd2 = oracle.quantize_q8(wl.activations_f32(14, 1, K2))
    d_a = np.tile(np.uint16([0x3C00, 0]), (8, 1))
    d_b = np.tile(np.uint16([0, 0x3C00]), (8, 1))
    d_ab = np.tile(np.uint16([0x3C00, 0x3C00]), (8, 1))
    ya, _, _ = oracle.matvec_q8(w2, d_a, xq2[0], xd2[0])
    yb, _, _ = oracle.matvec_q8(w2, d_b, xq2[0], xd2[0])
    yab, _, _ = oracle.matvec_q8(w2, d_ab, xq2[0], xd2[0])
    assert np.allclose(ya + yb, yab, rtol=1e-14, atol=0)


def test_grid1_matvec_row_sums():
    # every index points at an all-ones entry -> y = scale * sum of dequantized x
    K = 512
    grid = np.zeros((2048, 8), np.int8)
    grid[:] = 1
    qs, qh, d = wl.grid1_expert(15, "w", 0, 16, K)
    w = oracle.unpack_grid1(qs, qh, grid, K)
    xq, xd = oracle.quantize_q8(wl.activations_f32(15, 1, K))
    y, _, _ = oracle.matvec_q8(w, d, xq[0], xd[0])
    xdq = xq[0].astype(np.float64) * np.repeat(xd[0].astype(np.float64), 32)
    ref = (_deq_scales(d, K) * xdq[None]).sum(-1)
    assert np.allclose(y, ref, rtol=1e-12, atol=0)


def test_matvec_bf16_vs_numpy():
    K = 1024
    grid = wl.codebook(16)
    qs, qh, d = wl.grid1_expert(16, "w", 0, 64, K)
    w = oracle.unpack_grid1(qs, qh, grid, K)
    xb = wl.activations_bf16(16, 1, K)[0]
    y, t = oracle.matvec_bf16(w, d, xb)
    xf = (xb.astype(np.uint32) << 16).view(np.float32).astype(np.float64)
    ref = (w.astype(np.float64) * _deq_scales(d, K)) @ xf
    assert np.all(np.abs(y - ref) <= 1e-12 * t)
    tref = (np.abs(w.astype(np.float64)) * _deq_scales(d, K)) @ np.abs(xf)
    assert np.allclose(t, tref, rtol=1e-12)


def test_sign1_matvec_bf16_vs_numpy_dequant():
    """The bf16 prefill oracle path on sub-scaled signs (the reference of the
    sign1 GEMM): grouped_matvec_bf16 against sign * sc * anchor @ x in fp64,
    and its term sums against |w| @ |x|."""
    K, N = 1024, 24
    planes = wl.stack_experts("sign1", 33, "w", 3, N, K)
    xb = wl.activations_bf16(33, 2, K)
    ids = np.array([[2, 0]], np.int32)
    y, t = moe.grouped_matvec_bf16("sign1", planes, None, ids, xb, np.array([0, 1]), K)
    for a, e in enumerate(ids.ravel()):
        W = oracle.unpack_sign1(planes["signs"][e], planes["sc"][e], K).astype(np.float64)
        Wd = W * planes["d"][e].view(np.float16).astype(np.float64)[:, None]
        xf = (xb[a].astype(np.uint32) << 16).view(np.float32).astype(np.float64)
        assert np.all(np.abs(y[a] - Wd @ xf) <= 1e-12 * t[a] + 1e-300)
        assert np.allclose(t[a], np.abs(Wd) @ np.abs(xf), rtol=1e-12)


def test_matvec_thread_count_determinism():
    K = 2048
    qs, d = wl.ternary_expert(17, "w", 0, 768, K)
    w = oracle.unpack_ternary(qs, K)
    xq, xd = oracle.quantize_q8(wl.activations_f32(17, 1, K))
    oracle.set_num_threads(1)
    y1, t1, i1 = oracle.matvec_q8(w, d, xq[0], xd[0])
    oracle.set_num_threads(8)
    y8, t8, i8 = oracle.matvec_q8(w, d, xq[0], xd[0])
    assert y1.tobytes() == y8.tobytes() and t1.tobytes() == t8.tobytes() and i1.tobytes() == i8.tobytes()


# ----------------------------------------------------------------- routing

@pytest.mark.parametrize("kind,E,k", [("normal", 128, 8), ("uniform", 256, 8), ("zipf", 256, 8), ("normal", 16, 1)])
def test_route_vs_numpy_stable_argsort(kind, E, k):
    logits = wl.router_logits(21, 64, E, kind)
    ids, w = oracle.route_topk(logits, k)
    ref_ids = np.argsort(-logits.astype(np.float64), axis=1, kind="stable")[:, :k]
    assert np.array_equal(ids, ref_ids)
    sel = np.take_along_axis(logits.astype(np.float64), ref_ids, 1)
    assert np.allclose(w, scipy.special.softmax(sel, axis=1), rtol=1e-13, atol=0)
    assert np.allclose(w.sum(1), 1.0, rtol=0, atol=1e-12)


def test_route_closed_forms_and_ties():
    E = 32
    ids, w = oracle.route_topk(np.arange(E, dtype=np.float32)[None], 8)
    assert list(ids[0]) == list(range(E - 1, E - 9, -1))
    ref = np.exp(np.arange(7, -1, -1, dtype=np.float64))
    assert np.allclose(w[0], ref / ref.sum(), rtol=1e-14)
    # all equal: lower index first, uniform weights
    ids, w = oracle.route_topk(np.zeros((1, E), np.float32), 8)
    assert list(ids[0]) == list(range(8)) and np.allclose(w, 1 / 8)
    # duplicated maxima straddling the cut
    l = np.zeros((1, 16), np.float32)
    l[0, [3, 9, 12]] = 5.0
    ids, _ = oracle.route_topk(l, 2)
    assert list(ids[0]) == [3, 9]


def test_zipf_logits_are_skewed():
    logits = wl.router_logits(103, 64, 256, "zipf")
    ids, _ = oracle.route_topk(logits, 8)
    counts = np.bincount(ids.ravel(), minlength=256)
    assert counts.max() >= 30 and (counts > 0).sum() > 80


# ---------------------------------------------------------------- grouping

@pytest.mark.parametrize("T,E", [(1, 128), (8, 256), (64, 256), (2048, 256), (5, 3)])
def test_group_vs_numpy(T, E):
    logits = wl.router_logits(31, T, E, "zipf" if E == 256 else "normal")
    ids, _ = oracle.route_topk(logits, min(8, E))
    offsets, srt, active = oracle.group(ids, E)
    flat = ids.ravel()
    assert np.array_equal(srt, np.argsort(flat, kind="stable"))
    assert np.array_equal(offsets, np.concatenate([[0], np.cumsum(np.bincount(flat, minlength=E))]))
    assert np.array_equal(active, np.nonzero(np.bincount(flat, minlength=E))[0])
    # invariants: permutation, increasing inside each segment, right expert
    assert np.array_equal(np.sort(srt), np.arange(flat.size))
    for e in range(E):
        seg = srt[offsets[e]: offsets[e + 1]]
        assert np.all(np.diff(seg) > 0) and np.all(flat[seg] == e)


# ------------------------------------------------------------------ swiglu

def test_swiglu():
    g = np.float32([0.0, 1.0, -1.0, 30.0, -30.0, 2.5, -100.0])
    u = np.float32([3.0, 2.0, 2.0, 1.5, 1.5, -1.0, 4.0])
    h = oracle.swiglu(g, u)
    ref = g.astype(np.float64) * scipy.special.expit(g.astype(np.float64)) * u
    assert np.allclose(h, ref, rtol=1e-14, atol=0)
    assert h[0] == 0.0
    assert abs(h[3] - 45.0) < 1e-10  # silu(z) -> z for large z


def test_combine_vs_numpy():
    rng = np.random.default_rng(3)
    out = rng.standard_normal((5 * 4, 33)).astype(np.float32)
    w = rng.random((5, 4)).astype(np.float32)
    y, ty = oracle.combine(out, w, 4)
    ref = np.einsum("tj,tjn->tn", w.astype(np.float64), out.reshape(5, 4, 33).astype(np.float64))
    assert np.allclose(y, ref, rtol=1e-14, atol=1e-15)
    assert np.all(ty >= np.abs(y) - 1e-12)
    # ty exactly: sum over the slots of |w * out| (numpy)
    tref = np.einsum("tj,tjn->tn", np.abs(w.astype(np.float64)),
                     np.abs(out.reshape(5, 4, 33).astype(np.float64)))
    assert np.allclose(ty, tref, rtol=1e-14, atol=0)
    # opposite signs cancel in y but not in ty
    y2, ty2 = oracle.combine(np.float32([[2.0], [-2.0]]), np.float32([[0.5, 0.5]]), 2)
    assert y2[0, 0] == 0.0 and ty2[0, 0] == 2.0


# ------------------------------------------------------------------- MoE

def test_moe_topk1_single_expert_is_dense_swiglu_mlp():
    # E = 1, k = 1: the layer reduces to a dense SwiGLU MLP through one expert
    inp = wl.make_workload("ternary_moe_decode_t1", E=1, H=512, I=256, T=3, top_k=1)
    r = moe.decode_ffn(inp)
    assert np.all(r["ids"] == 0) and np.all(r["w"] == 1.0)
    xdq = r["xq"].astype(np.float64) * np.repeat(r["xd"].astype(np.float64), 32, axis=1)
    Wg = oracle.unpack_ternary(inp["gate"]["qs"][0], 512) * _deq_scales(inp["gate"]["d"][0], 512)
    Wu = oracle.unpack_ternary(inp["up"]["qs"][0], 512) * _deq_scales(inp["up"]["d"][0], 512)
    Wd = oracle.unpack_ternary(inp["down"]["qs"][0], 256) * _deq_scales(inp["down"]["d"][0], 256)
    g, u = xdq @ Wg.T, xdq @ Wu.T
    assert np.allclose(r["g"], g, rtol=1e-12, atol=1e-12)
    assert np.allclose(r["u"], u, rtol=1e-12, atol=1e-12)
    h = r["g"] * scipy.special.expit(r["g"]) * r["u"]
    assert np.allclose(r["h"], h, rtol=1e-6, atol=1e-9)  # oracle feeds fp32 g, u
    hdq = r["hq"].astype(np.float64) * np.repeat(r["hd"].astype(np.float64), 32, axis=1)
    assert np.allclose(r["y"], hdq @ Wd.T, rtol=1e-6, atol=1e-6)
    assert np.all(np.abs(hdq - r["h"]) <= np.repeat(r["hd"], 32, axis=1) * 0.50002)


def test_moe_weights_sum_and_slot_order():
    inp = wl.make_workload("ternary_moe_decode_t1", E=16, H=256, I=256, T=4, top_k=4)
    r = moe.decode_ffn(inp)
    # y equals the w-weighted sum of the per-slot outputs of each token
    out = r["out"].reshape(4, 4, 256)
    ref = np.einsum("tj,tjn->tn", r["w"].astype(np.float32).astype(np.float64),
                    out.astype(np.float32).astype(np.float64))
    assert np.allclose(r["y"], ref, rtol=1e-12, atol=1e-12)
    # outputs are indexed by assignment a = t*k + j, not by grouped order
    a = 5
    e = int(r["ids"].ravel()[a])
    W = oracle.unpack_ternary(inp["down"]["qs"][e], 256)
    y, _, _ = oracle.matvec_q8(W, inp["down"]["d"][e], r["hq"][a], r["hd"][a])
    assert np.array_equal(y, r["out"][a])


def _bf16_float(bits):
    return (np.asarray(bits, np.uint16).astype(np.uint32) << 16).view(np.float32).astype(np.float64)


def _torch_bf16_bits(x32):
    import torch
    return torch.from_numpy(np.ascontiguousarray(x32, np.float32)).to(torch.bfloat16).view(
        torch.int16).numpy().view(np.uint16)


@pytest.mark.parametrize("name", ["grid1_moe_prefill_t2048", "sign1_moe_prefill_t2048"])
def test_prefill_topk1_single_expert_is_dense_bf16_swiglu_mlp(name):
    """E = 1, k = 1: the prefill layer is a dense SwiGLU MLP through one
    expert, computed here with numpy matmuls on the dequantized weights and
    torch's bf16 rounding of h (a library routine), independently of the
    oracle's own unpack-free arithmetic."""
    H, I, T = 512, 512, 6
    inp = wl.make_workload(name, E=1, H=H, I=I, T=T, top_k=1)
    r = moe.prefill_ffn(inp)
    fmt, grid = inp["cfg"]["fmt"], inp.get("grid")
    assert np.all(r["ids"] == 0) and np.all(r["w"] == 1.0)

    def deq(planes, K):
        W = moe.unpack_expert(fmt, planes, 0, K, grid).astype(np.float64)
        if fmt == "sign1":
            return W * planes["d"][0].view(np.float16).astype(np.float64)[:, None]
        return W * _deq_scales(planes["d"][0], K)

    xf = _bf16_float(inp["x_bf16"])
    G, U = xf @ deq(inp["gate"], H).T, xf @ deq(inp["up"], H).T
    assert np.allclose(r["g"], G, rtol=1e-12, atol=1e-12)
    assert np.allclose(r["u"], U, rtol=1e-12, atol=1e-12)
    g32, u32 = G.astype(np.float32), U.astype(np.float32)
    h = g32.astype(np.float64) * scipy.special.expit(g32.astype(np.float64)) * u32.astype(np.float64)
    hb = _torch_bf16_bits(h.astype(np.float32))
    assert np.array_equal(r["h_bf16"], hb)
    out = _bf16_float(hb) @ deq(inp["down"], I).T
    assert np.allclose(r["out"], out, rtol=1e-12, atol=1e-12)
    # one slot of weight 1: y is out rounded to fp32 and summed once
    assert np.array_equal(r["y"], r["out"].astype(np.float32).astype(np.float64))


def test_prefill_layer_vs_numpy_per_assignment():
    """Several experts, top-2: every assignment's output is the dense MLP of
    its own expert on its token's row, and y the weighted sum of a token's two
    slots (numpy einsum); the term sums are |x| @ |W| products."""
    H, I, T, E, k = 256, 256, 10, 4, 2
    inp = wl.make_workload("grid1_moe_prefill_t2048", E=E, H=H, I=I, T=T, top_k=k)
    r = moe.prefill_ffn(inp)
    grid = inp["grid"]
    ids = r["ids"].ravel()
    xf = _bf16_float(inp["x_bf16"])
    for a in range(T * k):
        e, t = int(ids[a]), a // k
        Wg = oracle.unpack_grid1(inp["gate"]["qs"][e], inp["gate"]["qh"][e], grid, H) * _deq_scales(inp["gate"]["d"][e], H)
        Wd = oracle.unpack_grid1(inp["down"]["qs"][e], inp["down"]["qh"][e], grid, I) * _deq_scales(inp["down"]["d"][e], I)
        assert np.allclose(r["g"][a], Wg @ xf[t], rtol=1e-12, atol=1e-12)
        assert np.allclose(r["tg"][a], np.abs(Wg) @ np.abs(xf[t]), rtol=1e-12, atol=0)
        assert np.allclose(r["out"][a], Wd @ _bf16_float(r["h_bf16"][a]), rtol=1e-12, atol=1e-12)
    y = np.einsum("tj,tjn->tn", r["w"].astype(np.float32).astype(np.float64),
                  r["out"].astype(np.float32).astype(np.float64).reshape(T, k, H))
    assert np.allclose(r["y"], y, rtol=1e-14, atol=1e-15)
