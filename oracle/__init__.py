"""CPU oracle for the packed 1-bit-class MoE expert path.

TEST INFRASTRUCTURE ONLY: the tests, the smoke check and the benchmark's CPU
baseline leg may import this package; the library in
``bit_quantized_moe_q8_amd`` never does, and the two share no code.

``oracle.c`` holds the arithmetic (plain C, fp64 / exact integers, fixed order
per output).  This module loads it with ctypes and adds thin numpy wrappers;
``oracle.moe`` composes the steps of a MoE FFN layer.

Every function is pinned by the tests in ``tests/test_oracle_*.py`` against
hand-derived fixtures (``tests/golden``), closed forms, invariants, numpy
library routines or brute force.
"""
from __future__ import annotations

import ctypes
import os
import subprocess

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "oracle.c")
_LIB_PATH = os.path.join(_HERE, "liboracle.so")

CFLAGS = ["-O2", "-std=c11", "-fno-fast-math", "-ffp-contract=off", "-fopenmp",
          "-shared", "-fPIC", "-Wall", "-Wextra"]


def build(force: bool = True) -> str:
    """Compile liboracle.so with gcc (always, when force)."""
    if force or not os.path.exists(_LIB_PATH):
        tmp = _LIB_PATH + ".tmp%d" % os.getpid()
        subprocess.check_call(["gcc", *CFLAGS, _SRC, "-o", tmp, "-lm"])
        os.replace(tmp, _LIB_PATH)
    return _LIB_PATH


_lib = None


def lib():
    global _lib
    if _lib is None:
        if not os.path.exists(_LIB_PATH):
            build(force=True)
        L = ctypes.CDLL(_LIB_PATH)
        p = ctypes.c_void_p
        i64 = ctypes.c_int64
        i32 = ctypes.c_int32
        L.or_num_threads.restype = ctypes.c_int
        L.or_set_num_threads.argtypes = [ctypes.c_int]
        L.or_set_num_threads.restype = None
        L.or_half_to_float.argtypes = [ctypes.c_uint16]
        L.or_half_to_float.restype = ctypes.c_float
        L.or_bf16_to_float.argtypes = [ctypes.c_uint16]
        L.or_bf16_to_float.restype = ctypes.c_float
        L.or_float_to_bf16.argtypes = [ctypes.c_float]
        L.or_float_to_bf16.restype = ctypes.c_uint16
        L.or_quantize_q8.argtypes = [p, i64, i64, p, p]
        L.or_unpack_ternary.argtypes = [p, i64, i64, p]
        L.or_unpack_ternary.restype = i64
        L.or_unpack_grid1.argtypes = [p, p, p, i64, i64, p]
        L.or_unpack_sign1.argtypes = [p, p, i64, i64, p]
        L.or_matvec_q8.argtypes = [p, p, i64, i64, p, p, p, p, p]
        L.or_matvec_bf16.argtypes = [p, p, i64, i64, p, p, p]
        L.or_route_topk.argtypes = [p, i64, i64, ctypes.c_int, p, p]
        L.or_group.argtypes = [p, i64, i32, p, p, p, p]
        L.or_swiglu.argtypes = [p, p, i64, p]
        L.or_swiglu.restype = None
        L.or_combine.argtypes = [p, p, i64, ctypes.c_int, i64, p, p]
        L.or_combine.restype = None
        _lib = L
    return _lib


def _p(a: np.ndarray):
    assert a.flags["C_CONTIGUOUS"], "oracle inputs must be C-contiguous"
    return a.ctypes.data_as(ctypes.c_void_p)


def _c(a, dtype):
    return np.ascontiguousarray(a, dtype=dtype)


class OracleError(RuntimeError):
    pass


def num_threads() -> int:
    return lib().or_num_threads()


def set_num_threads(n: int) -> None:
    lib().or_set_num_threads(int(n))


def half_to_float(h: int) -> float:
    return lib().or_half_to_float(int(h))


def halves_to_f64(d16: np.ndarray) -> np.ndarray:
    """fp16 bit patterns -> float64, through the oracle's own bit-level conversion."""
    f = np.vectorize(lambda h: lib().or_half_to_float(int(h)), otypes=[np.float64])
    return f(np.asarray(d16, dtype=np.uint16)) if np.size(d16) else np.zeros(np.shape(d16))


def bf16_to_float(b: int) -> float:
    return lib().or_bf16_to_float(int(b))


def float_to_bf16(x: np.ndarray) -> np.ndarray:
    x = _c(x, np.float32).ravel()
    out = np.empty(x.shape, np.uint16)
    fn = lib().or_float_to_bf16
    for i, v in enumerate(x):
        out[i] = fn(float(v))
    return out


def quantize_q8(x: np.ndarray):
    """q8 per 32 values of each row: returns (q int8 [rows][cols], d float32 [rows][cols/32])."""
    x = _c(x, np.float32)
    if x.ndim == 1:
        x = x[None, :]
    rows, cols = x.shape
    q = np.empty((rows, cols), np.int8)
    d = np.empty((rows, cols // 32), np.float32)
    rc = lib().or_quantize_q8(_p(x), rows, cols, _p(q), _p(d))
    if rc != 0:
        raise OracleError("or_quantize_q8 failed (%d)" % rc)
    return q, d


def unpack_ternary(qs: np.ndarray, k: int) -> np.ndarray:
    qs = _c(qs, np.uint8)
    n = qs.size // (k // 4)
    w = np.empty((n, k), np.int8)
    bad = lib().or_unpack_ternary(_p(qs), n, k, _p(w))
    if bad != 0:
        raise OracleError("ternary planes hold %d code-3 fields" % bad)
    return w


def count_invalid_ternary(qs: np.ndarray, k: int) -> int:
    """Number of code-3 fields in ternary planes (rows of k weights; k/4 bytes
    per row).  The format defines codes 0, 1, 2 only (ternary format of the
    Parakon Runtime README, "How it works")."""
    qs = _c(qs, np.uint8)
    n = qs.size // (k // 4)
    w = np.empty((n, k), np.int8)
    bad = lib().or_unpack_ternary(_p(qs), n, k, _p(w))
    if bad < 0:
        raise OracleError("or_unpack_ternary failed (%d)" % bad)
    return int(bad)


def unpack_grid1(qs: np.ndarray, qh: np.ndarray, grid: np.ndarray, k: int) -> np.ndarray:
    qs = _c(qs, np.uint8)
    qh = _c(qh, np.uint16)
    grid = _c(grid, np.int8)
    n = qs.size // (k // 8)
    w = np.empty((n, k), np.int8)
    rc = lib().or_unpack_grid1(_p(qs), _p(qh), _p(grid), n, k, _p(w))
    if rc != 0:
        raise OracleError("or_unpack_grid1 failed (%d)" % rc)
    return w


def unpack_sign1(signs: np.ndarray, sc: np.ndarray, k: int) -> np.ndarray:
    """Integer weights sc * (+-1) of the sub-scaled sign format, rows of k
    weights (signs k/8 bytes, sub-scales k/32 bytes per row); the per-row
    anchor is applied by the mat-vec as the row's scale."""
    signs = _c(signs, np.uint8)
    sc = _c(sc, np.uint8)
    n = signs.size // (k // 8)
    w = np.empty((n, k), np.int8)
    rc = lib().or_unpack_sign1(_p(signs), _p(sc), n, k, _p(w))
    if rc != 0:
        raise OracleError("or_unpack_sign1 failed (%d)" % rc)
    return w


def matvec_q8(w: np.ndarray, d16: np.ndarray, xq: np.ndarray, xd: np.ndarray, want_isums=True):
    """Rows of unpacked weights against one q8 row: (y f64 [R], tsum f64 [R], isums i32 [R][K/32])."""
    w = _c(w, np.int8)
    R, K = w.shape
    d16 = _c(d16, np.uint16).reshape(R, K // 256)
    xq = _c(xq, np.int8).reshape(K)
    xd = _c(xd, np.float32).reshape(K // 32)
    y = np.empty(R, np.float64)
    t = np.empty(R, np.float64)
    isums = np.empty((R, K // 32), np.int32) if want_isums else None
    rc = lib().or_matvec_q8(_p(w), _p(d16), R, K, _p(xq), _p(xd),
                            _p(isums) if want_isums else None, _p(y), _p(t))
    if rc != 0:
        raise OracleError("or_matvec_q8 failed (%d)" % rc)
    return y, t, isums


def matvec_bf16(w: np.ndarray, d16: np.ndarray, x_bf16: np.ndarray):
    """Rows of unpacked weights against one bf16 row: (y f64 [R], tsum f64 [R])."""
    w = _c(w, np.int8)
    R, K = w.shape
    d16 = _c(d16, np.uint16).reshape(R, K // 256)
    x = _c(x_bf16, np.uint16).reshape(K)
    y = np.empty(R, np.float64)
    t = np.empty(R, np.float64)
    rc = lib().or_matvec_bf16(_p(w), _p(d16), R, K, _p(x), _p(y), _p(t))
    if rc != 0:
        raise OracleError("or_matvec_bf16 failed (%d)" % rc)
    return y, t


def route_topk(logits: np.ndarray, top_k: int):
    logits = _c(logits, np.float32)
    T, E = logits.shape
    ids = np.empty((T, top_k), np.int32)
    w = np.empty((T, top_k), np.float64)
    rc = lib().or_route_topk(_p(logits), T, E, top_k, _p(ids), _p(w))
    if rc != 0:
        raise OracleError("or_route_topk failed (%d)" % rc)
    return ids, w


def group(ids: np.ndarray, n_experts: int):
    """(offsets [E+1], sorted [A], active [n_active]) for flat assignment ids."""
    ids = _c(ids, np.int32).ravel()
    A = ids.size
    offsets = np.empty(n_experts + 1, np.int32)
    srt = np.empty(max(A, 1), np.int32)
    active = np.empty(max(n_experts, 1), np.int32)
    na = np.zeros(1, np.int32)
    rc = lib().or_group(_p(ids), A, n_experts, _p(offsets), _p(srt), _p(active), _p(na))
    if rc != 0:
        raise OracleError("or_group failed (%d)" % rc)
    return offsets, srt[:A].copy(), active[: int(na[0])].copy()


def swiglu(g: np.ndarray, u: np.ndarray) -> np.ndarray:
    g = _c(g, np.float32)
    u = _c(u, np.float32)
    h = np.empty(g.shape, np.float64)
    lib().or_swiglu(_p(g), _p(u), g.size, _p(h))
    return h


def combine(out: np.ndarray, w: np.ndarray, top_k: int):
    """(y f64 [T][H], ty f64 [T][H]) from out float32 [T*top_k][H] and w float32 [T][top_k]."""
    out = _c(out, np.float32)
    w = _c(w, np.float32)
    A, H = out.shape
    T = A // top_k
    y = np.empty((T, H), np.float64)
    ty = np.empty((T, H), np.float64)
    lib().or_combine(_p(out), _p(w), T, top_k, H, _p(y), _p(ty))
    return y, ty
