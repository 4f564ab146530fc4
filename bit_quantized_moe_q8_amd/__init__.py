"""Python binding of libpq (include/pq.h): packed 1-bit-class MoE expert kernels for MI355X.

Argument marshalling only: each function checks tensor dtypes, sizes,
devices and contiguity on the host (an undersized buffer raises ValueError
before anything is launched), then calls the C entry point of the same name on
torch's current HIP stream.  Every step of the computation runs in the library's HIP kernels;
there is no host fallback, and importing this module fails if libpq.so has not
been built (``python bit_quantized_moe_q8_amd/_build.py``).
"""
from __future__ import annotations

import ctypes
import os
from dataclasses import dataclass

import torch

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "libpq.so")

PQ_OK, PQ_ERR_NULL, PQ_ERR_SHAPE, PQ_ERR_ALIGN, PQ_ERR_UNSUPPORTED, PQ_ERR_HIP, PQ_ERR_SELFTEST = range(7)
PQ_EPI_F32, PQ_EPI_SWIGLU_Q8, PQ_EPI_SWIGLU_BF16, PQ_EPI_F32_COMBINE = 0, 1, 2, 3
PQ_FMT = {"ternary": 0, "grid1": 1, "sign1": 2}
PQ_CALL_MATVEC, PQ_CALL_TILE_Q8, PQ_CALL_GEMM, PQ_CALL_DECODE1_GATE_UP = 0, 1, 2, 3
(PQ_PLAN_MATVEC, PQ_PLAN_MATVEC_PAIRS, PQ_PLAN_MATVEC_TOK1, PQ_PLAN_TILE_Q8, PQ_PLAN_GEMM,
 PQ_PLAN_DECODE1_ROUTED, PQ_PLAN_DEBUG, PQ_PLAN_MIXED) = 1, 2, 4, 8, 16, 32, 64, 128

EXPORTS = (
    "pq_quantize_act_q8", "pq_moe_route_topk", "pq_group_tokens_by_expert", "pq_moe_decode_prep",
    "pq_moe_matvec_ternary", "pq_moe_matvec_grid1", "pq_moe_matvec_sign1",
    "pq_moe_tile_q8_ternary", "pq_moe_tile_q8_grid1", "pq_moe_tile_q8_sign1",
    "pq_moe_gemm_dequant_tile", "pq_moe_gemm_dequant_tile_sign1",
    "pq_moe_combine", "pq_moe_decode1_gate_up_ternary", "pq_moe_decode1_gate_up_grid1",
    "pq_moe_decode1_gate_up_sign1", "pq_validate_ternary",
    "pq_selftest", "pq_plan", "pq_peak_read", "pq_peak_mfma_bf16", "pq_status_str", "pq_abi_version",
    "pq_tile_layout_grid1", "pq_tile_layout_sign1",
)


class PQError(RuntimeError):
    def __init__(self, fn: str, status: int):
        super().__init__("%s failed: %s (%d)" % (fn, status_str(status), status))
        self.status = status


class TernaryW(ctypes.Structure):
    _fields_ = [("qs", ctypes.c_void_p), ("d", ctypes.c_void_p),
                ("n_experts", ctypes.c_int32), ("rows", ctypes.c_int32), ("cols", ctypes.c_int32)]


class Grid1W(ctypes.Structure):
    _fields_ = [("qs", ctypes.c_void_p), ("qh", ctypes.c_void_p), ("d", ctypes.c_void_p),
                ("grid", ctypes.c_void_p),
                ("n_experts", ctypes.c_int32), ("rows", ctypes.c_int32), ("cols", ctypes.c_int32)]


class Sign1W(ctypes.Structure):
    _fields_ = [("signs", ctypes.c_void_p), ("sc", ctypes.c_void_p), ("d", ctypes.c_void_p),
                ("n_experts", ctypes.c_int32), ("rows", ctypes.c_int32), ("cols", ctypes.c_int32)]


class Groups(ctypes.Structure):
    _fields_ = [("expert_offsets", ctypes.c_void_p), ("sorted_assign", ctypes.c_void_p),
                ("active_experts", ctypes.c_void_p), ("n_active", ctypes.c_void_p),
                ("n_tokens", ctypes.c_int32), ("top_k", ctypes.c_int32),
                ("n_experts", ctypes.c_int32)]


class Debug(ctypes.Structure):
    _fields_ = [("isums", ctypes.c_void_p), ("isums_up", ctypes.c_void_p),
                ("g", ctypes.c_void_p), ("u", ctypes.c_void_p), ("h", ctypes.c_void_p)]


def _load():
    if not os.path.exists(LIB_PATH):
        raise ImportError("libpq.so is not built; run: python bit_quantized_moe_q8_amd/_build.py")
    L = ctypes.CDLL(LIB_PATH)
    p, i32 = ctypes.c_void_p, ctypes.c_int32
    sig = {
        "pq_quantize_act_q8": [p, i32, i32, p, p, p],
        "pq_moe_route_topk": [p, i32, i32, i32, p, p, p],
        "pq_group_tokens_by_expert": [p, i32, i32, i32, p, p, p, p, p],
        "pq_moe_decode_prep": [p, p, i32, i32, i32, i32, p, p, p, p, p, p, p, p, p, p],
        "pq_moe_matvec_ternary": [ctypes.POINTER(TernaryW), ctypes.POINTER(TernaryW),
                                  ctypes.POINTER(Groups), p, p, i32, i32, p, p,
                                  ctypes.POINTER(Debug), p],
        "pq_moe_matvec_grid1": [ctypes.POINTER(Grid1W), ctypes.POINTER(Grid1W),
                                ctypes.POINTER(Groups), p, p, i32, i32, p, p,
                                ctypes.POINTER(Debug), p],
        "pq_moe_matvec_sign1": [ctypes.POINTER(Sign1W), ctypes.POINTER(Sign1W),
                                ctypes.POINTER(Groups), p, p, i32, i32, p, p,
                                ctypes.POINTER(Debug), p],
        "pq_moe_tile_q8_ternary": [ctypes.POINTER(TernaryW), ctypes.POINTER(TernaryW),
                                   ctypes.POINTER(Groups), p, p, i32, i32, p, p,
                                   ctypes.POINTER(Debug), p],
        "pq_moe_tile_q8_grid1": [ctypes.POINTER(Grid1W), ctypes.POINTER(Grid1W),
                                 ctypes.POINTER(Groups), p, p, i32, i32, p, p,
                                 ctypes.POINTER(Debug), p],
        "pq_moe_tile_q8_sign1": [ctypes.POINTER(Sign1W), ctypes.POINTER(Sign1W),
                                 ctypes.POINTER(Groups), p, p, i32, i32, p, p,
                                 ctypes.POINTER(Debug), p],
        "pq_moe_gemm_dequant_tile": [ctypes.POINTER(Grid1W), ctypes.POINTER(Grid1W),
                                     ctypes.POINTER(Groups), p, i32, i32, p, p,
                                     ctypes.POINTER(Debug), p],
        "pq_moe_gemm_dequant_tile_sign1": [ctypes.POINTER(Sign1W), ctypes.POINTER(Sign1W),
                                           ctypes.POINTER(Groups), p, i32, i32, p, p,
                                           ctypes.POINTER(Debug), p],
        "pq_moe_combine": [p, p, i32, i32, i32, p, p],
        "pq_moe_decode1_gate_up_ternary": [p, p, i32, i32, ctypes.POINTER(TernaryW),
                                           ctypes.POINTER(TernaryW)] + [p] * 10,
        "pq_moe_decode1_gate_up_sign1": [p, p, i32, i32, ctypes.POINTER(Sign1W),
                                         ctypes.POINTER(Sign1W)] + [p] * 10,
        "pq_moe_decode1_gate_up_grid1": [p, p, i32, i32, ctypes.POINTER(Grid1W),
                                         ctypes.POINTER(Grid1W)] + [p] * 10,
        "pq_validate_ternary": [ctypes.POINTER(TernaryW), p, p],
        "pq_selftest": [p],
        "pq_peak_read": [p, ctypes.c_int64, p, p],
        "pq_peak_mfma_bf16": [i32, i32, p, p, p, p],
        "pq_tile_layout_grid1": [ctypes.POINTER(Grid1W), p, p, p],
        "pq_tile_layout_sign1": [ctypes.POINTER(Sign1W), p, p, p],
        "pq_matvec_x32_ternary": [ctypes.POINTER(TernaryW), i32, p, p, p],
        "pq_matvec_x32_grid1": [ctypes.POINTER(Grid1W), i32, p, p, p],
        "pq_matvec_x32_sign1": [ctypes.POINTER(Sign1W), i32, p, p, p],
    }
    for name, args in sig.items():
        fn = getattr(L, name)
        fn.argtypes = args
        fn.restype = ctypes.c_int
    L.pq_plan.argtypes = [i32] * 9
    L.pq_plan.restype = i32
    L.pq_status_str.argtypes = [ctypes.c_int]
    L.pq_status_str.restype = ctypes.c_char_p
    L.pq_abi_version.restype = ctypes.c_int32
    return L


_lib = _load()


def lib():
    return _lib


def gemm_available() -> bool:
    """True once the prefill GEMM kernel is part of the build."""
    return GEMM_READY


GEMM_READY = True


def status_str(status: int) -> str:
    return _lib.pq_status_str(int(status)).decode()


def abi_version() -> int:
    return int(_lib.pq_abi_version())


def _stream():
    return ctypes.c_void_p(torch.cuda.current_stream().cuda_stream)


def _ptr(t):
    if t is None:
        return None
    if not t.is_cuda:
        raise ValueError("expected a device tensor")
    if not t.is_contiguous():
        raise ValueError("expected a contiguous tensor")
    return ctypes.c_void_p(t.data_ptr())


def _check(fn: str, rc: int):
    if rc != PQ_OK:
        raise PQError(fn, rc)


def _dt(t, *dtypes):
    if t.dtype not in dtypes:
        raise TypeError("expected dtype in %s, got %s" % (dtypes, t.dtype))


def _need(t, what: str, numel: int, *dtypes):
    """Host-side check of a buffer the kernels will index: dtype, and at
    least `numel` elements (an undersized buffer would be read or written
    out of bounds on the device)."""
    if t is None:
        return
    if dtypes:
        _dt(t, *dtypes)
    if t.numel() < numel:
        raise ValueError("%s holds %d elements, the call needs %d" % (what, t.numel(), numel))


_F32 = (torch.float32,)
_I8 = (torch.int8,)
_I32 = (torch.int32,)
_BF16 = (torch.bfloat16, torch.int16, torch.uint16)


def _need_plane(t, what, shape, *dtypes):
    _dt(t, *dtypes)
    if tuple(t.shape) != tuple(shape):
        raise ValueError("%s has shape %s, expected %s" % (what, tuple(t.shape), tuple(shape)))


def _check_groups(groups, n_tokens=None, top_k=None, n_experts=None):
    g = groups
    for v, want, what in ((n_tokens, g.n_tokens, "n_tokens"), (top_k, g.top_k, "top_k"),
                          (n_experts, g.n_experts, "n_experts")):
        if v is not None and v != want:
            raise ValueError("groups were built for %s = %d, the call has %d" % (what, want, v))
    _need(g.expert_offsets, "expert_offsets", g.n_experts + 1, *_I32)
    _need(g.sorted_assign, "sorted_assign", g.n_tokens * g.top_k, *_I32)
    _need(g.active_experts, "active_experts", g.n_experts, *_I32)
    _need(g.n_active, "n_active", 1, *_I32)


def _check_debug(dbg, A, rows, cols, two):
    if not dbg:
        return
    _need(dbg.get("isums"), "dbg isums", A * rows * (cols // 32), *_I32)
    if two:
        _need(dbg.get("isums_up"), "dbg isums_up", A * rows * (cols // 32), *_I32)
    elif dbg.get("isums_up") is not None:
        raise ValueError("dbg isums_up needs w_up")
    for f in ("g", "u", "h"):
        _need(dbg.get(f), "dbg " + f, A * rows, *_F32)


@dataclass
class TernaryWeights:
    """Packed ternary expert tensor: qs uint8 [E][rows][cols/4], d fp16 bits [E][rows][cols/256]."""
    qs: torch.Tensor
    d: torch.Tensor

    @property
    def shape(self):
        E, rows, q = self.qs.shape
        return E, rows, q * 4

    def cstruct(self) -> TernaryW:
        _dt(self.qs, torch.uint8)
        if self.qs.dim() != 3:
            raise ValueError("qs must be [E][rows][cols/4]")
        E, rows, cols = self.shape
        _need_plane(self.d, "d", (E, rows, cols // 256), torch.int16, torch.float16, torch.uint16)
        return TernaryW(_ptr(self.qs), _ptr(self.d), E, rows, cols)


@dataclass
class Sign1Weights:
    """Sub-scaled sign expert tensor: signs uint8 [E][rows][cols/8], sc uint8
    [E][rows][cols/32] (4-bit sub-scales), d fp16 bits [E][rows] (row anchors)."""
    signs: torch.Tensor
    sc: torch.Tensor
    d: torch.Tensor
    tiled: bool = False   # signs and sc in the tile layout (tile_layout), for the prefill GEMM only

    @property
    def shape(self):
        E, rows, q = self.signs.shape
        return E, rows, q * 8

    def cstruct(self) -> Sign1W:
        _dt(self.signs, torch.uint8)
        if self.signs.dim() != 3:
            raise ValueError("signs must be [E][rows][cols/8]")
        E, rows, cols = self.shape
        _need_plane(self.sc, "sc", (E, rows, cols // 32), torch.uint8)
        _need_plane(self.d, "d", (E, rows), torch.int16, torch.float16, torch.uint16)
        return Sign1W(_ptr(self.signs), _ptr(self.sc), _ptr(self.d), E, rows, cols)


@dataclass
class Grid1Weights:
    """Packed grid1 expert tensor: qs uint8 [E][rows][cols/8], qh [E][rows][cols/32],
    d fp16 bits [E][rows][cols/256], grid int8 [2048][8]."""
    qs: torch.Tensor
    qh: torch.Tensor
    d: torch.Tensor
    grid: torch.Tensor
    tiled: bool = False   # qs and qh in the tile layout (tile_layout), for the prefill GEMM only

    @property
    def shape(self):
        E, rows, q = self.qs.shape
        return E, rows, q * 8

    def cstruct(self) -> Grid1W:
        _dt(self.qs, torch.uint8)
        if self.qs.dim() != 3:
            raise ValueError("qs must be [E][rows][cols/8]")
        E, rows, cols = self.shape
        _need_plane(self.qh, "qh", (E, rows, cols // 32), torch.int16, torch.uint16)
        _need_plane(self.d, "d", (E, rows, cols // 256), torch.int16, torch.float16, torch.uint16)
        _need(self.grid, "grid", 2048 * 8, torch.int8)
        return Grid1W(_ptr(self.qs), _ptr(self.qh), _ptr(self.d), _ptr(self.grid), E, rows, cols)


@dataclass
class GroupBuffers:
    """Grouping of assignments by expert (filled by group_tokens_by_expert)."""
    expert_offsets: torch.Tensor  # int32 [E+1]
    sorted_assign: torch.Tensor   # int32 [A]
    active_experts: torch.Tensor  # int32 [E]
    n_active: torch.Tensor        # int32 [1]
    n_tokens: int
    top_k: int
    n_experts: int

    @staticmethod
    def empty(n_tokens: int, top_k: int, n_experts: int, device="cuda"):
        i32 = torch.int32
        return GroupBuffers(torch.empty(n_experts + 1, dtype=i32, device=device),
                            torch.empty(max(n_tokens * top_k, 1), dtype=i32, device=device),
                            torch.empty(n_experts, dtype=i32, device=device),
                            torch.empty(1, dtype=i32, device=device),
                            n_tokens, top_k, n_experts)

    def cstruct(self) -> Groups:
        return Groups(_ptr(self.expert_offsets), _ptr(self.sorted_assign),
                      _ptr(self.active_experts), _ptr(self.n_active),
                      self.n_tokens, self.top_k, self.n_experts)


def _debug_struct(dbg):
    if dbg is None:
        return None
    return ctypes.byref(Debug(*[_ptr(dbg.get(k)) for k in ("isums", "isums_up", "g", "u", "h")]))


# ------------------------------------------------------------------ entry points

def plan(call: int, fmt: str, n_tokens: int, top_k: int, n_experts: int, rows: int, cols: int,
         epilogue: int = PQ_EPI_F32, debug: bool = False) -> int:
    """pq_plan: the PQ_PLAN_* flags of the kernels an entry point of family
    `call` launches for these sizes (host only; negative: -status)."""
    return int(_lib.pq_plan(int(call), PQ_FMT[fmt], int(n_tokens), int(top_k), int(n_experts),
                            int(rows), int(cols), int(epilogue), int(bool(debug))))


def quantize_act_q8(x: torch.Tensor, xq: torch.Tensor = None, xd: torch.Tensor = None):
    """pq_quantize_act_q8: x float32 [rows][cols] -> (xq int8 [rows][cols], xd float32 [rows][cols/32])."""
    _dt(x, torch.float32)
    rows, cols = x.shape
    _need(xq, "xq", rows * cols, *_I8)
    _need(xd, "xd", rows * (cols // 32), *_F32)
    if xq is None:
        xq = torch.empty((rows, cols), dtype=torch.int8, device=x.device)
    if xd is None:
        xd = torch.empty((rows, cols // 32), dtype=torch.float32, device=x.device)
    _check("pq_quantize_act_q8", _lib.pq_quantize_act_q8(_ptr(x), rows, cols, _ptr(xq), _ptr(xd), _stream()))
    return xq, xd


def moe_route_topk(logits: torch.Tensor, top_k: int, ids: torch.Tensor = None, w: torch.Tensor = None):
    """pq_moe_route_topk: logits float32 [T][E] -> (ids int32 [T][k], w float32 [T][k])."""
    _dt(logits, torch.float32)
    T, E = logits.shape
    _need(ids, "ids", T * top_k, *_I32)
    _need(w, "w", T * top_k, *_F32)
    if ids is None:
        ids = torch.empty((T, top_k), dtype=torch.int32, device=logits.device)
    if w is None:
        w = torch.empty((T, top_k), dtype=torch.float32, device=logits.device)
    _check("pq_moe_route_topk", _lib.pq_moe_route_topk(_ptr(logits), T, E, top_k, _ptr(ids), _ptr(w), _stream()))
    return ids, w


def group_tokens_by_expert(ids: torch.Tensor, n_experts: int, groups: GroupBuffers = None) -> GroupBuffers:
    """pq_group_tokens_by_expert: ids int32 [T][k] -> GroupBuffers."""
    _dt(ids, torch.int32)
    T, k = ids.shape
    if groups is None:
        groups = GroupBuffers.empty(T, k, n_experts, ids.device)
    _check_groups(groups, T, k, n_experts)
    g = groups
    _check("pq_group_tokens_by_expert", _lib.pq_group_tokens_by_expert(
        _ptr(ids), T, k, n_experts, _ptr(g.expert_offsets), _ptr(g.sorted_assign),
        _ptr(g.active_experts), _ptr(g.n_active), _stream()))
    return groups


def decode_prep(x: torch.Tensor, logits: torch.Tensor, top_k: int, xq, xd, ids, w,
                groups: GroupBuffers, y_zero: torch.Tensor = None):
    """pq_moe_decode_prep: q8(x), top-k routing and grouping for a few tokens in
    one launch, into the given buffers (and y_zero cleared if given)."""
    _dt(x, torch.float32)
    _dt(logits, torch.float32)
    T, H = x.shape
    E = logits.shape[1]
    if logits.shape[0] != T:
        raise ValueError("logits rows %d != tokens %d" % (logits.shape[0], T))
    _need(xq, "xq", T * H, *_I8)
    _need(xd, "xd", T * (H // 32), *_F32)
    _need(ids, "ids", T * top_k, *_I32)
    _need(w, "w", T * top_k, *_F32)
    _need(y_zero, "y_zero", T * H, *_F32)
    _check_groups(groups, T, top_k, E)
    g = groups
    _check("pq_moe_decode_prep", _lib.pq_moe_decode_prep(
        _ptr(x), _ptr(logits), T, H, E, top_k, _ptr(xq), _ptr(xd), _ptr(ids), _ptr(w),
        _ptr(g.expert_offsets), _ptr(g.sorted_assign), _ptr(g.active_experts), _ptr(g.n_active),
        _ptr(y_zero), _stream()))


def decode_prep_supported(n_tokens: int, n_experts: int, top_k: int) -> bool:
    """The limits of pq_moe_decode_prep (include/pq.h)."""
    return (0 <= n_tokens and 1 <= top_k <= min(16, n_experts) and n_experts <= 1024
            and n_tokens * top_k <= 1 << 20)


def decode_prep_one_launch(n_tokens: int, n_experts: int, top_k: int) -> bool:
    """pq_moe_decode_prep runs as one launch (one workgroup) at these sizes."""
    return (1 <= n_tokens <= 16 and n_experts <= 1024 and n_tokens * top_k <= 256 and top_k <= 16
            and n_tokens * n_experts <= 1024)


def _check_up(w, w_up):
    if w_up is None:
        return
    if type(w_up) is not type(w) or tuple(w_up.shape) != tuple(w.shape):
        raise ValueError("w_up must be the same format and shape as w")


def _matvec(fn_name, w, w_up, groups, xq, xd, act_by_token, epilogue, out0, out1, dbg):
    _need_layout(w, False, fn_name)
    _need_layout(w_up, False, fn_name)
    _dt(xq, torch.int8)
    _dt(xd, torch.float32)
    E, rows, cols = w.shape
    _check_up(w, w_up)
    _check_groups(groups, n_experts=E)
    A = groups.n_tokens * groups.top_k
    n_act = groups.n_tokens if act_by_token else A
    _need(xq, "xq", n_act * cols)
    _need(xd, "xd", n_act * (cols // 32))
    if epilogue == PQ_EPI_F32:
        _need(out0, "out0", A * rows, *_F32)
    elif epilogue == PQ_EPI_SWIGLU_Q8:
        _need(out0, "out0 (hq)", A * rows, *_I8)
        _need(out1, "out1 (hd)", A * (rows // 32), *_F32)
    elif epilogue == PQ_EPI_F32_COMBINE:
        if out0 is None or out1 is None:
            raise ValueError("PQ_EPI_F32_COMBINE needs out0 (y) and out1 (topk_w)")
        _need(out0, "out0 (y)", groups.n_tokens * rows, *_F32)
        _need(out1, "out1 (topk_w)", A, *_F32)
    _check_debug(dbg, A, rows, cols, w_up is not None)
    dev = xq.device
    if out0 is None:
        if epilogue == PQ_EPI_F32:
            out0 = torch.empty((A, rows), dtype=torch.float32, device=dev)
        else:
            out0 = torch.empty((A, rows), dtype=torch.int8, device=dev)
    if out1 is None and epilogue == PQ_EPI_SWIGLU_Q8:
        out1 = torch.empty((A, rows // 32), dtype=torch.float32, device=dev)
    ws = w.cstruct()
    wu = w_up.cstruct() if w_up is not None else None
    gs = groups.cstruct()
    rc = getattr(_lib, fn_name)(ctypes.byref(ws), ctypes.byref(wu) if wu is not None else None,
                                ctypes.byref(gs), _ptr(xq), _ptr(xd), int(act_by_token), int(epilogue),
                                _ptr(out0), _ptr(out1), _debug_struct(dbg), _stream())
    _check(fn_name, rc)
    return out0, out1


def moe_matvec_ternary(w: TernaryWeights, w_up, groups: GroupBuffers, xq, xd, act_by_token: bool,
                       epilogue: int = PQ_EPI_F32, out0=None, out1=None, dbg: dict = None):
    """pq_moe_matvec_ternary (see include/pq.h)."""
    return _matvec("pq_moe_matvec_ternary", w, w_up, groups, xq, xd, act_by_token, epilogue, out0, out1, dbg)


def moe_matvec_grid1(w: Grid1Weights, w_up, groups: GroupBuffers, xq, xd, act_by_token: bool,
                     epilogue: int = PQ_EPI_F32, out0=None, out1=None, dbg: dict = None):
    """pq_moe_matvec_grid1 (see include/pq.h)."""
    return _matvec("pq_moe_matvec_grid1", w, w_up, groups, xq, xd, act_by_token, epilogue, out0, out1, dbg)


def moe_matvec_sign1(w: Sign1Weights, w_up, groups: GroupBuffers, xq, xd, act_by_token: bool,
                     epilogue: int = PQ_EPI_F32, out0=None, out1=None, dbg: dict = None):
    """pq_moe_matvec_sign1 (see include/pq.h)."""
    return _matvec("pq_moe_matvec_sign1", w, w_up, groups, xq, xd, act_by_token, epilogue, out0, out1, dbg)


def matvec_x32(w, x, expert: int = 0, y=None):
    """pq_matvec_x32_{ternary,grid1,sign1} (see include/pq.h): y [rows] =
    W[expert] . q8(x) for one fp32 row x [cols], in one launch."""
    fn_name = {"TernaryWeights": "pq_matvec_x32_ternary", "Grid1Weights": "pq_matvec_x32_grid1",
               "Sign1Weights": "pq_matvec_x32_sign1"}.get(type(w).__name__)
    if fn_name is None:
        raise ValueError("expected TernaryWeights, Grid1Weights or Sign1Weights")
    _need_layout(w, False, fn_name)
    E, rows, cols = w.shape
    if not 0 <= int(expert) < E:
        raise ValueError("expert %d outside [0, %d)" % (expert, E))
    _dt(x, torch.float32)
    _need(x, "x", cols)
    if y is None:
        y = torch.empty((rows,), dtype=torch.float32, device=x.device)
    _need(y, "y", rows, *_F32)
    ws = w.cstruct()
    rc = getattr(_lib, fn_name)(ctypes.byref(ws), int(expert), _ptr(x), _ptr(y), _stream())
    _check(fn_name, rc)
    return y


def moe_tile_q8_ternary(w: TernaryWeights, w_up, groups: GroupBuffers, xq, xd, act_by_token: bool,
                        epilogue: int = PQ_EPI_F32, out0=None, out1=None, dbg: dict = None):
    """pq_moe_tile_q8_ternary (see include/pq.h)."""
    return _matvec("pq_moe_tile_q8_ternary", w, w_up, groups, xq, xd, act_by_token, epilogue, out0, out1, dbg)


def moe_tile_q8_grid1(w: Grid1Weights, w_up, groups: GroupBuffers, xq, xd, act_by_token: bool,
                      epilogue: int = PQ_EPI_F32, out0=None, out1=None, dbg: dict = None):
    """pq_moe_tile_q8_grid1 (see include/pq.h)."""
    return _matvec("pq_moe_tile_q8_grid1", w, w_up, groups, xq, xd, act_by_token, epilogue, out0, out1, dbg)


def moe_tile_q8_sign1(w: Sign1Weights, w_up, groups: GroupBuffers, xq, xd, act_by_token: bool,
                      epilogue: int = PQ_EPI_F32, out0=None, out1=None, dbg: dict = None):
    """pq_moe_tile_q8_sign1 (see include/pq.h)."""
    return _matvec("pq_moe_tile_q8_sign1", w, w_up, groups, xq, xd, act_by_token, epilogue, out0, out1, dbg)


def _need_layout(w, tiled: bool, what: str):
    if w is not None and bool(getattr(w, "tiled", False)) != tiled:
        raise ValueError("%s takes weights %s the tile layout" % (what, "in" if tiled else "not in"))


def tile_layout(w):
    """pq_tile_layout_grid1 / pq_tile_layout_sign1: a copy of w (Grid1Weights or
    Sign1Weights) with its code planes in the tile layout the prefill GEMM
    reads; d (and the grid) are shared with w."""
    _need_layout(w, False, "tile_layout")
    cw = w.cstruct()
    if isinstance(w, Sign1Weights):
        signs, sc = torch.empty_like(w.signs), torch.empty_like(w.sc)
        _check("pq_tile_layout_sign1", _lib.pq_tile_layout_sign1(ctypes.byref(cw), _ptr(signs), _ptr(sc), _stream()))
        return Sign1Weights(signs=signs, sc=sc, d=w.d, tiled=True)
    qs, qh = torch.empty_like(w.qs), torch.empty_like(w.qh)
    _check("pq_tile_layout_grid1", _lib.pq_tile_layout_grid1(ctypes.byref(cw), _ptr(qs), _ptr(qh), _stream()))
    return Grid1Weights(qs=qs, qh=qh, d=w.d, grid=w.grid, tiled=True)


def moe_gemm_dequant_tile(w: Grid1Weights, w_up, groups: GroupBuffers, x_bf16: torch.Tensor,
                          act_by_token: bool, epilogue: int = PQ_EPI_F32, out0=None, dbg: dict = None,
                          out1=None):
    """pq_moe_gemm_dequant_tile (grid1) or pq_moe_gemm_dequant_tile_sign1 (Sign1Weights):
    weights in the tile layout (tile_layout), x bf16 (torch.bfloat16 or int16 bits).
    PQ_EPI_F32_COMBINE: out0 = y float32 [T][rows] (accumulated into; zero it
    first), out1 = topk_w float32 [T][k]."""
    _need_layout(w, True, "moe_gemm_dequant_tile")
    _need_layout(w_up, True, "moe_gemm_dequant_tile")
    _dt(x_bf16, *_BF16)
    E, rows, cols = w.shape
    _check_up(w, w_up)
    _check_groups(groups, n_experts=E)
    A = groups.n_tokens * groups.top_k
    n_act = groups.n_tokens if act_by_token else A
    _need(x_bf16, "x", n_act * cols)
    if epilogue == PQ_EPI_F32:
        _need(out0, "out0", A * rows, *_F32)
    elif epilogue == PQ_EPI_F32_COMBINE:
        if out0 is None or out1 is None:
            raise ValueError("the fused combine needs y (out0) and topk_w (out1)")
        _need(out0, "y", groups.n_tokens * rows, *_F32)
        _need(out1, "topk_w", A, *_F32)
    else:
        _need(out0, "out0 (h)", A * rows, *_BF16)
    _check_debug(dbg, A, rows, cols, w_up is not None)
    if out0 is None:
        dt = torch.float32 if epilogue == PQ_EPI_F32 else torch.bfloat16
        out0 = torch.empty((A, rows), dtype=dt, device=x_bf16.device)
    ws = w.cstruct()
    wu = w_up.cstruct() if w_up is not None else None
    gs = groups.cstruct()
    fn = "pq_moe_gemm_dequant_tile_sign1" if isinstance(w, Sign1Weights) else "pq_moe_gemm_dequant_tile"
    rc = getattr(_lib, fn)(ctypes.byref(ws), ctypes.byref(wu) if wu is not None else None,
                           ctypes.byref(gs), _ptr(x_bf16), int(act_by_token), int(epilogue),
                           _ptr(out0), _ptr(out1), _debug_struct(dbg), _stream())
    _check(fn, rc)
    return out0


def moe_combine(out_assign: torch.Tensor, topk_w: torch.Tensor, top_k: int, y: torch.Tensor = None):
    """pq_moe_combine: out_assign float32 [T*k][rows], topk_w float32 [T][k] -> y float32 [T][rows]."""
    _dt(out_assign, torch.float32)
    A, rows = out_assign.shape
    if A % top_k:
        raise ValueError("out_assign rows %d are not a multiple of top_k %d" % (A, top_k))
    T = A // top_k
    _need(topk_w, "topk_w", A, *_F32)
    _need(y, "y", T * rows, *_F32)
    if y is None:
        y = torch.empty((T, rows), dtype=torch.float32, device=out_assign.device)
    _check("pq_moe_combine", _lib.pq_moe_combine(_ptr(out_assign), _ptr(topk_w), T, top_k, rows, _ptr(y), _stream()))
    return y


def validate_ternary(w: "TernaryWeights", n_bad: torch.Tensor = None) -> torch.Tensor:
    """pq_validate_ternary: device int32 [1] holding the number of code-3 fields in w.qs."""
    _need(n_bad, "n_bad", 1, *_I32)
    if n_bad is None:
        n_bad = torch.empty(1, dtype=torch.int32, device=w.qs.device)
    cw = w.cstruct()
    _check("pq_validate_ternary", _lib.pq_validate_ternary(ctypes.byref(cw), _ptr(n_bad), _stream()))
    return n_bad


def selftest() -> int:
    """pq_selftest on the current stream; returns the status code (PQ_OK on success)."""
    return int(_lib.pq_selftest(_stream()))


def moe_decode1_gate_up(gate, up, x: torch.Tensor, logits: torch.Tensor, top_k: int, ids, w, groups,
                        hq, hd, y_zero=None):
    """pq_moe_decode1_gate_up_{ternary,grid1,sign1}: one token's routing, q8 and gate/up
    (SwiGLU + q8) in one launch.  x float32 [1][H], logits float32 [1][E];
    writes ids int32 [1][k], w float32 [1][k], groups (GroupBuffers), hq int8
    [k][I], hd float32 [k][I/32], and zeros y_zero float32 [1][H] if given."""
    _need_layout(gate, False, "moe_decode1_gate_up")
    _need_layout(up, False, "moe_decode1_gate_up")
    _dt(x, torch.float32)
    _dt(logits, torch.float32)
    E = logits.shape[-1]
    Eg, I, H = gate.shape
    _check_up(gate, up)
    if Eg != E:
        raise ValueError("logits cover %d experts, the weights %d" % (E, Eg))
    if x.numel() != H or logits.numel() != E:
        raise ValueError("one token: x must hold %d values and logits %d" % (H, E))
    for t, what, n, dts in ((ids, "ids", top_k, _I32), (w, "w", top_k, _F32), (hq, "hq", top_k * I, _I8),
                            (hd, "hd", top_k * (I // 32), _F32)):
        if t is None:
            raise ValueError("%s is required" % what)
        _need(t, what, n, *dts)
    _need(y_zero, "y_zero", H, *_F32)
    _check_groups(groups, 1, top_k, E)
    fn = ("pq_moe_decode1_gate_up_ternary" if isinstance(gate, TernaryWeights)
          else "pq_moe_decode1_gate_up_sign1" if isinstance(gate, Sign1Weights)
          else "pq_moe_decode1_gate_up_grid1")
    cg, cu = gate.cstruct(), up.cstruct()
    rc = getattr(_lib, fn)(_ptr(x), _ptr(logits), E, top_k, ctypes.byref(cg), ctypes.byref(cu),
                           _ptr(ids), _ptr(w), _ptr(groups.expert_offsets), _ptr(groups.sorted_assign),
                           _ptr(groups.active_experts), _ptr(groups.n_active), _ptr(hq), _ptr(hd),
                           _ptr(y_zero), _stream())
    _check(fn, rc)


def peak_read(buf: torch.Tensor, sink: torch.Tensor):
    """pq_peak_read over every byte of `buf` (a measurement aid)."""
    _need(sink, "sink", 1024, torch.int32)
    n = buf.numel() * buf.element_size()
    _check("pq_peak_read", _lib.pq_peak_read(_ptr(buf), n - n % 16, _ptr(sink), _stream()))
    return n - n % 16


def peak_mfma_bf16(workgroups: int, iters: int, sink: torch.Tensor) -> float:
    """pq_peak_mfma_bf16 (a measurement aid); returns the flops it issues."""
    _need(sink, "sink", 1024, torch.float32)
    wpw, ch = ctypes.c_int32(0), ctypes.c_int32(0)
    _check("pq_peak_mfma_bf16", _lib.pq_peak_mfma_bf16(int(workgroups), int(iters), _ptr(sink),
                                                       ctypes.byref(wpw), ctypes.byref(ch), _stream()))
    return float(workgroups) * wpw.value * iters * ch.value * 16 * 16 * 32 * 2
