"""C-ABI checks that need no GPU: the library loads, exports every entry point
declared in include/pq.h, and rejects invalid arguments on the host before any
HIP call (fake, never-dereferenced pointer values are passed)."""
import ctypes
import os
import re

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def _declared():
    txt = open(os.path.join(ROOT, "include", "pq.h")).read()
    txt = re.sub(r"/\*.*?\*/", "", txt, flags=re.S)
    return sorted(set(re.findall(r"\b(pq_[a-z0-9_]+)\s*\(", txt)))


@pytest.fixture(scope="module")
def L():
    import bit_quantized_moe_q8_amd as pq
    return pq.lib()


def test_exports_every_declared_symbol(L):
    names = _declared()
    assert "pq_moe_matvec_ternary" in names and len(names) >= 9
    for n in names:
        assert hasattr(L, n), n


def test_abi_version_and_status_strings(L):
    import bit_quantized_moe_q8_amd as pq
    assert pq.abi_version() == 1
    for s in range(7):
        assert pq.status_str(s)
    assert pq.status_str(0) == "ok"


A16 = ctypes.c_void_p(0x10000)   # 16-byte aligned fake device address
A1 = ctypes.c_void_p(0x10001)    # misaligned fake address
S = None


def test_quantize_validation(L):
    import bit_quantized_moe_q8_amd as pq
    f = L.pq_quantize_act_q8
    assert f(A16, 1, 33, A16, A16, S) == pq.PQ_ERR_SHAPE
    assert f(A16, -1, 32, A16, A16, S) == pq.PQ_ERR_SHAPE
    assert f(None, 1, 32, A16, A16, S) == pq.PQ_ERR_NULL
    assert f(A1, 1, 32, A16, A16, S) == pq.PQ_ERR_ALIGN
    assert f(None, 0, 32, None, None, S) == pq.PQ_OK  # empty input: nothing enqueued


def test_route_validation(L):
    import bit_quantized_moe_q8_amd as pq
    f = L.pq_moe_route_topk
    assert f(A16, 4, 8, 9, A16, A16, S) == pq.PQ_ERR_SHAPE      # top_k > n_experts
    assert f(A16, 4, 2048, 8, A16, A16, S) == pq.PQ_ERR_SHAPE   # n_experts > 1024
    assert f(A16, 4, 64, 17, A16, A16, S) == pq.PQ_ERR_SHAPE    # top_k > 16
    assert f(A16, 4, 64, 0, A16, A16, S) == pq.PQ_ERR_SHAPE
    assert f(None, 4, 64, 8, A16, A16, S) == pq.PQ_ERR_NULL
    assert f(A1, 4, 64, 8, A16, A16, S) == pq.PQ_ERR_ALIGN


def test_group_validation(L):
    import bit_quantized_moe_q8_amd as pq
    f = L.pq_group_tokens_by_expert
    assert f(A16, 1 << 20, 8, 64, A16, A16, A16, A16, S) == pq.PQ_ERR_SHAPE  # A > 2^20
    assert f(A16, 4, 8, 64, None, A16, A16, A16, S) == pq.PQ_ERR_NULL
    assert f(A16, 4, 8, 64, A1, A16, A16, A16, S) == pq.PQ_ERR_ALIGN


def _groups(pq, E=8, T=2, k=2):
    return pq.Groups(A16, A16, A16, A16, T, k, E)


def test_matvec_validation(L):
    import bit_quantized_moe_q8_amd as pq
    f = L.pq_moe_matvec_ternary
    g = _groups(pq)
    ok_w = pq.TernaryW(A16, A16, 8, 64, 1024)
    b = ctypes.byref
    # cols not a multiple of 256
    assert f(b(pq.TernaryW(A16, A16, 8, 64, 1000)), None, b(g), A16, A16, 1, 0, A16, None, None, S) == pq.PQ_ERR_SHAPE
    # expert count mismatch with the groups
    assert f(b(pq.TernaryW(A16, A16, 4, 64, 1024)), None, b(g), A16, A16, 1, 0, A16, None, None, S) == pq.PQ_ERR_SHAPE
    # SwiGLU epilogue without w_up, or without out1, or rows % 32
    assert f(b(ok_w), None, b(g), A16, A16, 1, 1, A16, A16, None, S) == pq.PQ_ERR_NULL
    assert f(b(ok_w), b(ok_w), b(g), A16, A16, 1, 1, A16, None, None, S) == pq.PQ_ERR_NULL
    w48 = pq.TernaryW(A16, A16, 8, 48, 1024)
    assert f(b(w48), b(w48), b(g), A16, A16, 1, 1, A16, A16, None, S) == pq.PQ_ERR_SHAPE
    # up shape differs
    assert f(b(ok_w), b(pq.TernaryW(A16, A16, 8, 64, 2048)), b(g), A16, A16, 1, 1, A16, A16, None, S) == pq.PQ_ERR_SHAPE
    # misaligned packed codes / activations
    assert f(b(pq.TernaryW(A1, A16, 8, 64, 1024)), None, b(g), A16, A16, 1, 0, A16, None, None, S) == pq.PQ_ERR_ALIGN
    assert f(b(ok_w), None, b(g), A1, A16, 1, 0, A16, None, None, S) == pq.PQ_ERR_ALIGN
    # an unsupported (valid) width: cols/64 = 20
    assert f(b(pq.TernaryW(A16, A16, 8, 64, 1280)), None, b(g), A16, A16, 1, 0, A16, None, None, S) == pq.PQ_ERR_UNSUPPORTED
    # bf16 epilogue is not a decode epilogue
    assert f(b(ok_w), b(ok_w), b(g), A16, A16, 1, 2, A16, A16, None, S) == pq.PQ_ERR_UNSUPPORTED
    # bad groups
    assert f(b(ok_w), None, b(_groups(pq, E=8, T=2, k=9)), A16, A16, 1, 0, A16, None, None, S) == pq.PQ_ERR_SHAPE
    assert f(b(ok_w), None, None, A16, A16, 1, 0, A16, None, None, S) == pq.PQ_ERR_NULL
    # zero tokens: valid, nothing enqueued
    assert f(b(ok_w), None, b(_groups(pq, T=0)), None, None, 1, 0, A16, None, None, S) == pq.PQ_OK


def test_grid1_validation(L):
    import bit_quantized_moe_q8_amd as pq
    f = L.pq_moe_matvec_grid1
    g = _groups(pq)
    b = ctypes.byref
    assert f(b(pq.Grid1W(A16, None, A16, A16, 8, 64, 1024)), None, b(g), A16, A16, 1, 0, A16, None, None, S) == pq.PQ_ERR_NULL
    assert f(b(pq.Grid1W(A16, A16, A16, A1, 8, 64, 1024)), None, b(g), A16, A16, 1, 0, A16, None, None, S) == pq.PQ_ERR_ALIGN
    assert f(b(pq.Grid1W(A16, A16, A16, A16, 8, 64, 2560)), None, b(g), A16, A16, 1, 0, A16, None, None, S) == pq.PQ_ERR_UNSUPPORTED


def test_sign1_validation(L):
    import bit_quantized_moe_q8_amd as pq
    f = L.pq_moe_matvec_sign1
    b = ctypes.byref
    g = _groups(pq)
    ok_w = pq.Sign1W(A16, A16, A16, 8, 64, 1024)
    assert f(b(pq.Sign1W(A16, None, A16, 8, 64, 1024)), None, b(g), A16, A16, 1, 0, A16, None, None, S) == pq.PQ_ERR_NULL
    assert f(b(pq.Sign1W(A16, A16, A16, 8, 64, 1000)), None, b(g), A16, A16, 1, 0, A16, None, None, S) == pq.PQ_ERR_SHAPE
    assert f(b(pq.Sign1W(A16, A1, A16, 8, 64, 1024)), None, b(g), A16, A16, 1, 0, A16, None, None, S) == pq.PQ_ERR_ALIGN
    assert f(b(pq.Sign1W(A1, A16, A16, 8, 64, 1024)), None, b(g), A16, A16, 1, 0, A16, None, None, S) == pq.PQ_ERR_ALIGN
    assert f(b(pq.Sign1W(A16, A16, A16, 8, 64, 2560)), None, b(g), A16, A16, 1, 0, A16, None, None, S) == pq.PQ_ERR_UNSUPPORTED
    assert f(b(ok_w), None, b(g), A16, A16, 1, 1, A16, A16, None, S) == pq.PQ_ERR_NULL
    assert f(b(ok_w), b(ok_w), b(g), A16, A16, 1, 2, A16, A16, None, S) == pq.PQ_ERR_UNSUPPORTED
    assert f(b(ok_w), None, b(_groups(pq, T=0)), None, None, 1, 0, A16, None, None, S) == pq.PQ_OK


def test_tile_q8_validation(L):
    """The int8-MFMA tile entry points share the mat-vec's checks but accept
    any cols that is a multiple of 256 (e.g. 1280, which the mat-vec rejects)."""
    import bit_quantized_moe_q8_amd as pq
    b = ctypes.byref
    g = _groups(pq)
    for f, mk in ((L.pq_moe_tile_q8_ternary, lambda rows, cols: pq.TernaryW(A16, A16, 8, rows, cols)),
                  (L.pq_moe_tile_q8_grid1, lambda rows, cols: pq.Grid1W(A16, A16, A16, A16, 8, rows, cols)),
                  (L.pq_moe_tile_q8_sign1, lambda rows, cols: pq.Sign1W(A16, A16, A16, 8, rows, cols))):
        ok_w = mk(64, 1024)
        assert f(b(mk(64, 1000)), None, b(g), A16, A16, 1, 0, A16, None, None, S) == pq.PQ_ERR_SHAPE
        assert f(b(mk(64, 128)), None, b(g), A16, A16, 1, 0, A16, None, None, S) == pq.PQ_ERR_SHAPE
        assert f(b(ok_w), None, b(g), A16, A16, 1, 1, A16, A16, None, S) == pq.PQ_ERR_NULL
        w48 = mk(48, 1024)
        assert f(b(w48), b(w48), b(g), A16, A16, 1, 1, A16, A16, None, S) == pq.PQ_ERR_SHAPE
        assert f(b(ok_w), None, b(g), A1, A16, 1, 0, A16, None, None, S) == pq.PQ_ERR_ALIGN
        assert f(b(ok_w), b(ok_w), b(g), A16, A16, 1, 2, A16, A16, None, S) == pq.PQ_ERR_UNSUPPORTED
        assert f(b(ok_w), None, b(g), A16, A16, 1, 3, A16, A16, None, S) == pq.PQ_ERR_UNSUPPORTED
        assert f(b(ok_w), None, None, A16, A16, 1, 0, A16, None, None, S) == pq.PQ_ERR_NULL
        assert f(b(mk(64, 1280)), None, b(_groups(pq, T=0)), None, None, 1, 0, A16, None, None, S) == pq.PQ_OK


def test_combine_validation(L):
    import bit_quantized_moe_q8_amd as pq
    f = L.pq_moe_combine
    assert f(A16, A16, 2, 0, 64, A16, S) == pq.PQ_ERR_SHAPE
    assert f(None, A16, 2, 2, 64, A16, S) == pq.PQ_ERR_NULL
    assert f(A16, A16, 2, 2, 64, A1, S) == pq.PQ_ERR_ALIGN


def test_validate_ternary_validation(L):
    import bit_quantized_moe_q8_amd as pq
    f = L.pq_validate_ternary
    b = ctypes.byref
    assert f(None, A16, S) == pq.PQ_ERR_NULL
    assert f(b(pq.TernaryW(A16, A16, 8, 64, 1024)), None, S) == pq.PQ_ERR_NULL
    assert f(b(pq.TernaryW(None, A16, 8, 64, 1024)), A16, S) == pq.PQ_ERR_NULL
    assert f(b(pq.TernaryW(A16, A16, 8, 64, 1000)), A16, S) == pq.PQ_ERR_SHAPE
    assert f(b(pq.TernaryW(A16, A16, 0, 64, 1024)), A16, S) == pq.PQ_ERR_SHAPE
    assert f(b(pq.TernaryW(A1, A16, 8, 64, 1024)), A16, S) == pq.PQ_ERR_ALIGN
    assert f(b(pq.TernaryW(A16, A16, 8, 64, 1024)), A1, S) == pq.PQ_ERR_ALIGN


def test_decode1_gate_up_validation(L):
    import bit_quantized_moe_q8_amd as pq
    b = ctypes.byref
    tw = pq.TernaryW(A16, A16, 8, 256, 1024)
    f = L.pq_moe_decode1_gate_up_ternary
    args = lambda **kw: [kw.get("x", A16), kw.get("lg", A16), kw.get("E", 8), kw.get("k", 2),
                         b(kw.get("g", tw)), b(kw.get("u", tw))] + [A16] * 8 + [kw.get("y", A16), S]
    assert f(*args(x=None)) == pq.PQ_ERR_NULL
    assert f(*args(k=9)) == pq.PQ_ERR_SHAPE                                    # top_k > E
    assert f(*args(E=7)) == pq.PQ_ERR_SHAPE                                    # E != weights
    assert f(*args(u=pq.TernaryW(A16, A16, 8, 128, 1024))) == pq.PQ_ERR_SHAPE  # up shape
    assert f(*args(g=pq.TernaryW(A16, A16, 8, 256, 1024 + 256), u=pq.TernaryW(A16, A16, 8, 256, 1280))) \
        == pq.PQ_ERR_UNSUPPORTED                                               # cols/64 = 20
    assert f(*args(x=A1)) == pq.PQ_ERR_ALIGN
    assert f(*args(y=A1)) == pq.PQ_ERR_ALIGN
    gw = pq.Grid1W(A16, None, A16, A16, 8, 256, 1024)
    f2 = L.pq_moe_decode1_gate_up_grid1
    assert f2(A16, A16, 8, 2, b(gw), b(gw), *([A16] * 8), A16, S) == pq.PQ_ERR_NULL
    f3 = L.pq_moe_decode1_gate_up_sign1
    sw = pq.Sign1W(A16, A16, A16, 8, 256, 1024)
    assert f3(A16, A16, 8, 2, b(pq.Sign1W(A16, None, A16, 8, 256, 1024)), b(sw), *([A16] * 8), A16, S) \
        == pq.PQ_ERR_NULL                                                      # no sub-scales
    assert f3(A16, A16, 8, 2, b(pq.Sign1W(A16, ctypes.c_void_p(0x10002), A16, 8, 256, 1024)), b(sw),
              *([A16] * 8), A16, S) == pq.PQ_ERR_ALIGN                          # sc not 4-byte aligned
    assert f3(A16, A16, 8, 2, b(pq.Sign1W(A16, A16, A16, 8, 256, 768)), b(pq.Sign1W(A16, A16, A16, 8, 256, 768)),
              *([A16] * 8), A16, S) == pq.PQ_ERR_UNSUPPORTED                    # cols/128 = 6
    assert f3(A16, A16, 8, 9, b(sw), b(sw), *([A16] * 8), A16, S) == pq.PQ_ERR_SHAPE   # top_k > E


def test_gemm_validation(L):
    """The prefill GEMM entry points: grid1 and sub-scaled signs (cols % 512
    for the latter, sub-scales 16-byte aligned)."""
    import bit_quantized_moe_q8_amd as pq
    b = ctypes.byref
    g = _groups(pq)
    f = L.pq_moe_gemm_dequant_tile
    gw = pq.Grid1W(A16, A16, A16, A16, 8, 64, 1024)
    assert f(b(pq.Grid1W(A16, A16, A16, None, 8, 64, 1024)), None, b(g), A16, 1, 0, A16, None, S) == pq.PQ_ERR_NULL
    assert f(b(pq.Grid1W(A16, A16, A16, A16, 8, 64, 1000)), None, b(g), A16, 1, 0, A16, None, S) == pq.PQ_ERR_SHAPE
    assert f(b(gw), None, b(g), A1, 1, 0, A16, None, S) == pq.PQ_ERR_ALIGN
    assert f(b(gw), b(gw), b(g), A16, 1, 1, A16, None, S) == pq.PQ_ERR_UNSUPPORTED   # q8 epilogue
    f2 = L.pq_moe_gemm_dequant_tile_sign1
    sw = pq.Sign1W(A16, A16, A16, 8, 64, 1024)
    assert f2(b(pq.Sign1W(A16, None, A16, 8, 64, 1024)), None, b(g), A16, 1, 0, A16, None, S) == pq.PQ_ERR_NULL
    assert f2(b(pq.Sign1W(A16, A16, A16, 8, 64, 768)), None, b(g), A16, 1, 0, A16, None, S) \
        == pq.PQ_ERR_UNSUPPORTED                                                   # cols % 512 != 0
    assert f2(b(pq.Sign1W(A16, ctypes.c_void_p(0x10008), A16, 8, 64, 1024)), None, b(g), A16, 1, 0, A16,
              None, S) == pq.PQ_ERR_ALIGN                                          # sc 8-byte aligned only
    assert f2(b(sw), b(pq.Sign1W(A16, A16, A16, 8, 32, 1024)), b(g), A16, 1, 2, A16, None, S) \
        == pq.PQ_ERR_SHAPE                                                         # up shape
    assert f2(b(sw), None, b(_groups(pq, T=0)), None, 1, 0, A16, None, S) == pq.PQ_OK
