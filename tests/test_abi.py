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
    assert pq.abi_version() == 2
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


def test_decode_prep_validation(L):
    import bit_quantized_moe_q8_amd as pq
    f = L.pq_moe_decode_prep

    def args(T=4, H=256, E=64, k=8, x=A16, off=A16):
        return (x, A16, T, H, E, k, A16, A16, A16, A16, off, A16, A16, A16, None, S)

    assert f(*args(H=100)) == pq.PQ_ERR_SHAPE                # hidden % 32
    assert f(*args(k=65)) == pq.PQ_ERR_SHAPE                 # top_k > n_experts
    assert f(*args(T=(1 << 17) + 1)) == pq.PQ_ERR_SHAPE      # assignments > 2^20
    assert f(*args(x=None)) == pq.PQ_ERR_NULL
    assert f(*args(T=0, off=None)) == pq.PQ_ERR_NULL         # the grouping is written at 0 tokens too
    assert f(*args(x=A1)) == pq.PQ_ERR_ALIGN


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


def test_matvec_x32_validation(L):
    import bit_quantized_moe_q8_amd as pq
    b = ctypes.byref
    t, gr, sg = L.pq_matvec_x32_ternary, L.pq_matvec_x32_grid1, L.pq_matvec_x32_sign1
    ok_t = pq.TernaryW(A16, A16, 2, 64, 1024)
    # NULL weights, x or y
    assert t(None, 0, A16, A16, S) == pq.PQ_ERR_NULL
    assert t(b(pq.TernaryW(None, A16, 2, 64, 1024)), 0, A16, A16, S) == pq.PQ_ERR_NULL
    assert t(b(ok_t), 0, None, A16, S) == pq.PQ_ERR_NULL
    assert t(b(ok_t), 0, A16, None, S) == pq.PQ_ERR_NULL
    # expert outside [0, n_experts)
    assert t(b(ok_t), 2, A16, A16, S) == pq.PQ_ERR_SHAPE
    assert t(b(ok_t), -1, A16, A16, S) == pq.PQ_ERR_SHAPE
    # cols not a multiple of 256, rows < 1
    assert t(b(pq.TernaryW(A16, A16, 2, 64, 1000)), 0, A16, A16, S) == pq.PQ_ERR_SHAPE
    assert t(b(pq.TernaryW(A16, A16, 2, 0, 1024)), 0, A16, A16, S) == pq.PQ_ERR_SHAPE
    # misaligned x (16 bytes), codes
    assert t(b(ok_t), 0, ctypes.c_void_p(0x10004), A16, S) == pq.PQ_ERR_ALIGN
    assert t(b(pq.TernaryW(A1, A16, 2, 64, 1024)), 0, A16, A16, S) == pq.PQ_ERR_ALIGN
    # an unsupported (valid) width: cols/64 = 20
    assert t(b(pq.TernaryW(A16, A16, 2, 64, 1280)), 0, A16, A16, S) == pq.PQ_ERR_UNSUPPORTED
    assert gr(b(pq.Grid1W(A16, A16, A16, None, 1, 64, 1024)), 0, A16, A16, S) == pq.PQ_ERR_NULL
    assert gr(b(pq.Grid1W(A16, A16, A16, A1, 1, 64, 1024)), 0, A16, A16, S) == pq.PQ_ERR_ALIGN
    assert gr(b(pq.Grid1W(A16, A16, A16, A16, 1, 64, 2560)), 0, A16, A16, S) == pq.PQ_ERR_UNSUPPORTED
    assert sg(b(pq.Sign1W(A16, None, A16, 1, 64, 1024)), 0, A16, A16, S) == pq.PQ_ERR_NULL
    assert sg(b(pq.Sign1W(A16, A1, A16, 1, 64, 1024)), 0, A16, A16, S) == pq.PQ_ERR_ALIGN
    assert sg(b(pq.Sign1W(A16, A16, A16, 1, 64, 1024)), 1, A16, A16, S) == pq.PQ_ERR_SHAPE


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
    assert f(b(pq.Grid1W(A16, A16, A16, None, 8, 64, 1024)), None, b(g), A16, 1, 0, A16, None, None, S) == pq.PQ_ERR_NULL
    assert f(b(pq.Grid1W(A16, A16, A16, A16, 8, 64, 1000)), None, b(g), A16, 1, 0, A16, None, None, S) == pq.PQ_ERR_SHAPE
    assert f(b(gw), None, b(g), A1, 1, 0, A16, None, None, S) == pq.PQ_ERR_ALIGN
    assert f(b(gw), b(gw), b(g), A16, 1, 1, A16, None, None, S) == pq.PQ_ERR_UNSUPPORTED   # q8 epilogue
    assert f(b(gw), None, b(g), A16, 0, 3, A16, None, None, S) == pq.PQ_ERR_NULL   # fused combine: no topk_w
    assert f(b(gw), None, b(g), A16, 0, 3, A16, A1, None, S) == pq.PQ_ERR_ALIGN
    assert f(b(pq.Grid1W(A16, A16, A16, A16, 8, 60, 1024)), None, b(g), A16, 1, 0, A16, None, None, S) \
        == pq.PQ_ERR_SHAPE                                                         # rows % 8 != 0
    f2 = L.pq_moe_gemm_dequant_tile_sign1
    sw = pq.Sign1W(A16, A16, A16, 8, 64, 1024)
    assert f2(b(pq.Sign1W(A16, None, A16, 8, 64, 1024)), None, b(g), A16, 1, 0, A16, None, None, S) == pq.PQ_ERR_NULL
    assert f2(b(pq.Sign1W(A16, A16, A16, 8, 64, 768)), None, b(g), A16, 1, 0, A16, None, None, S) \
        == pq.PQ_ERR_UNSUPPORTED                                                   # cols % 512 != 0
    assert f2(b(pq.Sign1W(A16, ctypes.c_void_p(0x10008), A16, 8, 64, 1024)), None, b(g), A16, 1, 0, A16,
              None, None, S) == pq.PQ_ERR_ALIGN                                          # sc 8-byte aligned only
    assert f2(b(sw), b(pq.Sign1W(A16, A16, A16, 8, 32, 1024)), b(g), A16, 1, 2, A16, None, None, S) \
        == pq.PQ_ERR_SHAPE                                                         # up shape
    assert f2(b(sw), None, b(_groups(pq, T=0)), None, 1, 0, A16, None, None, S) == pq.PQ_OK
    assert f2(b(pq.Sign1W(A16, A16, A16, 8, 36, 1024)), None, b(g), A16, 1, 0, A16, None, None, S) \
        == pq.PQ_ERR_SHAPE                                                         # rows % 8 != 0


def test_tile_layout_validation(L):
    """pq_tile_layout_{grid1,sign1}: every check returns before a HIP call."""
    import bit_quantized_moe_q8_amd as pq
    b = ctypes.byref
    B, C, D = ctypes.c_void_p(0x200000), ctypes.c_void_p(0x400000), ctypes.c_void_p(0x600000)
    f = L.pq_tile_layout_grid1
    gw = pq.Grid1W(A16, ctypes.c_void_p(0x100000), A16, A16, 4, 64, 1024)   # qs 32 KB, qh 8 KB
    assert f(None, B, C, S) == pq.PQ_ERR_NULL
    assert f(b(gw), None, C, S) == pq.PQ_ERR_NULL
    assert f(b(pq.Grid1W(A16, A16, A16, A16, 4, 60, 1024)), B, C, S) == pq.PQ_ERR_SHAPE    # rows % 8
    assert f(b(pq.Grid1W(A16, A16, A16, A16, 4, 64, 1000)), B, C, S) == pq.PQ_ERR_SHAPE    # cols % 256
    assert f(b(pq.Grid1W(A16, A16, A16, A16, 0, 64, 1024)), B, C, S) == pq.PQ_ERR_SHAPE    # no experts
    assert f(b(gw), ctypes.c_void_p(0x200008), C, S) == pq.PQ_ERR_ALIGN
    assert f(b(gw), A16, C, S) == pq.PQ_ERR_SHAPE                  # output over the input qs
    assert f(b(gw), B, ctypes.c_void_p(0x201000), S) == pq.PQ_ERR_SHAPE   # the two outputs overlap
    assert f(b(gw), B, ctypes.c_void_p(0x100000 + 4096), S) == pq.PQ_ERR_SHAPE   # qh output over qh
    f2 = L.pq_tile_layout_sign1
    sw = pq.Sign1W(A16, ctypes.c_void_p(0x100000), A16, 4, 64, 1024)
    assert f2(b(sw), None, C, S) == pq.PQ_ERR_NULL
    assert f2(b(pq.Sign1W(A16, ctypes.c_void_p(0x100000), A16, 4, 64, 768)), B, C, S) == pq.PQ_ERR_SHAPE
    assert f2(b(pq.Sign1W(A16, ctypes.c_void_p(0x100000), A16, 4, 12, 1024)), B, C, S) == pq.PQ_ERR_SHAPE
    assert f2(b(sw), B, ctypes.c_void_p(0x400004), S) == pq.PQ_ERR_ALIGN
    assert f2(b(sw), D, D, S) == pq.PQ_ERR_SHAPE


# ------------------------------------------------------- dispatch plan (host only)

def test_plan_of_each_workload():
    """Which kernels each entry point launches at the workload shapes: the
    routed one-token gate/up at one token, the one-token mat-vec for its down
    projection, the grouped mat-vec at 8 tokens, the tile for the heavy experts
    of the skewed 64-token batch, the GEMM for prefill, every expert on the tile
    at 2048 tokens with q8 activations."""
    import bit_quantized_moe_q8_amd as pq
    P = pq
    # one token, ternary: gate/up routed launch, down one-token mat-vec
    assert pq.plan(P.PQ_CALL_DECODE1_GATE_UP, "ternary", 1, 8, 128, 768, 2048, P.PQ_EPI_SWIGLU_Q8) == P.PQ_PLAN_DECODE1_ROUTED
    assert pq.plan(P.PQ_CALL_MATVEC, "ternary", 1, 8, 128, 2048, 768, P.PQ_EPI_F32_COMBINE) == P.PQ_PLAN_MATVEC_TOK1
    # the debug outputs of a one-token call come from the grouped kernel
    assert pq.plan(P.PQ_CALL_MATVEC, "ternary", 1, 8, 128, 768, 2048, P.PQ_EPI_SWIGLU_Q8, True) == \
        P.PQ_PLAN_MATVEC | P.PQ_PLAN_DEBUG
    # 8 tokens over 256 grid1 experts: 64 assignments <= 256 experts
    for fmt in ("grid1", "sign1"):
        assert pq.plan(P.PQ_CALL_MATVEC, fmt, 8, 8, 256, 1536, 4096, P.PQ_EPI_SWIGLU_Q8) == P.PQ_PLAN_MATVEC
    # 64 skewed tokens: pairs of assignments, heavy experts on the tile
    assert pq.plan(P.PQ_CALL_MATVEC, "ternary", 64, 8, 256, 768, 2048, P.PQ_EPI_SWIGLU_Q8) == \
        P.PQ_PLAN_MATVEC_PAIRS | P.PQ_PLAN_TILE_Q8 | P.PQ_PLAN_MIXED
    # fewer than 8 tokens but more assignments than experts: pairs, no tile
    assert pq.plan(P.PQ_CALL_MATVEC, "ternary", 4, 2, 3, 256, 512) == P.PQ_PLAN_MATVEC_PAIRS
    # 2048 tokens with q8 activations: the mat-vec entry hands every expert
    # with 8+ assignments to the tile (all of them at this load)
    assert pq.plan(P.PQ_CALL_MATVEC, "grid1", 2048, 8, 256, 1536, 4096, P.PQ_EPI_SWIGLU_Q8) & P.PQ_PLAN_TILE_Q8
    assert pq.plan(P.PQ_CALL_TILE_Q8, "grid1", 2048, 8, 256, 1536, 4096, P.PQ_EPI_SWIGLU_Q8) == P.PQ_PLAN_TILE_Q8
    # prefill GEMM, both formats
    assert pq.plan(P.PQ_CALL_GEMM, "grid1", 2048, 8, 256, 1536, 4096, P.PQ_EPI_SWIGLU_BF16) == P.PQ_PLAN_GEMM
    assert pq.plan(P.PQ_CALL_GEMM, "sign1", 2048, 8, 256, 4096, 1536, P.PQ_EPI_F32) == P.PQ_PLAN_GEMM
    # sub-scaled signs on the GEMM need rows of a multiple of 512 weights
    assert pq.plan(P.PQ_CALL_GEMM, "sign1", 2048, 8, 256, 4096, 768, P.PQ_EPI_F32) == -P.PQ_ERR_UNSUPPORTED
    assert pq.plan(P.PQ_CALL_GEMM, "ternary", 2048, 8, 256, 1536, 4096, P.PQ_EPI_F32) == -P.PQ_ERR_UNSUPPORTED
    # the single 1024 x 1024 matrix: E = T = k = 1 takes the one-token kernel
    assert pq.plan(P.PQ_CALL_MATVEC, "ternary", 1, 1, 1, 1024, 1024) == P.PQ_PLAN_MATVEC_TOK1
    # nothing to do, invalid sizes
    assert pq.plan(P.PQ_CALL_MATVEC, "ternary", 0, 8, 128, 768, 2048) == 0
    assert pq.plan(P.PQ_CALL_MATVEC, "ternary", 1, 9, 8, 768, 2048) == -P.PQ_ERR_SHAPE
    assert pq.plan(P.PQ_CALL_MATVEC, "ternary", 1, 8, 128, 768, 2000) == -P.PQ_ERR_SHAPE
    assert pq.plan(P.PQ_CALL_MATVEC, "ternary", 1, 8, 128, 768, 8192) == -P.PQ_ERR_UNSUPPORTED
    assert pq.plan(P.PQ_CALL_DECODE1_GATE_UP, "grid1", 1, 8, 128, 768, 2048, P.PQ_EPI_SWIGLU_Q8, True) == \
        -P.PQ_ERR_UNSUPPORTED


# ------------------------------------------------ binding: sizes checked on the host

def _cpu_ternary(E, N, K):
    import torch
    import bit_quantized_moe_q8_amd as pq
    return pq.TernaryWeights(torch.zeros((E, N, K // 4), dtype=torch.uint8),
                             torch.zeros((E, N, K // 256), dtype=torch.int16))


def test_binding_rejects_undersized_buffers():
    """Every wrapper checks dtype and size of each buffer before the C call;
    host tensors of the wrong size raise ValueError/TypeError before the
    device check (so nothing here needs a GPU)."""
    import torch
    import bit_quantized_moe_q8_amd as pq
    f32, i8, i32 = torch.float32, torch.int8, torch.int32
    x = torch.zeros((2, 64), dtype=f32)
    with pytest.raises(ValueError, match="xq"):
        pq.quantize_act_q8(x, torch.zeros(127, dtype=i8), torch.zeros(4, dtype=f32))
    with pytest.raises(ValueError, match="xd"):
        pq.quantize_act_q8(x, torch.zeros(128, dtype=i8), torch.zeros(3, dtype=f32))
    with pytest.raises(TypeError):
        pq.quantize_act_q8(x, torch.zeros(128, dtype=i32), torch.zeros(4, dtype=f32))
    lg = torch.zeros((3, 16), dtype=f32)
    with pytest.raises(ValueError, match="ids"):
        pq.moe_route_topk(lg, 4, torch.zeros(11, dtype=i32), torch.zeros(12, dtype=f32))
    ids = torch.zeros((3, 4), dtype=i32)
    g = pq.GroupBuffers(torch.zeros(16, dtype=i32), torch.zeros(12, dtype=i32), torch.zeros(16, dtype=i32),
                        torch.zeros(1, dtype=i32), 3, 4, 16)
    with pytest.raises(ValueError, match="expert_offsets"):
        pq.group_tokens_by_expert(ids, 16, g)
    g = pq.GroupBuffers.empty(3, 4, 16, "cpu")
    with pytest.raises(ValueError, match="n_experts"):
        pq.group_tokens_by_expert(ids, 8, g)
    # mat-vec: activations, outputs, weights, debug
    W = _cpu_ternary(16, 64, 256)
    xq, xd = torch.zeros((3, 256), dtype=i8), torch.zeros((3, 8), dtype=f32)
    with pytest.raises(ValueError, match="xq"):
        pq.moe_matvec_ternary(W, None, g, xq, xd, False)      # by assignment: 12 rows needed
    xq12, xd12 = torch.zeros((12, 256), dtype=i8), torch.zeros((12, 8), dtype=f32)
    with pytest.raises(ValueError, match="out0"):
        pq.moe_matvec_ternary(W, None, g, xq12, xd12, False, pq.PQ_EPI_F32, torch.zeros((12, 63), dtype=f32))
    with pytest.raises(ValueError, match="hd"):
        pq.moe_matvec_ternary(W, W, g, xq, xd, True, pq.PQ_EPI_SWIGLU_Q8, torch.zeros((12, 64), dtype=i8),
                              torch.zeros((12, 1), dtype=f32))
    with pytest.raises(ValueError, match="topk_w"):
        pq.moe_matvec_ternary(W, None, g, xq12, xd12, False, pq.PQ_EPI_F32_COMBINE,
                              torch.zeros((3, 64), dtype=f32), torch.zeros(11, dtype=f32))
    with pytest.raises(ValueError, match="w_up"):
        pq.moe_matvec_ternary(W, _cpu_ternary(16, 32, 256), g, xq, xd, True, pq.PQ_EPI_SWIGLU_Q8)
    with pytest.raises(ValueError, match="dbg isums"):
        pq.moe_matvec_ternary(W, None, g, xq12, xd12, False, dbg={"isums": torch.zeros(10, dtype=i32)})
    bad_d = pq.TernaryWeights(W.qs, torch.zeros((16, 64, 2), dtype=torch.int16))
    with pytest.raises(ValueError, match="d has shape"):
        pq.moe_matvec_ternary(bad_d, None, g, xq12, xd12, False, pq.PQ_EPI_F32, torch.zeros((12, 64), dtype=f32))
    # single mat-vec from fp32 activations: expert range, x and y sizes, dtype
    x256 = torch.zeros(256, dtype=f32)
    with pytest.raises(ValueError, match="expert"):
        pq.matvec_x32(W, x256, 16)
    with pytest.raises(ValueError, match="x holds"):
        pq.matvec_x32(W, torch.zeros(255, dtype=f32), 0)
    with pytest.raises(ValueError, match="y holds"):
        pq.matvec_x32(W, x256, 0, torch.zeros(63, dtype=f32))
    with pytest.raises(TypeError):
        pq.matvec_x32(W, torch.zeros(256, dtype=torch.float16), 0)
    # GEMM and combine
    Wg = pq.Grid1Weights(torch.zeros((16, 64, 32), dtype=torch.uint8), torch.zeros((16, 64, 8), dtype=torch.int16),
                         torch.zeros((16, 64, 1), dtype=torch.int16), torch.zeros((2048, 8), dtype=i8), tiled=True)
    with pytest.raises(ValueError, match="x holds"):
        pq.moe_gemm_dequant_tile(Wg, None, g, torch.zeros((3, 256), dtype=torch.bfloat16), False)
    with pytest.raises(ValueError, match="grid"):
        pq.moe_gemm_dequant_tile(pq.Grid1Weights(Wg.qs, Wg.qh, Wg.d, torch.zeros(100, dtype=i8), tiled=True), None,
                                 g, torch.zeros((12, 256), dtype=torch.bfloat16), False, pq.PQ_EPI_F32,
                                 torch.zeros((12, 64), dtype=f32))
    with pytest.raises(ValueError, match="tile layout"):   # the GEMM reads only the tile layout
        pq.moe_gemm_dequant_tile(pq.Grid1Weights(Wg.qs, Wg.qh, Wg.d, Wg.grid), None, g,
                                 torch.zeros((12, 256), dtype=torch.bfloat16), False)
    with pytest.raises(ValueError, match="tile layout"):   # and the mat-vec never does
        pq.moe_matvec_grid1(Wg, None, g, torch.zeros((12, 256), dtype=i8), torch.zeros((12, 8), dtype=f32), False)
    with pytest.raises(ValueError, match="tile layout"):
        pq.tile_layout(Wg)
    with pytest.raises(ValueError, match="topk_w"):
        pq.moe_combine(torch.zeros((12, 64), dtype=f32), torch.zeros(11, dtype=f32), 4)
    with pytest.raises(ValueError, match="multiple of top_k"):
        pq.moe_combine(torch.zeros((10, 64), dtype=f32), torch.zeros(12, dtype=f32), 4)
    # one-token gate/up
    g1 = pq.GroupBuffers.empty(1, 4, 16, "cpu")
    with pytest.raises(ValueError, match="hq"):
        pq.moe_decode1_gate_up(W, W, torch.zeros((1, 256), dtype=f32), torch.zeros((1, 16), dtype=f32), 4,
                               torch.zeros(4, dtype=i32), torch.zeros(4, dtype=f32), g1,
                               torch.zeros((4, 63), dtype=i8), torch.zeros((4, 2), dtype=f32))
    with pytest.raises(ValueError, match="experts"):
        pq.moe_decode1_gate_up(W, W, torch.zeros((1, 256), dtype=f32), torch.zeros((1, 8), dtype=f32), 4,
                               torch.zeros(4, dtype=i32), torch.zeros(4, dtype=f32), g1,
                               torch.zeros((4, 64), dtype=i8), torch.zeros((4, 2), dtype=f32))
