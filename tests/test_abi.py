"""The C-ABI library loads, exports every symbol include/coli.h declares, and
rejects bad arguments on the host before any HIP call (CPU only: none of
these calls reaches the device)."""
import ctypes
import os
import re

import pytest

import int4_routed_expert_sigmoid_amd as coli

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "coli.h")
FAKE = 0x1000   # never dereferenced: every call below fails validation first


def declared_functions():
    src = open(HEADER).read()
    src = re.sub(r"/\*.*?\*/", "", src, flags=re.S)
    src = re.sub(r"//[^\n]*", "", src)
    return sorted(set(re.findall(r"^\s*(?:const\s+)?\w+\s*\*?\s*(coli_\w+)\s*\(", src, re.M)))


def test_header_declares_the_boundary():
    names = declared_functions()
    for n in ("coli_quant_act_q8", "coli_route_topk", "coli_moe_forward"):
        assert n in names
    assert names == sorted(coli.EXPORTED)


def test_library_exports_every_declared_symbol():
    L = ctypes.CDLL(coli.LIB_PATH)
    for name in declared_functions():
        assert hasattr(L, name), name


def test_status_strings():
    L = coli.lib()
    for st in range(-6, 1):
        assert L.coli_status_string(st)
    assert L.coli_status_string(-99) == b"unknown status"


def test_table_bytes():
    L = coli.lib()
    sizes = [ctypes.c_size_t() for _ in range(4)]
    tot = L.coli_table_bytes(256, 1, 6144, 2048, 4, *[ctypes.byref(s) for s in sizes])
    # 257 experts x (3 * 6144 * 2048 / 2 nibble bytes + 4 * (2 * 2048 + 6144) scale bytes)
    assert tot == 257 * 18915328
    assert [s.value for s in sizes] == [257 * 6144 * 2048, 257 * 2 * 2048 * 4,
                                       257 * 6144 * 1024, 257 * 6144 * 4]
    # int8 tables: one byte per weight, the same scales
    tot = L.coli_table_bytes(256, 1, 6144, 2048, 8, *[ctypes.byref(s) for s in sizes])
    assert [s.value for s in sizes] == [257 * 6144 * 4096, 257 * 2 * 2048 * 4,
                                       257 * 6144 * 2048, 257 * 6144 * 4]
    assert tot == 257 * (3 * 6144 * 2048 + 4 * (2 * 2048 + 6144))
    assert L.coli_table_bytes(256, 1, 6144 + 32, 2048, 4, None, None, None, None) == 0  # D % 64
    assert L.coli_table_bytes(257, 1, 6144, 2048, 4, None, None, None, None) == 0
    assert L.coli_table_bytes(16, 2, 256, 128, 4, None, None, None, None) == 0
    assert L.coli_table_bytes(16, 0, 256, 128 + 16, 4, None, None, None, None) == 0
    for bits in (0, 3, 16):
        assert L.coli_table_bytes(16, 1, 256, 128, bits, None, None, None, None) == 0
    # int2 tables: four codes per byte, the same scales; d_ff % 64 == 0
    tot = L.coli_table_bytes(256, 1, 6144, 2048, 2, *[ctypes.byref(s) for s in sizes])
    assert [s.value for s in sizes] == [257 * 6144 * 1024, 257 * 2 * 2048 * 4,
                                       257 * 6144 * 512, 257 * 6144 * 4]
    assert L.coli_table_bytes(16, 1, 256, 96, 2, None, None, None, None) == 0
    # the limits of coli.h are accepted, one step past them is not
    assert L.coli_table_bytes(coli.COLI_MAX_EXPERTS, 1, coli.COLI_MAX_DIM, 64, 4, None, None, None, None) > 0
    assert L.coli_table_bytes(4, 1, 64, coli.COLI_MAX_DIM, 4, None, None, None, None) > 0
    assert L.coli_table_bytes(4, 1, coli.COLI_MAX_DIM + 64, 64, 4, None, None, None, None) == 0
    assert L.coli_table_bytes(4, 1, 64, coli.COLI_MAX_DIM + 32, 4, None, None, None, None) == 0


def _table(E=16, S=1, D=256, F=128, ptr=FAKE, bits=4, slots=0, slot_of=None):
    return coli.coli_expert_table(E, S, D, F, bits, ptr, ptr, ptr, ptr, slots, slot_of)


def test_validation_quant():
    L = coli.lib()
    assert L.coli_quant_act_q8(FAKE, 1, 33, FAKE, FAKE, None) == coli.COLI_E_SHAPE
    assert L.coli_quant_act_q8(FAKE, -1, 32, FAKE, FAKE, None) == coli.COLI_E_SHAPE
    assert L.coli_quant_act_q8(None, 1, 32, FAKE, FAKE, None) == coli.COLI_E_INVAL
    assert L.coli_quant_act_q8(None, 0, 32, None, None, None) == coli.COLI_OK      # no work
    assert L.coli_quant_weight_q4(FAKE, 4, 48, FAKE, FAKE, None) == coli.COLI_E_SHAPE
    assert L.coli_quant_weight_q4(FAKE, 4, 64, None, FAKE, None) == coli.COLI_E_INVAL
    assert L.coli_quant_weight_q8(FAKE, 4, 48, FAKE, FAKE, None) == coli.COLI_E_SHAPE
    assert L.coli_quant_weight_q8(FAKE, 4, 64, FAKE, None, None) == coli.COLI_E_INVAL
    assert L.coli_quant_weight_q8(FAKE + 4, 4, 64, FAKE, FAKE, None) == coli.COLI_E_INVAL
    assert L.coli_quant_weight_q8(None, 0, 64, None, None, None) == coli.COLI_OK
    assert L.coli_quant_weight_q2(FAKE, 4, 48, FAKE, FAKE, None) == coli.COLI_E_SHAPE
    assert L.coli_quant_weight_q2(FAKE, 4, 64, None, FAKE, None) == coli.COLI_E_INVAL
    assert L.coli_rmsnorm_q8(FAKE, 1, 40, 1e-6, FAKE, FAKE, None, None) == coli.COLI_E_SHAPE
    assert L.coli_rmsnorm_q8(FAKE, 1, 64, -1.0, FAKE, FAKE, None, None) == coli.COLI_E_INVAL
    assert L.coli_rmsnorm_q8(FAKE, 1, 64, float("nan"), FAKE, FAKE, None, None) == coli.COLI_E_INVAL


def test_validation_router_logits():
    L = coli.lib()
    f = L.coli_router_logits
    assert f(FAKE, FAKE, 1, 6144, 257, FAKE, None) == coli.COLI_E_SHAPE     # E > 256
    assert f(FAKE, FAKE, 1, 6144, 0, FAKE, None) == coli.COLI_E_SHAPE       # E = 0
    assert f(FAKE, FAKE, 1, 96, 16, FAKE, None) == coli.COLI_E_SHAPE        # D % 64
    assert f(FAKE, FAKE, -1, 64, 16, FAKE, None) == coli.COLI_E_SHAPE
    assert f(None, FAKE, 1, 64, 16, FAKE, None) == coli.COLI_E_INVAL
    assert f(FAKE + 4, FAKE, 1, 64, 16, FAKE, None) == coli.COLI_E_INVAL    # x not 16-byte aligned
    assert f(None, None, 0, 64, 16, None, None) == coli.COLI_OK             # T = 0


def test_validation_route_and_dispatch():
    L = coli.lib()
    r = L.coli_route_topk
    assert r(FAKE, None, 1, 0, 1, 1.0, FAKE, FAKE, None) == coli.COLI_E_SHAPE       # E = 0
    assert r(FAKE, None, 1, 257, 8, 1.0, FAKE, FAKE, None) == coli.COLI_E_SHAPE     # E > 256
    assert r(FAKE, None, 1, 16, 17, 1.0, FAKE, FAKE, None) == coli.COLI_E_SHAPE     # k > E
    assert r(FAKE, None, 1, 200, 65, 1.0, FAKE, FAKE, None) == coli.COLI_E_SHAPE    # k > 64
    assert r(FAKE, None, 1, 16, 0, 1.0, FAKE, FAKE, None) == coli.COLI_E_SHAPE
    assert r(None, None, 1, 16, 2, 1.0, FAKE, FAKE, None) == coli.COLI_E_INVAL
    assert r(FAKE, None, 1, 16, 2, float("inf"), FAKE, FAKE, None) == coli.COLI_E_INVAL
    assert r(None, None, 0, 16, 2, 1.0, None, None, None) == coli.COLI_OK          # T = 0
    d = L.coli_dispatch
    assert d(FAKE, 4, 2, 16, 2, FAKE, FAKE, FAKE, FAKE, FAKE, None) == coli.COLI_E_SHAPE   # S = 2
    assert d(FAKE, 4, 17, 16, 1, FAKE, FAKE, FAKE, FAKE, FAKE, None) == coli.COLI_E_SHAPE
    assert d(FAKE, 4, 2, 16, 1, FAKE, FAKE, None, FAKE, FAKE, None) == coli.COLI_E_INVAL
    assert d(FAKE, 2**31, 8, 256, 1, FAKE, FAKE, FAKE, FAKE, FAKE, None) == coli.COLI_E_SHAPE


def test_validation_forward():
    L = coli.lib()
    t = _table()
    ws = L.coli_moe_workspace_bytes(ctypes.byref(t), 4, 2)
    assert ws > 0
    f = L.coli_moe_forward
    args = lambda tab, T=4, k=2, acc=0, wsb=ws, y=FAKE: (ctypes.byref(tab), FAKE, FAKE, T, FAKE,
                                                          FAKE, k, y, acc, FAKE, wsb, None)
    assert f(*args(t, wsb=ws - 1)) == coli.COLI_E_WORKSPACE
    assert f(*args(t, k=0)) == coli.COLI_E_SHAPE
    assert f(*args(t, k=17)) == coli.COLI_E_SHAPE
    assert f(*args(t, acc=2)) == coli.COLI_E_INVAL
    assert f(*args(t, y=None)) == coli.COLI_E_INVAL
    assert f(*args(t, y=FAKE + 4)) == coli.COLI_E_INVAL      # y must be 16-byte aligned
    assert f(*args(_table(D=96))) == coli.COLI_E_SHAPE
    assert f(*args(_table(F=48))) == coli.COLI_E_SHAPE
    assert f(*args(_table(E=300))) == coli.COLI_E_SHAPE
    assert f(*args(_table(ptr=None))) == coli.COLI_E_INVAL
    assert f(*args(_table(bits=3))) == coli.COLI_E_SHAPE
    assert f(*args(_table(bits=0))) == coli.COLI_E_SHAPE
    assert f(*args(_table(F=96, bits=2))) == coli.COLI_E_SHAPE      # int2 needs d_ff % 64
    assert f(*args(t, T=0, wsb=0)) == coli.COLI_OK          # empty batch: nothing to do
    assert L.coli_moe_forward_traced(*args(t), None) == coli.COLI_E_INVAL
    assert L.coli_moe_status(None, 64, None) == coli.COLI_E_INVAL
    assert L.coli_table_set_expert(ctypes.byref(t), 17, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE,
                                   None) == coli.COLI_E_INVAL
    assert L.coli_table_set_expert(ctypes.byref(t), 0, None, FAKE, FAKE, FAKE, FAKE, FAKE,
                                   None) == coli.COLI_E_INVAL


def test_workspace_grows_with_tokens():
    L = coli.lib()
    t = _table(256, 1, 6144, 2048)
    a, b = (L.coli_moe_workspace_bytes(ctypes.byref(t), T, 8) for T in (1, 2048))
    assert 0 < a < b
    # per-pair outputs dominate: T (k+S) D fp32
    assert b >= 2048 * 9 * 6144 * 4


def test_validation_layer():
    L = coli.lib()
    t = _table()
    ws = L.coli_moe_layer_workspace_bytes(ctypes.byref(t), 4, 2)
    assert ws > L.coli_moe_workspace_bytes(ctypes.byref(t), 4, 2)
    f = L.coli_moe_layer
    args = lambda tab, T=4, k=2, sc=1.0, acc=0, wsb=ws, x=FAKE: (
        ctypes.byref(tab), x, FAKE, None, T, k, sc, FAKE, acc, FAKE, wsb, None)
    assert f(*args(t, wsb=ws - 1)) == coli.COLI_E_WORKSPACE
    assert f(*args(t, k=3 * 0)) == coli.COLI_E_SHAPE
    assert f(*args(t, sc=float("nan"))) == coli.COLI_E_INVAL
    assert f(*args(t, x=None)) == coli.COLI_E_INVAL
    assert f(*args(t, x=FAKE + 4)) == coli.COLI_E_INVAL     # x must be 16-byte aligned
    assert f(*args(t, acc=5)) == coli.COLI_E_INVAL
    assert f(*args(t, T=0, wsb=0)) == coli.COLI_OK


def test_validation_block():
    """coli_moe_block: the layer's checks plus eps, all before any HIP call."""
    L = coli.lib()
    t = _table()
    ws = L.coli_moe_layer_workspace_bytes(ctypes.byref(t), 4, 2)
    f = L.coli_moe_block
    args = lambda tab, T=4, k=2, sc=1.0, eps=1e-6, wsb=ws, h=FAKE: (
        ctypes.byref(tab), h, FAKE, None, T, k, sc, eps, FAKE, wsb, None)
    assert f(*args(t, wsb=ws - 1)) == coli.COLI_E_WORKSPACE
    assert f(*args(t, k=0)) == coli.COLI_E_SHAPE
    assert f(*args(t, eps=-1e-6)) == coli.COLI_E_INVAL
    assert f(*args(t, eps=float("nan"))) == coli.COLI_E_INVAL
    assert f(*args(t, eps=float("inf"))) == coli.COLI_E_INVAL
    assert f(*args(t, sc=float("nan"))) == coli.COLI_E_INVAL
    assert f(*args(t, h=None)) == coli.COLI_E_INVAL
    assert f(*args(t, h=FAKE + 4)) == coli.COLI_E_INVAL     # h must be 16-byte aligned
    assert f(*args(t, T=0, wsb=0)) == coli.COLI_OK


def test_tier_host_checks():
    """Tier entry points: sizes, rank (host logic), and argument checks."""
    import numpy as np
    L = coli.lib()
    sizes = [ctypes.c_size_t() for _ in range(4)]
    tot = L.coli_tier_table_bytes(32, 6144, 2048, 4, *[ctypes.byref(s) for s in sizes])
    assert tot == 32 * 18915328
    assert L.coli_tier_table_bytes(0, 6144, 2048, 4, None, None, None, None) == 0
    assert L.coli_tier_table_bytes(258, 6144, 2048, 4, None, None, None, None) == 0
    assert L.coli_tier_table_bytes(8, 6144, 2048, 3, None, None, None, None) == 0
    assert L.coli_tier_table_bytes(8, 6144, 2048, 2, None, None, None, None) == 8 * (
        3 * 6144 * 512 + 4 * (2 * 2048 + 6144))
    rng = np.random.default_rng(5)
    u = rng.integers(0, 6, size=256).astype(np.int32)
    assert coli.coli_tier_rank(u, 40).tolist() == sorted(range(256), key=lambda e: (-int(u[e]), e))[:40]
    assert L.coli_tier_rank(None, 16, 2, None) == coli.COLI_E_INVAL
    assert L.coli_tier_rank(FAKE, 16, 17, FAKE) == coli.COLI_E_SHAPE
    st = coli.coli_tier_state(*([FAKE] * 7))
    t = _table(slots=8, slot_of=FAKE)
    f = L.coli_tier_plan
    assert f(ctypes.byref(t), ctypes.byref(st), FAKE, 1, 0, 1, None) == coli.COLI_E_SHAPE
    assert f(ctypes.byref(t), ctypes.byref(st), FAKE, 1, 2, 2, None) == coli.COLI_E_INVAL
    assert f(ctypes.byref(_table(slots=8, slot_of=FAKE + 64)), ctypes.byref(st), FAKE, 1, 2, 1,
             None) == coli.COLI_E_INVAL                        # table map != state map
    assert f(ctypes.byref(_table(slots=18, slot_of=FAKE)), ctypes.byref(st), FAKE, 1, 2, 1,
             None) == coli.COLI_E_SHAPE                        # more slots than experts
    store = _table()
    pin = (ctypes.c_int32 * 3)(1, 2, 1)
    assert L.coli_tier_init(ctypes.byref(t), ctypes.byref(st), pin, 3, ctypes.byref(store),
                            None) == coli.COLI_E_INVAL                   # repeated pin
    pin = (ctypes.c_int32 * 8)(*range(8))
    assert L.coli_tier_init(ctypes.byref(t), ctypes.byref(st), pin, 8, ctypes.byref(store),
                            None) == coli.COLI_E_INVAL                   # 1 + 8 > 8 slots
    assert L.coli_tier_fetch(ctypes.byref(t), ctypes.byref(st), ctypes.byref(_table(E=15)),
                             None) == coli.COLI_E_SHAPE
    assert L.coli_tier_status(None, None) == coli.COLI_E_INVAL


def test_path_choice_host():
    """The automatic path choice (host logic) and the path argument's checks."""
    L = coli.lib()
    t = _table(256, 1, 6144, 2048)
    path = lambda tab, T, k=8: L.coli_moe_path(ctypes.byref(tab), T, k)
    assert path(t, 1) == coli.COLI_PATH_GEMV
    assert path(t, 4) == coli.COLI_PATH_GEMV
    assert path(t, 5) == coli.COLI_PATH_GROUPED
    assert path(t, 2048) == coli.COLI_PATH_GROUPED
    # no size limit on the grouped path: 2^17 tokens (1.2 M pairs) stay grouped
    assert path(t, 1 << 17) == coli.COLI_PATH_GROUPED
    assert path(_table(256, 1, 6144, 2048, bits=8), 2048) == coli.COLI_PATH_GEMV   # int8
    assert path(_table(256, 1, 6144, 2048, slots=64, slot_of=FAKE), 2048) == coli.COLI_PATH_GEMV
    assert path(t, 4, 0) == coli.COLI_E_SHAPE
    ws = L.coli_moe_workspace_bytes(ctypes.byref(t), 4, 8)
    f = L.coli_moe_forward_path
    args = lambda tab, p: (ctypes.byref(tab), FAKE, FAKE, 4, FAKE, FAKE, 8, FAKE, 0, FAKE, ws, p,
                           None)
    assert f(*args(t, 3)) == coli.COLI_E_INVAL
    assert f(*args(t, -1)) == coli.COLI_E_INVAL
    t8 = _table(256, 1, 6144, 2048, bits=8)
    assert f(*args(t8, coli.COLI_PATH_GROUPED)) == coli.COLI_E_SHAPE


def test_constants_match_header():
    """The binding's status codes, path ids and limits are the header's."""
    text = open(os.path.join(os.path.dirname(os.path.dirname(os.path.abspath(__file__))),
                             "include", "coli.h")).read()
    found = {m.group(1): int(m.group(2))
             for m in re.finditer(r"\b(COLI_[A-Z0-9_]+)\s*=\s*(-?\d+)", text)}
    found.update({m.group(1): int(m.group(2))
                  for m in re.finditer(r"#define\s+(COLI_[A-Z_]+)\s+(\d+)", text)})
    assert len(found) >= 13, sorted(found)
    for name, value in found.items():
        assert getattr(coli, name) == value, name
