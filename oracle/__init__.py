"""ctypes binding of the oracle (liboracle.so, built from coli_oracle.c).

TEST INFRASTRUCTURE ONLY: imported by tests/, __graft_entry__.smoke() and the
CPU-baseline leg of bench.py.  The product package never imports it.

Every function takes and returns numpy arrays on the host; the arithmetic
is all in coli_oracle.c.
"""
from __future__ import annotations

import ctypes
import os

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "liboracle.so")

_P = ctypes.c_void_p
_I64 = ctypes.c_int64
_I32 = ctypes.c_int32
_F = ctypes.c_float

_SIG = {
    "orc_num_threads": ([], ctypes.c_int),
    "orc_set_threads": ([ctypes.c_int], None),
    "orc_expf": ([_F], _F),
    "orc_sigmoidf": ([_F], _F),
    "orc_siluf": ([_F], _F),
    "orc_expf_vec": ([_P, _I64, _P], None),
    "orc_sigmoidf_vec": ([_P, _I64, _P], None),
    "orc_siluf_vec": ([_P, _I64, _P], None),
    "orc_q8_quant": ([_P, _I64, _P, _P], None),
    "orc_q4_quant_row": ([_P, _I64, _P, _P], None),
    "orc_q4_quant": ([_P, _I64, _I64, _P, _P], None),
    "orc_q8w_quant_row": ([_P, _I64, _P, _P], None),
    "orc_q2_quant_row": ([_P, _I64, _P, _P], None),
    "orc_q2_quant": ([_P, _I64, _I64, _P, _P], None),
    "orc_pack_q2": ([_P, _I64, _P], None),
    "orc_unpack_q2": ([_P, _I64, _P], None),
    "orc_q8w_quant": ([_P, _I64, _I64, _P, _P], None),
    "orc_pack_q4": ([_P, _I64, _P], None),
    "orc_unpack_q4": ([_P, _I64, _P], None),
    "orc_route": ([_P, _P, _I64, _I32, _I32, _F, _P, _P], None),
    "orc_row_partials": ([_P, ctypes.c_int, _P, _I64, _P], None),
    "orc_rescale": ([_P, _P, _I64, _F], _F),
    "orc_matvec": ([_P, ctypes.c_int, _P, _I64, _I64, _P, _P, _P, _P, _P], None),
    "orc_expert": ([_P] * 6 + [ctypes.c_int, _I64, _I64] + [_P] * 12, None),
    "orc_moe_layer": ([_P, ctypes.c_int, _I32, _I32, _I64, _I64, _I64, _P, _P, _P, _P, _I32, _P,
                       _P, ctypes.c_int, _P], ctypes.c_int),
    "orc_keep_entries": ([_P, _I64, _I32, _I32, _P], _I64),
    "orc_rmsnorm": ([_P, _I64, _I64, _F, _P, _P], None),
    "orc_router_logits": ([_P, _P, _I64, _I64, _I32, _P], None),
    "orc_dispatch": ([_P, _I64, _I32, _I32, _I32, _P, _P, _P, _P, _P], ctypes.c_int),
    "orc_tier_init": ([_I32, _I32, _I32, _P, _I32, _P, _P, _P, _P, _P, _P, _P], ctypes.c_int),
    "orc_tier_plan": ([_I32, _I32, _I32, _P, _I64, _I32, _I32, ctypes.c_int, _P, _P, _P, _P, _P,
                       _P, _P, _P], ctypes.c_int),
    "orc_tier_pin_top": ([_I32, _P, _I32, _P], None),
}


def _c(a, dtype):
    a = np.ascontiguousarray(a, dtype=dtype)
    return a


def _ptr(a):
    return None if a is None else a.ctypes.data


def _container(q, bits):
    """A weight container as the C side reads it: uint8 nibble pairs (bits 4),
    uint8 2-bit quadruples (bits 2) or int8 codes (bits 8)."""
    if bits in (2, 4):
        assert q.dtype == np.uint8, "the packed containers are uint8"
        return _c(q, np.uint8)
    assert bits == 8 and q.dtype == np.int8, "the int8 container is int8"
    return _c(q, np.int8)


class Expert:
    """One expert's canonical container (host arrays): the int4 nibble
    container (bits 4, uint8 [rows][k/2]) or the int8 one (bits 8, int8
    [rows][k]), with one f32 scale per row."""

    def __init__(self, gate_q, gate_s, up_q, up_s, down_q, down_s, bits=4):
        self.bits = bits
        self.gate_q = _container(np.asarray(gate_q), bits)
        self.gate_s = _c(gate_s, np.float32)
        self.up_q = _container(np.asarray(up_q), bits)
        self.up_s = _c(up_s, np.float32)
        self.down_q = _container(np.asarray(down_q), bits)
        self.down_s = _c(down_s, np.float32)

    @classmethod
    def quantize(cls, w_gate, w_up, w_down, orc=None, bits=4):
        """Quantise fp32 matrices with the oracle's per-row rule for `bits`."""
        orc = orc or get()
        quant = {4: orc.q4_quant, 8: orc.q8w_quant, 2: orc.q2_quant}[bits]
        gq, gs = quant(w_gate)
        uq, us = quant(w_up)
        dq, ds = quant(w_down)
        return cls(gq, gs, uq, us, dq, ds, bits=bits)

    def ptrs(self):
        return [_ptr(self.gate_q), _ptr(self.gate_s), _ptr(self.up_q), _ptr(self.up_s),
                _ptr(self.down_q), _ptr(self.down_s)]

    @property
    def D(self):
        return self.gate_q.shape[1] * (8 // self.bits)

    @property
    def F(self):
        return self.gate_q.shape[0]


class Oracle:
    """The oracle library at `path`, with numpy-in / numpy-out methods."""

    def __init__(self, path: str = LIB_PATH):
        if not os.path.exists(path):
            raise RuntimeError(f"{path} is not built; run __graft_entry__.build()")
        self.path = path
        self.L = ctypes.CDLL(path)
        for name, (args, res) in _SIG.items():
            fn = getattr(self.L, name)
            fn.argtypes = args
            fn.restype = res

    def num_threads(self) -> int:
        return int(self.L.orc_num_threads())

    def set_threads(self, n: int) -> None:
        """OpenMP threads of the calling thread's later oracle calls."""
        self.L.orc_set_threads(int(n))

    # ---------------------------------------------------------------- scalar math
    def expf(self, x: float) -> float:
        return self.L.orc_expf(x)

    def sigmoidf(self, x: float) -> float:
        return self.L.orc_sigmoidf(x)

    def siluf(self, x: float) -> float:
        return self.L.orc_siluf(x)

    def expf_vec(self, x):
        x = _c(x, np.float32)
        out = np.empty_like(x)
        self.L.orc_expf_vec(_ptr(x), x.size, _ptr(out))
        return out

    def sigmoidf_vec(self, x):
        x = _c(x, np.float32)
        out = np.empty_like(x)
        self.L.orc_sigmoidf_vec(_ptr(x), x.size, _ptr(out))
        return out

    def siluf_vec(self, x):
        x = _c(x, np.float32)
        out = np.empty_like(x)
        self.L.orc_siluf_vec(_ptr(x), x.size, _ptr(out))
        return out

    # ---------------------------------------------------------------- quantisers
    def q8_quant(self, x):
        """x [..., n] fp32 -> (q int8 [..., n], d fp32 [..., n/32])."""
        x = _c(x, np.float32)
        assert x.shape[-1] % 32 == 0
        q = np.empty(x.shape, dtype=np.int8)
        d = np.empty(x.shape[:-1] + (x.shape[-1] // 32,), dtype=np.float32)
        self.L.orc_q8_quant(_ptr(x), x.size, _ptr(q), _ptr(d))
        return q, d

    def q4_quant_row(self, w):
        w = _c(w, np.float32)
        q = np.empty(w.shape, dtype=np.int8)
        s = np.empty(1, dtype=np.float32)
        self.L.orc_q4_quant_row(_ptr(w), w.size, _ptr(q), _ptr(s))
        return q, float(s[0])

    def q4_quant(self, w):
        """w [rows][k] fp32 -> (packed uint8 [rows][k/2], s fp32 [rows])."""
        w = _c(w, np.float32)
        rows, k = w.shape
        packed = np.empty((rows, k // 2), dtype=np.uint8)
        s = np.empty(rows, dtype=np.float32)
        self.L.orc_q4_quant(_ptr(w), rows, k, _ptr(packed), _ptr(s))
        return packed, s

    def q8w_quant_row(self, w):
        w = _c(w, np.float32)
        q = np.empty(w.shape, dtype=np.int8)
        s = np.empty(1, dtype=np.float32)
        self.L.orc_q8w_quant_row(_ptr(w), w.size, _ptr(q), _ptr(s))
        return q, float(s[0])

    def q8w_quant(self, w):
        """w [rows][k] fp32 -> (int8 container [rows][k], s fp32 [rows])."""
        w = _c(w, np.float32)
        rows, k = w.shape
        q = np.empty((rows, k), dtype=np.int8)
        s = np.empty(rows, dtype=np.float32)
        self.L.orc_q8w_quant(_ptr(w), rows, k, _ptr(q), _ptr(s))
        return q, s

    def q2_quant_row(self, w):
        w = _c(w, np.float32)
        q = np.empty(w.shape, dtype=np.int8)
        s = np.empty(1, dtype=np.float32)
        self.L.orc_q2_quant_row(_ptr(w), w.size, _ptr(q), _ptr(s))
        return q, float(s[0])

    def q2_quant(self, w):
        """w [rows][k] fp32 -> (packed uint8 [rows][k/4], s fp32 [rows])."""
        w = _c(w, np.float32)
        rows, k = w.shape
        packed = np.empty((rows, k // 4), dtype=np.uint8)
        s = np.empty(rows, dtype=np.float32)
        self.L.orc_q2_quant(_ptr(w), rows, k, _ptr(packed), _ptr(s))
        return packed, s

    def pack_q2(self, q):
        q = _c(q, np.int8)
        out = np.empty(q.shape[:-1] + (q.shape[-1] // 4,), dtype=np.uint8)
        self.L.orc_pack_q2(_ptr(q), q.size, _ptr(out))
        return out

    def unpack_q2(self, packed):
        packed = _c(packed, np.uint8)
        q = np.empty(packed.shape[:-1] + (packed.shape[-1] * 4,), dtype=np.int8)
        self.L.orc_unpack_q2(_ptr(packed), q.size, _ptr(q))
        return q

    def pack_q4(self, q):
        q = _c(q, np.int8)
        out = np.empty(q.shape[:-1] + (q.shape[-1] // 2,), dtype=np.uint8)
        self.L.orc_pack_q4(_ptr(q), q.size, _ptr(out))
        return out

    def unpack_q4(self, packed):
        packed = _c(packed, np.uint8)
        q = np.empty(packed.shape[:-1] + (packed.shape[-1] * 2,), dtype=np.int8)
        self.L.orc_unpack_q4(_ptr(packed), q.size, _ptr(q))
        return q

    # ---------------------------------------------------------------- routing
    def route(self, logits, bias, k, routed_scale=1.0):
        logits = _c(logits, np.float32)
        bias = _c(bias, np.float32)
        T, E = logits.shape
        idx = np.empty((T, k), dtype=np.int32)
        w = np.empty((T, k), dtype=np.float32)
        self.L.orc_route(_ptr(logits), _ptr(bias), T, E, k, routed_scale, _ptr(idx), _ptr(w))
        return idx, w

    def keep_entries(self, idx, E):
        """keep [T][k] uint8: 1 for an entry the forward serves (in [0, E) and not
        a repeat of an earlier slot of its token); returns (keep, dropped)."""
        idx = _c(idx, np.int32)
        T, k = idx.shape
        keep = np.empty((T, k), dtype=np.uint8)
        n = self.L.orc_keep_entries(_ptr(idx), T, k, E, _ptr(keep))
        return keep, int(n)

    def dispatch(self, idx, E, S, keep=None):
        idx = _c(idx, np.int32)
        T, k = idx.shape
        if keep is not None:
            keep = _c(keep, np.uint8)
            assert keep.shape == idx.shape
        counts = np.zeros(E + S, dtype=np.int32)
        lists = np.full((E + S, T), -1, dtype=np.int32)
        n_active = np.zeros(1, dtype=np.int32)
        active = np.full(E + S, -1, dtype=np.int32)
        rc = self.L.orc_dispatch(_ptr(idx), T, k, E, S, _ptr(keep), _ptr(counts), _ptr(lists),
                                _ptr(n_active), _ptr(active))
        if rc != 0:
            raise ValueError("orc_dispatch rejected the index array")
        return counts, lists, int(n_active[0]), active[: int(n_active[0])]

    # ---------------------------------------------------------------- dots
    def row_partials(self, wrow, xq, bits=4):
        wrow = _container(np.asarray(wrow), bits)
        xq = _c(xq, np.int8)
        P = np.empty(xq.size // 32, dtype=np.int32)
        self.L.orc_row_partials(_ptr(wrow), bits, _ptr(xq), xq.size, _ptr(P))
        return P

    def rescale(self, P, d, s):
        P = _c(P, np.int32)
        d = _c(d, np.float32)
        return self.L.orc_rescale(_ptr(P), _ptr(d), P.size, s)

    def matvec(self, Wq, Ws, xq, xd, want_partials=False, want_absterm=False, bits=4):
        Wq = _container(np.asarray(Wq), bits)
        Ws = _c(Ws, np.float32)
        xq = _c(xq, np.int8)
        xd = _c(xd, np.float32)
        rows = Wq.shape[0]
        k = Wq.shape[1] * (8 // bits)
        y = np.empty(rows, dtype=np.float32)
        P = np.empty((rows, k // 32), dtype=np.int32) if want_partials else None
        A = np.empty(rows, dtype=np.float64) if want_absterm else None
        self.L.orc_matvec(_ptr(Wq), bits, _ptr(Ws), rows, k, _ptr(xq), _ptr(xd), _ptr(y), _ptr(P),
                          _ptr(A))
        return y, P, A

    def expert_forward(self, ex: Expert, xq, xd, want_partials=False):
        """One token through one expert; returns a dict of every intermediate."""
        D, F = ex.D, ex.F
        xq = _c(xq, np.int8)
        xd = _c(xd, np.float32)
        out = {
            "g": np.empty(F, np.float32), "u": np.empty(F, np.float32), "h": np.empty(F, np.float32),
            "hq": np.empty(F, np.int8), "hd": np.empty(F // 32, np.float32),
            "o": np.empty(D, np.float32), "abs_o": np.empty(D, np.float64),
        }
        if want_partials:
            out["P_gate"] = np.empty((F, D // 32), np.int32)
            out["P_up"] = np.empty((F, D // 32), np.int32)
            out["P_down"] = np.empty((D, F // 32), np.int32)
        self.L.orc_expert(*ex.ptrs(), ex.bits, D, F, _ptr(xq), _ptr(xd), _ptr(out["g"]),
                          _ptr(out["u"]),
                         _ptr(out["h"]), _ptr(out["hq"]), _ptr(out["hd"]), _ptr(out["o"]),
                         _ptr(out.get("P_gate")), _ptr(out.get("P_up")), _ptr(out.get("P_down")),
                         _ptr(out["abs_o"]))
        return out

    def moe_layer(self, experts, E, S, xq, xd, idx, w, out=None, accumulate=False, keep=None):
        """experts: dict or list mapping expert id (0..E+S-1) -> Expert (missing = unused).
        keep [T][k] (optional, keep_entries): the entries to serve; without it every
        entry must be valid.

        Returns (out [T][D] fp32, absterm [T][D] fp64)."""
        xq = _c(xq, np.int8)
        xd = _c(xd, np.float32)
        idx = _c(idx, np.int32)
        w = _c(w, np.float32)
        T, k = idx.shape
        if keep is not None:
            keep = _c(keep, np.uint8)
            assert keep.shape == idx.shape
        any_ex = next(iter(experts.values())) if isinstance(experts, dict) else experts[0]
        D, F, bits = any_ex.D, any_ex.F, any_ex.bits
        table = (ctypes.c_void_p * (6 * (E + S)))()
        for e in range(E + S):
            ex = experts.get(e) if isinstance(experts, dict) else experts[e]
            if ex is not None:
                assert ex.bits == bits, "one container kind per layer"
                for m, p in enumerate(ex.ptrs()):
                    table[6 * e + m] = p
        if out is None:
            out = np.zeros((T, D), dtype=np.float32)
        else:
            out = np.array(out, dtype=np.float32, copy=True, order="C")
        absterm = np.empty((T, D), dtype=np.float64)
        rc = self.L.orc_moe_layer(table, bits, E, S, D, F, T, _ptr(xq), _ptr(xd), _ptr(idx),
                                 _ptr(w), k, _ptr(keep), _ptr(out), int(bool(accumulate)),
                                 _ptr(absterm))
        if rc != 0:
            raise ValueError("orc_moe_layer: a selected expert is missing or an index is invalid")
        return out, absterm

    def router_logits(self, x, wr):
        """logits [T][E] = x [T][D] . wr [E][D]^T, fp64 sum in ascending d, rounded once."""
        x = _c(x, np.float32)
        wr = _c(wr, np.float32)
        T, D = x.shape
        E = wr.shape[0]
        out = np.empty((T, E), dtype=np.float32)
        self.L.orc_router_logits(_ptr(x), _ptr(wr), T, D, E, _ptr(out))
        return out

    def rmsnorm(self, h, eps):
        h = _c(h, np.float32)
        T, D = h.shape
        out = np.empty_like(h)
        r = np.empty(T, dtype=np.float32)
        self.L.orc_rmsnorm(_ptr(h), T, D, eps, _ptr(out), _ptr(r))
        return out, r


class Tier:
    """The oracle's expert tier of one layer (state in numpy arrays)."""

    def __init__(self, orc, E, S, slots, pin=()):
        self.orc, self.E, self.S, self.slots = orc, E, S, slots
        self.slot_of = np.empty(E + S, np.int32)
        self.expert_in = np.empty(slots, np.int32)
        self.stamp = np.empty(slots, np.int32)
        self.pinned = np.empty(slots, np.int32)
        self.usage = np.empty(E + S, np.int32)
        self.step = 0
        pin = _c(np.asarray(pin, np.int32), np.int32)
        loads = np.empty(slots, np.int32)
        n = np.zeros(1, np.int32)
        rc = orc.L.orc_tier_init(E, S, slots, _ptr(pin), pin.size, _ptr(self.slot_of),
                                 _ptr(self.expert_in), _ptr(self.stamp), _ptr(self.pinned),
                                 _ptr(self.usage), _ptr(loads), _ptr(n))
        if rc != 0:
            raise ValueError("orc_tier_init rejected the pin list")
        self.init_loads = loads[: int(n[0])].copy()

    def plan(self, idx, count_usage=True):
        """One pass: returns (loads: slots to fill in order, hits)."""
        idx = _c(idx, np.int32)
        T, k = idx.shape
        loads = np.empty(self.slots, np.int32)
        n = np.zeros(1, np.int32)
        hits = np.zeros(1, np.int32)
        rc = self.orc.L.orc_tier_plan(self.E, self.S, self.slots, _ptr(idx), T, k, self.step,
                                      int(bool(count_usage)), _ptr(self.slot_of),
                                      _ptr(self.expert_in), _ptr(self.stamp), _ptr(self.pinned),
                                      _ptr(self.usage), _ptr(loads), _ptr(n), _ptr(hits))
        if rc != 0:
            raise ValueError("orc_tier_plan: invalid index or not enough slots")
        self.step += 1
        return loads[: int(n[0])].copy(), int(hits[0])

    def pin_top(self, n):
        out = np.empty(n, np.int32)
        u = _c(self.usage, np.int32)
        self.orc.L.orc_tier_pin_top(self.E, _ptr(u), n, _ptr(out))
        return out


_default = None


def get() -> Oracle:
    """The oracle built in-tree (oracle/liboracle.so)."""
    global _default
    if _default is None:
        _default = Oracle()
    return _default


def __getattr__(name):
    # module-level access to the default oracle's methods: oracle.q8_quant(...)
    if name.startswith("_"):
        raise AttributeError(name)
    return getattr(get(), name)
