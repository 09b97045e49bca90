"""Python binding of libcoli.so, the gfx950 routed int4 MoE FFN library.

Argument marshalling only: every function here forwards torch CUDA tensors'
device pointers and the current HIP stream to the C ABI of include/coli.h
under the same name, and raises ColiError on a non-OK status.  All
arithmetic runs in the library's HIP kernels; if the library is missing the
import still succeeds but every call raises.

torch provides device memory and streams only.
"""
from __future__ import annotations

import ctypes
import os

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "libcoli.so")

COLI_OK = 0
COLI_E_INVAL = -1
COLI_E_SHAPE = -2
COLI_E_WORKSPACE = -3
COLI_E_DEVICE = -4
COLI_E_HIP = -5
COLI_E_INDEX = -6
COLI_E_TIER = -7
COLI_PATH_AUTO, COLI_PATH_GEMV, COLI_PATH_GROUPED = 0, 1, 2
COLI_GROUPED_MIN_TOKENS = 5
COLI_NOALLOC_BYTES = 64 << 20
COLI_MAX_EXPERTS = 256
COLI_MAX_TOPK = 64
COLI_MAX_DIM = 32768

EXPORTED = [
    "coli_table_bytes", "coli_table_set_expert", "coli_quant_act_q8", "coli_quant_weight_q4",
    "coli_quant_weight_q8", "coli_quant_weight_q2",
    "coli_rmsnorm_q8", "coli_route_topk", "coli_router_logits", "coli_dispatch",
    "coli_moe_workspace_bytes",
    "coli_moe_forward", "coli_moe_forward_traced", "coli_moe_forward_profiled",
    "coli_moe_forward_path", "coli_moe_path",
    "coli_moe_layer_workspace_bytes", "coli_moe_layer", "coli_moe_layer_ex", "coli_moe_block",
    "coli_moe_layer_noalloc",
    "coli_moe_status", "coli_status_string", "coli_last_hip_error",
    "coli_tier_table_bytes", "coli_tier_init", "coli_tier_plan", "coli_tier_fetch",
    "coli_tier_status", "coli_tier_rank",
]


class ColiError(RuntimeError):
    def __init__(self, fn: str, status: int, hip: int = 0):
        msg = f"{fn}: status {status}"
        if _lib is not None:
            msg += f" ({_lib.coli_status_string(status).decode()})"
        if status == COLI_E_HIP:
            msg += f", hipError {hip}"
        super().__init__(msg)
        self.status = status


class coli_expert_table(ctypes.Structure):
    _fields_ = [("n_routed", ctypes.c_int32), ("n_shared", ctypes.c_int32),
                ("d_model", ctypes.c_int32), ("d_ff", ctypes.c_int32),
                ("weight_bits", ctypes.c_int32), ("gu_q", ctypes.c_void_p), ("gu_s", ctypes.c_void_p),
                ("dn_q", ctypes.c_void_p), ("dn_s", ctypes.c_void_p),
                ("n_slots", ctypes.c_int32), ("slot_of", ctypes.c_void_p)]


class coli_tier_state(ctypes.Structure):
    _fields_ = [(n, ctypes.c_void_p) for n in
                ("slot_of", "expert_in", "stamp", "pinned", "usage", "loads", "counters")]


class coli_moe_events(ctypes.Structure):
    _fields_ = [(n, ctypes.c_void_p) for n in ("begin", "gate_up", "down", "combine", "end")]


class coli_moe_trace(ctypes.Structure):
    _fields_ = [(n, ctypes.c_void_p) for n in
                ("counts", "lists", "n_active", "active", "p_gate", "p_up", "p_down", "g", "u",
                 "h", "hq", "hd", "o", "xq", "xd", "idx", "w")]


_lib = None
_P = ctypes.c_void_p
_I64 = ctypes.c_int64
_I32 = ctypes.c_int32


def lib():
    """The loaded library; raises if libcoli.so was not built."""
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            raise RuntimeError(f"{LIB_PATH} is missing: run __graft_entry__.build() first")
        L = ctypes.CDLL(LIB_PATH)
        sz = ctypes.c_size_t
        sig = {
            "coli_table_bytes": ([_I32, _I32, _I64, _I64, _I32, _P, _P, _P, _P], sz),
            "coli_table_set_expert": ([_P, _I32, _P, _P, _P, _P, _P, _P, _P], ctypes.c_int),
            "coli_quant_act_q8": ([_P, _I64, _I64, _P, _P, _P], ctypes.c_int),
            "coli_quant_weight_q4": ([_P, _I64, _I64, _P, _P, _P], ctypes.c_int),
            "coli_quant_weight_q8": ([_P, _I64, _I64, _P, _P, _P], ctypes.c_int),
            "coli_quant_weight_q2": ([_P, _I64, _I64, _P, _P, _P], ctypes.c_int),
            "coli_rmsnorm_q8": ([_P, _I64, _I64, ctypes.c_float, _P, _P, _P, _P], ctypes.c_int),
            "coli_route_topk": ([_P, _P, _I64, _I32, _I32, ctypes.c_float, _P, _P, _P],
                                ctypes.c_int),
            "coli_router_logits": ([_P, _P, _I64, _I64, _I32, _P, _P], ctypes.c_int),
            "coli_dispatch": ([_P, _I64, _I32, _I32, _I32, _P, _P, _P, _P, _P, _P], ctypes.c_int),
            "coli_moe_workspace_bytes": ([_P, _I64, _I32], sz),
            "coli_moe_forward": ([_P, _P, _P, _I64, _P, _P, _I32, _P, ctypes.c_int, _P, sz, _P],
                                 ctypes.c_int),
            "coli_moe_forward_traced": ([_P, _P, _P, _I64, _P, _P, _I32, _P, ctypes.c_int, _P,
                                         sz, _P, _P], ctypes.c_int),
            "coli_moe_forward_profiled": ([_P, _P, _P, _I64, _P, _P, _I32, _P, ctypes.c_int, _P,
                                           sz, _P, _P], ctypes.c_int),
            "coli_moe_forward_path": ([_P, _P, _P, _I64, _P, _P, _I32, _P, ctypes.c_int, _P, sz,
                                       _I32, _P], ctypes.c_int),
            "coli_moe_path": ([_P, _I64, _I32], ctypes.c_int),
            "coli_moe_layer_workspace_bytes": ([_P, _I64, _I32], sz),
            "coli_moe_layer": ([_P, _P, _P, _P, _I64, _I32, ctypes.c_float, _P, ctypes.c_int, _P,
                                sz, _P], ctypes.c_int),
            "coli_moe_layer_ex": ([_P, _P, _P, _P, _I64, _I32, ctypes.c_float, _P, ctypes.c_int,
                                   _P, sz, _P, _P, _P], ctypes.c_int),
            "coli_moe_block": ([_P, _P, _P, _P, _I64, _I32, ctypes.c_float, ctypes.c_float, _P,
                                sz, _P], ctypes.c_int),
            "coli_moe_layer_noalloc": ([_P, _P, _P, _P, _I64, _I32, ctypes.c_float, _P,
                                        ctypes.c_int, _P], ctypes.c_int),
            "coli_moe_status": ([_P, sz, _P], ctypes.c_int),
            "coli_status_string": ([ctypes.c_int], ctypes.c_char_p),
            "coli_tier_table_bytes": ([_I32, _I64, _I64, _I32, _P, _P, _P, _P], sz),
            "coli_tier_init": ([_P, _P, _P, _I32, _P, _P], ctypes.c_int),
            "coli_tier_plan": ([_P, _P, _P, _I64, _I32, _I32, _P], ctypes.c_int),
            "coli_tier_fetch": ([_P, _P, _P, _P], ctypes.c_int),
            "coli_tier_status": ([_P, _P], ctypes.c_int),
            "coli_tier_rank": ([_P, _I32, _I32, _P], ctypes.c_int),
            "coli_last_hip_error": ([], ctypes.c_int),
        }
        for name, (args, res) in sig.items():
            fn = getattr(L, name)
            fn.argtypes = args
            fn.restype = res
        _lib = L
    return _lib


def _check(fn: str, status: int) -> None:
    if status != COLI_OK:
        raise ColiError(fn, status, lib().coli_last_hip_error() if status == COLI_E_HIP else 0)


def _ptr(t):
    """Device pointer of a tensor (None -> NULL)."""
    if t is None:
        return None
    if not t.is_contiguous():
        raise ValueError("tensor arguments must be contiguous")
    return t.data_ptr()


def _stream(stream):
    if stream is not None:
        return stream
    import torch
    return torch.cuda.current_stream().cuda_stream


def _dtype(t, dt, name):
    if t is not None and t.dtype != dt:
        raise TypeError(f"{name} must be {dt}, got {t.dtype}")


# --------------------------------------------------------------------------- table
class ExpertTable:
    """A device-resident expert table (torch-allocated) and its C descriptor.
    weight_bits 4: int4 nibble codes; 8: int8 codes (the int8 head); 2: 2-bit codes."""

    def __init__(self, n_routed: int, n_shared: int, d_model: int, d_ff: int, device="cuda",
                 weight_bits: int = 4, _arrays=None):
        import torch
        self.E, self.S, self.D, self.F = n_routed, n_shared, d_model, d_ff
        self.weight_bits = weight_bits
        if _arrays is None:
            sizes = [ctypes.c_size_t() for _ in range(4)]
            total = lib().coli_table_bytes(n_routed, n_shared, d_model, d_ff, weight_bits,
                                           *[ctypes.byref(s) for s in sizes])
            if total == 0:
                raise ColiError("coli_table_bytes", COLI_E_SHAPE)
            _arrays = (torch.empty(sizes[0].value, dtype=torch.uint8, device=device),
                       torch.empty(sizes[1].value // 4, dtype=torch.float32, device=device),
                       torch.empty(sizes[2].value, dtype=torch.uint8, device=device),
                       torch.empty(sizes[3].value // 4, dtype=torch.float32, device=device))
        self.gu_q, self.gu_s, self.dn_q, self.dn_s = _arrays
        self.bytes = sum(a.numel() * a.element_size() for a in _arrays)
        self.c = coli_expert_table(n_routed, n_shared, d_model, d_ff, weight_bits,
                                   self.gu_q.data_ptr(), self.gu_s.data_ptr(),
                                   self.dn_q.data_ptr(), self.dn_s.data_ptr(), 0, None)

    def ref(self):
        return ctypes.byref(self.c)

    def to_host_store(self):
        """A copy of the table in pinned host memory: the store of an ExpertTier."""
        import torch
        arrays = []
        for a in (self.gu_q, self.gu_s, self.dn_q, self.dn_s):
            h = torch.empty(a.shape, dtype=a.dtype, pin_memory=True)   # hipHostMalloc'd
            h.copy_(a)
            arrays.append(h)
        arrays = tuple(arrays)
        return ExpertTable(self.E, self.S, self.D, self.F, weight_bits=self.weight_bits,
                           _arrays=arrays)


class ExpertTier:
    """An HBM tier of `slots` experts of one layer (table storage + device
    state), filled from a store by coli_tier_plan / coli_tier_fetch."""

    def __init__(self, n_routed: int, n_shared: int, d_model: int, d_ff: int, slots: int,
                 weight_bits: int = 4, device="cuda"):
        import torch
        sizes = [ctypes.c_size_t() for _ in range(4)]
        total = lib().coli_tier_table_bytes(slots, d_model, d_ff, weight_bits,
                                            *[ctypes.byref(s) for s in sizes])
        if total == 0:
            raise ColiError("coli_tier_table_bytes", COLI_E_SHAPE)
        self.E, self.S, self.D, self.F, self.slots = n_routed, n_shared, d_model, d_ff, slots
        self.weight_bits = weight_bits
        i32 = dict(dtype=torch.int32, device=device)
        A = n_routed + n_shared
        self.st = {"slot_of": torch.full((A,), -1, **i32),
                   "expert_in": torch.full((slots,), -1, **i32),
                   "stamp": torch.full((slots,), -1, **i32),
                   "pinned": torch.zeros(slots, **i32), "usage": torch.zeros(A, **i32),
                   "loads": torch.zeros(1 + slots, **i32), "counters": torch.zeros(4, **i32)}
        self.state = coli_tier_state(*[self.st[n].data_ptr() for n, _ in coli_tier_state._fields_])
        self.gu_q = torch.empty(sizes[0].value, dtype=torch.uint8, device=device)
        self.gu_s = torch.empty(sizes[1].value // 4, dtype=torch.float32, device=device)
        self.dn_q = torch.empty(sizes[2].value, dtype=torch.uint8, device=device)
        self.dn_s = torch.empty(sizes[3].value // 4, dtype=torch.float32, device=device)
        self.bytes = total
        self.c = coli_expert_table(n_routed, n_shared, d_model, d_ff, weight_bits,
                                   self.gu_q.data_ptr(), self.gu_s.data_ptr(),
                                   self.dn_q.data_ptr(), self.dn_s.data_ptr(), slots,
                                   self.st["slot_of"].data_ptr())

    def ref(self):
        """The tier as a table: pass it to coli_moe_forward / coli_moe_layer."""
        return ctypes.byref(self.c)

    def init(self, store: "ExpertTable", pin=(), stream=None):
        """Reset; the shared expert and the pinned ones are filled from store."""
        arr = (ctypes.c_int32 * max(1, len(pin)))(*[int(e) for e in pin])
        _check("coli_tier_init", lib().coli_tier_init(self.ref(), ctypes.byref(self.state), arr,
                                                       len(pin), store.ref(), _stream(stream)))

    def plan(self, idx, count_usage=True, stream=None):
        import torch
        _dtype(idx, torch.int32, "idx")
        T, k = idx.shape
        _check("coli_tier_plan", lib().coli_tier_plan(self.ref(), ctypes.byref(self.state),
                                                       _ptr(idx), T, k, int(bool(count_usage)),
                                                       _stream(stream)))

    def fetch(self, store: "ExpertTable", stream=None):
        _check("coli_tier_fetch", lib().coli_tier_fetch(self.ref(), ctypes.byref(self.state),
                                                         store.ref(), _stream(stream)))

    def status(self, stream=None) -> int:
        return int(lib().coli_tier_status(ctypes.byref(self.state), _stream(stream)))


def coli_tier_rank(usage, n: int):
    """The n routed experts with the largest usage (host numpy int32 [E])."""
    import numpy as np
    u = np.ascontiguousarray(usage, dtype=np.int32)
    out = np.empty(n, dtype=np.int32)
    _check("coli_tier_rank", lib().coli_tier_rank(u.ctypes.data, u.size, n, out.ctypes.data))
    return out


def coli_table_set_expert(table: ExpertTable, expert: int, gate_q, gate_s, up_q, up_s, down_q,
                          down_s, stream=None):
    _check("coli_table_set_expert",
           lib().coli_table_set_expert(table.ref(), expert, _ptr(gate_q), _ptr(gate_s),
                                       _ptr(up_q), _ptr(up_s), _ptr(down_q), _ptr(down_s),
                                       _stream(stream)))


# --------------------------------------------------------------------------- quantisers
def coli_quant_act_q8(x, q, d, stream=None):
    import torch
    _dtype(x, torch.float32, "x"); _dtype(q, torch.int8, "q"); _dtype(d, torch.float32, "d")
    rows, k = (x.shape[0], x.shape[1]) if x.dim() == 2 else (1, x.shape[0])
    _check("coli_quant_act_q8",
           lib().coli_quant_act_q8(_ptr(x), rows, k, _ptr(q), _ptr(d), _stream(stream)))


def coli_quant_weight_q4(w, q, s, stream=None):
    import torch
    _dtype(w, torch.float32, "w"); _dtype(q, torch.uint8, "q"); _dtype(s, torch.float32, "s")
    rows, k = w.shape
    _check("coli_quant_weight_q4",
           lib().coli_quant_weight_q4(_ptr(w), rows, k, _ptr(q), _ptr(s), _stream(stream)))


def coli_quant_weight_q8(w, q, s, stream=None):
    import torch
    _dtype(w, torch.float32, "w"); _dtype(q, torch.int8, "q"); _dtype(s, torch.float32, "s")
    rows, k = w.shape
    _check("coli_quant_weight_q8",
           lib().coli_quant_weight_q8(_ptr(w), rows, k, _ptr(q), _ptr(s), _stream(stream)))


def coli_quant_weight_q2(w, q, s, stream=None):
    import torch
    _dtype(w, torch.float32, "w"); _dtype(q, torch.uint8, "q"); _dtype(s, torch.float32, "s")
    rows, k = w.shape
    _check("coli_quant_weight_q2",
           lib().coli_quant_weight_q2(_ptr(w), rows, k, _ptr(q), _ptr(s), _stream(stream)))


def coli_rmsnorm_q8(h, eps, q, d, r_out=None, stream=None):
    import torch
    _dtype(h, torch.float32, "h"); _dtype(q, torch.int8, "q"); _dtype(d, torch.float32, "d")
    T, D = h.shape
    _check("coli_rmsnorm_q8", lib().coli_rmsnorm_q8(_ptr(h), T, D, eps, _ptr(q), _ptr(d),
                                                    _ptr(r_out), _stream(stream)))


# --------------------------------------------------------------------------- routing
def coli_router_logits(x, wr, logits, stream=None):
    """logits [T][E] = x [T][D] . wr [E][D]^T (F32 router weights, fp64 sum)."""
    import torch
    _dtype(x, torch.float32, "x"); _dtype(wr, torch.float32, "wr")
    _dtype(logits, torch.float32, "logits")
    T, D = x.shape
    E = wr.shape[0]
    _check("coli_router_logits", lib().coli_router_logits(_ptr(x), _ptr(wr), T, D, E, _ptr(logits),
                                                          _stream(stream)))


def coli_route_topk(logits, bias, k, idx, w, routed_scale=1.0, stream=None):
    import torch
    _dtype(logits, torch.float32, "logits"); _dtype(bias, torch.float32, "bias")
    _dtype(idx, torch.int32, "idx"); _dtype(w, torch.float32, "w")
    T, E = logits.shape
    _check("coli_route_topk", lib().coli_route_topk(_ptr(logits), _ptr(bias), T, E, k,
                                                    routed_scale, _ptr(idx), _ptr(w),
                                                    _stream(stream)))


def coli_dispatch(idx, E, S, counts, lists, n_active, active, err, stream=None):
    T, k = idx.shape
    _check("coli_dispatch", lib().coli_dispatch(_ptr(idx), T, k, E, S, _ptr(counts), _ptr(lists),
                                                _ptr(n_active), _ptr(active), _ptr(err),
                                                _stream(stream)))


# --------------------------------------------------------------------------- forward
def coli_moe_workspace_bytes(table: ExpertTable, T: int, k: int) -> int:
    return int(lib().coli_moe_workspace_bytes(table.ref(), T, k))


def coli_moe_forward(table: ExpertTable, xq, xd, idx, w, y, workspace, accumulate=False,
                     stream=None):
    T, k = idx.shape
    _check("coli_moe_forward",
           lib().coli_moe_forward(table.ref(), _ptr(xq), _ptr(xd), T, _ptr(idx), _ptr(w), k,
                                  _ptr(y), int(bool(accumulate)), _ptr(workspace),
                                  workspace.numel() * workspace.element_size(), _stream(stream)))


def coli_moe_forward_path(table: ExpertTable, xq, xd, idx, w, y, workspace, path: int,
                          accumulate=False, stream=None):
    T, k = idx.shape
    _check("coli_moe_forward_path",
           lib().coli_moe_forward_path(table.ref(), _ptr(xq), _ptr(xd), T, _ptr(idx), _ptr(w), k,
                                       _ptr(y), int(bool(accumulate)), _ptr(workspace),
                                       workspace.numel() * workspace.element_size(), path,
                                       _stream(stream)))


def coli_moe_path(table: ExpertTable, T: int, k: int) -> int:
    """The path COLI_PATH_AUTO takes for T tokens per pass (host only)."""
    r = int(lib().coli_moe_path(table.ref(), T, k))
    if r < 0:
        raise ColiError("coli_moe_path", r)
    return r


def coli_moe_forward_traced(table: ExpertTable, xq, xd, idx, w, y, workspace, trace: dict,
                            accumulate=False, stream=None):
    """trace: name -> tensor for any field of coli_moe_trace (missing = not written)."""
    tr = coli_moe_trace(*[_ptr(trace.get(n)) for n, _ in coli_moe_trace._fields_])
    T, k = idx.shape
    _check("coli_moe_forward_traced",
           lib().coli_moe_forward_traced(table.ref(), _ptr(xq), _ptr(xd), T, _ptr(idx), _ptr(w),
                                         k, _ptr(y), int(bool(accumulate)), _ptr(workspace),
                                         workspace.numel() * workspace.element_size(),
                                         ctypes.byref(tr), _stream(stream)))


def coli_moe_forward_profiled(table: ExpertTable, xq, xd, idx, w, y, workspace, events: dict,
                              accumulate=False, stream=None):
    """events: name -> hipEvent_t handle (int) for fields of coli_moe_events."""
    ev = coli_moe_events(*[events.get(n) for n, _ in coli_moe_events._fields_])
    T, k = idx.shape
    _check("coli_moe_forward_profiled",
           lib().coli_moe_forward_profiled(table.ref(), _ptr(xq), _ptr(xd), T, _ptr(idx), _ptr(w),
                                           k, _ptr(y), int(bool(accumulate)), _ptr(workspace),
                                           workspace.numel() * workspace.element_size(),
                                           ctypes.byref(ev), _stream(stream)))


def coli_moe_layer_workspace_bytes(table: ExpertTable, T: int, k: int) -> int:
    return int(lib().coli_moe_layer_workspace_bytes(table.ref(), T, k))


def coli_moe_layer(table: ExpertTable, x, logits, bias, k, y, workspace, routed_scale=1.0,
                   accumulate=False, trace: dict | None = None, events: dict | None = None,
                   stream=None):
    """x [T][D] f32, logits [T][E] f32, bias [E] f32 or None -> y [T][D] f32."""
    import torch
    _dtype(x, torch.float32, "x"); _dtype(logits, torch.float32, "logits")
    _dtype(bias, torch.float32, "bias"); _dtype(y, torch.float32, "y")
    T = x.shape[0]
    ws = workspace.numel() * workspace.element_size()
    if trace is None and events is None:
        _check("coli_moe_layer",
               lib().coli_moe_layer(table.ref(), _ptr(x), _ptr(logits), _ptr(bias), T, k,
                                    routed_scale, _ptr(y), int(bool(accumulate)),
                                    _ptr(workspace), ws, _stream(stream)))
        return
    tr = None if trace is None else coli_moe_trace(
        *[_ptr(trace.get(n)) for n, _ in coli_moe_trace._fields_])
    ev = None if events is None else coli_moe_events(
        *[events.get(n) for n, _ in coli_moe_events._fields_])
    _check("coli_moe_layer_ex",
           lib().coli_moe_layer_ex(table.ref(), _ptr(x), _ptr(logits), _ptr(bias), T, k,
                                   routed_scale, _ptr(y), int(bool(accumulate)), _ptr(workspace),
                                   ws, None if tr is None else ctypes.byref(tr),
                                   None if ev is None else ctypes.byref(ev), _stream(stream)))


def coli_moe_block(table: ExpertTable, h, logits, bias, k, workspace, eps=1e-6,
                   routed_scale=1.0, stream=None):
    """In place: h [T][D] f32 <- h + MoE(RMSNorm(h)); logits [T][E] f32, bias [E] f32 or None."""
    import torch
    _dtype(h, torch.float32, "h"); _dtype(logits, torch.float32, "logits")
    _dtype(bias, torch.float32, "bias")
    _check("coli_moe_block",
           lib().coli_moe_block(table.ref(), _ptr(h), _ptr(logits), _ptr(bias), h.shape[0], k,
                                routed_scale, eps, _ptr(workspace),
                                workspace.numel() * workspace.element_size(), _stream(stream)))


def coli_moe_layer_noalloc(table: ExpertTable, x, logits, bias, k, y, routed_scale=1.0,
                           accumulate=False, stream=None):
    """coli_moe_layer on the library's own device scratch (no workspace argument)."""
    import torch
    _dtype(x, torch.float32, "x"); _dtype(logits, torch.float32, "logits")
    _dtype(bias, torch.float32, "bias"); _dtype(y, torch.float32, "y")
    _check("coli_moe_layer_noalloc",
           lib().coli_moe_layer_noalloc(table.ref(), _ptr(x), _ptr(logits), _ptr(bias), x.shape[0],
                                        k, routed_scale, _ptr(y), int(bool(accumulate)),
                                        _stream(stream)))


def coli_moe_status(workspace, stream=None) -> int:
    """Synchronising: COLI_OK or COLI_E_INDEX for the last forward on `workspace`."""
    return int(lib().coli_moe_status(_ptr(workspace), workspace.numel() * workspace.element_size(),
                                     _stream(stream)))
