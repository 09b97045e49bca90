"""Helpers shared by the GPU parity tests: build the device table from the
seeded generator with the library's own quantiser, and the oracle's experts
from the same seeded generator with the oracle's quantiser."""
from __future__ import annotations

import numpy as np

import oracle
import synth

TOL_REL = 1e-5   # |gpu - oracle| <= 1e-5 * sum|terms| + 1e-6
TOL_ABS = 1e-6


def stream_ptr():
    import torch
    return torch.cuda.current_stream().cuda_stream


def build_table(w: synth.Workload, layer: int = 0, bits: int = 4):
    """Device table: device-generated fp32 weights, coli_quant_weight_q4 (or
    coli_quant_weight_q8 for an int8 table), coli_table_set_expert."""
    import torch
    import int4_routed_expert_sigmoid_amd as coli
    table = coli.ExpertTable(w.E, w.S, w.D, w.F, weight_bits=bits)
    F, D = w.F, w.D
    scratch = torch.empty(F * D, dtype=torch.float32, device="cuda")
    quant, qdt, per = {4: (coli.coli_quant_weight_q4, torch.uint8, 2),
                       8: (coli.coli_quant_weight_q8, torch.int8, 1),
                       2: (coli.coli_quant_weight_q2, torch.uint8, 4)}[bits]
    gq = torch.empty((F, D // per), dtype=qdt, device="cuda")
    uq = torch.empty_like(gq)
    dq = torch.empty((D, F // per), dtype=qdt, device="cuda")
    gs = torch.empty(F, dtype=torch.float32, device="cuda")
    us = torch.empty_like(gs)
    ds = torch.empty(D, dtype=torch.float32, device="cuda")
    sp = stream_ptr()
    for e in range(w.E + w.S):
        for m, (q, s) in enumerate(((gq, gs), (uq, us), (dq, ds))):
            rows, cols = synth.weight_shape(w, m)
            synth.weight_device(w, layer, e, m, scratch.data_ptr(), sp)
            quant(scratch[: rows * cols].view(rows, cols), q, s)
        coli.coli_table_set_expert(table, e, gq, gs, uq, us, dq, ds)
    torch.cuda.synchronize()
    return table


def table_from_experts(w: synth.Workload, experts, bits: int):
    """Device table filled from host containers (oracle.Expert, any source)."""
    import torch
    import int4_routed_expert_sigmoid_amd as coli
    table = coli.ExpertTable(w.E, w.S, w.D, w.F, weight_bits=bits)
    dev = lambda a: torch.from_numpy(np.ascontiguousarray(a)).to("cuda")
    for e in range(w.E + w.S):
        ex = experts[e]
        assert ex.bits == bits
        coli.coli_table_set_expert(table, e, dev(ex.gate_q), dev(ex.gate_s), dev(ex.up_q),
                                   dev(ex.up_s), dev(ex.down_q), dev(ex.down_s))
    torch.cuda.synchronize()
    return table


class OracleExperts:
    """The oracle's containers (int4, or int8 with bits=8), generated on the
    host on first use."""

    def __init__(self, w: synth.Workload, layer: int = 0, bits: int = 4):
        self.w, self.layer, self.bits, self.cache = w, layer, bits, {}

    def __getitem__(self, e: int) -> oracle.Expert:
        if e not in self.cache:
            mats = [synth.weight_host(self.w, self.layer, e, m) for m in range(3)]
            self.cache[e] = oracle.Expert.quantize(*mats, bits=self.bits)
        return self.cache[e]

    def table_for(self, idx) -> dict:
        need = set(int(v) for v in np.asarray(idx).reshape(-1) if 0 <= v < self.w.E)
        if self.w.S:
            need.add(self.w.E)
        return {e: self[e] for e in sorted(need)}


def decode_table_expert(w: synth.Workload, gu_q, gu_s, dn_q, dn_s, e: int):
    """Test-side decoder of the documented table layout back to int codes.

    gu_q/dn_q: uint8 numpy arrays of the whole table.  Returns
    (gate_codes [F][D], up_codes [F][D], gate_s, up_s, down_codes [D][F], down_s).
    """
    D, F = w.D, w.F
    nbd, nbf = D // 32, F // 32

    def chunk_codes(chunks):          # [..., 16] bytes -> [..., 32] codes, column order
        words = chunks.reshape(chunks.shape[:-1] + (4, 4))   # word kk, byte j
        lo = (words & 0x0F).astype(np.int64) - 8             # column 8kk + j
        hi = (words >> 4).astype(np.int64) - 8               # column 8kk + 4 + j
        out = np.empty(chunks.shape[:-1] + (4, 8), dtype=np.int64)
        out[..., 0:4] = lo
        out[..., 4:8] = hi
        return out.reshape(chunks.shape[:-1] + (32,))

    gu = gu_q[e * F * D:(e + 1) * F * D].reshape(F // 32, nbd, 64, 16)
    codes = chunk_codes(gu)                                   # [g][b][lane][32]
    codes = codes.transpose(0, 2, 1, 3).reshape(F // 32, 64, D)   # [g][lane][col]
    gate = codes[:, :32, :].reshape(F, D)
    up = codes[:, 32:, :].reshape(F, D)
    s = gu_s[e * 2 * F:(e + 1) * 2 * F].reshape(F // 32, 64)
    gate_s, up_s = s[:, :32].reshape(F), s[:, 32:].reshape(F)
    dn = dn_q[e * D * F // 2:(e + 1) * D * F // 2].reshape(D // 64, nbf, 64, 16)
    dcodes = chunk_codes(dn).transpose(0, 2, 1, 3).reshape(D, F)
    down_s = dn_s[e * D:(e + 1) * D]
    return gate, up, gate_s, up_s, dcodes, down_s


def decode_table_expert8(w: synth.Workload, gu_q, gu_s, dn_q, dn_s, e: int):
    """Test-side decoder of the documented int8 table layout (chunk c of a
    lane = columns 16c..16c+15 of its row, bytes in column order)."""
    D, F = w.D, w.F
    gu = gu_q[e * 2 * F * D:(e + 1) * 2 * F * D].view(np.int8).reshape(F // 32, D // 16, 64, 16)
    codes = gu.transpose(0, 2, 1, 3).reshape(F // 32, 64, D).astype(np.int64)
    gate = codes[:, :32, :].reshape(F, D)
    up = codes[:, 32:, :].reshape(F, D)
    s = gu_s[e * 2 * F:(e + 1) * 2 * F].reshape(F // 32, 64)
    dn = dn_q[e * D * F:(e + 1) * D * F].view(np.int8).reshape(D // 64, F // 16, 64, 16)
    dcodes = dn.transpose(0, 2, 1, 3).reshape(D, F).astype(np.int64)
    return gate, up, s[:, :32].reshape(F), s[:, 32:].reshape(F), dcodes, dn_s[e * D:(e + 1) * D]


def decode_table_expert2(w: synth.Workload, gu_q, gu_s, dn_q, dn_s, e: int):
    """Test-side decoder of the documented int2 table layout (chunk of 64
    columns; word m, byte j, field i = column 16m + 4i + j, stored q + 2)."""
    D, F = w.D, w.F

    def chunk_codes(chunks):          # [..., 16] bytes -> [..., 64] codes
        b = chunks.reshape(chunks.shape[:-1] + (4, 4)).astype(np.int64)   # word m, byte j
        out = np.empty(chunks.shape[:-1] + (64,), dtype=np.int64)
        for m in range(4):
            for j in range(4):
                for i in range(4):
                    out[..., 16 * m + 4 * i + j] = ((b[..., m, j] >> (2 * i)) & 3) - 2
        return out

    per_gu = 2 * F * D // 4
    gu = gu_q[e * per_gu:(e + 1) * per_gu].reshape(F // 32, D // 64, 64, 16)
    codes = chunk_codes(gu).transpose(0, 2, 1, 3).reshape(F // 32, 64, D)
    per_dn = D * F // 4
    dn = dn_q[e * per_dn:(e + 1) * per_dn].reshape(D // 64, F // 64, 64, 16)
    dcodes = chunk_codes(dn).transpose(0, 2, 1, 3).reshape(D, F)
    s = gu_s[e * 2 * F:(e + 1) * 2 * F].reshape(F // 32, 64)
    return (codes[:, :32, :].reshape(F, D), codes[:, 32:, :].reshape(F, D), s[:, :32].reshape(F),
            s[:, 32:].reshape(F), dcodes, dn_s[e * D:(e + 1) * D])


def assert_bitexact(name, got, ref):
    got = np.asarray(got)
    ref = np.asarray(ref)
    assert got.shape == ref.shape, f"{name}: shape {got.shape} vs {ref.shape}"
    if got.dtype.kind == "f":
        g, r = got.view(np.uint32 if got.itemsize == 4 else np.uint64), ref.view(
            np.uint32 if ref.itemsize == 4 else np.uint64)
    else:
        g, r = got, ref
    bad = np.nonzero(g.reshape(-1) != r.reshape(-1))[0]
    assert bad.size == 0, (f"{name}: {bad.size}/{g.size} differ; first at {bad[:5]}: "
                           f"gpu {got.reshape(-1)[bad[:5]]} oracle {ref.reshape(-1)[bad[:5]]}")


def assert_within_tol(name, got, ref, absterm):
    err = np.abs(np.asarray(got, np.float64) - np.asarray(ref, np.float64))
    bound = TOL_REL * np.asarray(absterm) + TOL_ABS
    bad = np.nonzero(err.reshape(-1) > bound.reshape(-1))[0]
    assert bad.size == 0, f"{name}: {bad.size} outside 1e-5*sum|terms|+1e-6; first {bad[:5]}"
