"""int2-container expert tables against the oracle (GPU).

Per-row int2 weights (s = max|w|, codes in [-1, 1]) packed four to a byte;
the GEMV reads two 32-column blocks per 16-byte chunk.  Checked: the int2
quantiser and the table layout bit for bit, every partial and intermediate of
traced passes at the tiny shape, the pages' invariant (one code set in the
2-bit, nibble and int8 tables gives identical layer outputs), and decode and
verify passes at the page shape.
"""
import numpy as np
import pytest

import oracle
import synth
from tests.gpu_util import (OracleExperts, assert_bitexact, assert_within_tol, build_table,
                            decode_table_expert2, table_from_experts)
from tests.test_gpu_moe import GpuLayer, check_front, check_trace, oracle_layer, to_dev

pytestmark = pytest.mark.gpu
torch = pytest.importorskip("torch")
if not torch.cuda.is_available():
    pytest.skip("no GPU", allow_module_level=True)
import int4_routed_expert_sigmoid_amd as coli  # noqa: E402

dev = "cuda"


def test_quant_weight_q2_bitexact():
    rng = np.random.default_rng(51)
    w = (rng.standard_normal((67, 512)) * 0.02).astype(np.float32)
    w[3] = 0.0
    w[4] = -0.75
    ties = np.array([0.5, -0.5, 0.75, -0.25, 1.0, -1.0, 0.0, 0.25], np.float32) * np.float32(0.25)
    w[5] = 0.0
    w[5, :ties.size] = ties
    q = torch.empty((67, 128), dtype=torch.uint8, device=dev)
    s = torch.empty(67, dtype=torch.float32, device=dev)
    coli.coli_quant_weight_q2(to_dev(w), q, s)
    rq, rs = oracle.q2_quant(w)
    assert_bitexact("int2 codes", q.cpu().numpy(), rq)
    assert_bitexact("int2 scales", s.cpu().numpy(), rs)


@pytest.fixture(scope="module")
def tiny2():
    w = synth.WORKLOADS[0]
    return w, build_table(w, bits=2), OracleExperts(w, bits=2)


def test_int2_table_layout(tiny2):
    w, table, ox = tiny2
    host = [t.cpu().numpy() for t in (table.gu_q, table.gu_s, table.dn_q, table.dn_s)]
    for e in (0, 11, w.E):
        gate, up, gs, us, down, ds = decode_table_expert2(w, *host, e)
        ref = ox[e]
        assert_bitexact(f"gate {e}", gate, oracle.unpack_q2(ref.gate_q).astype(np.int64))
        assert_bitexact(f"up {e}", up, oracle.unpack_q2(ref.up_q).astype(np.int64))
        assert_bitexact(f"down {e}", down, oracle.unpack_q2(ref.down_q).astype(np.int64))
        assert_bitexact(f"scales {e}", np.concatenate([gs, us, ds]),
                        np.concatenate([ref.gate_s, ref.up_s, ref.down_s]))


@pytest.mark.parametrize("T", [1, 2, 3, 4, 5, 9, 17])
def test_int2_tiny_traced(tiny2, T):
    w, table, ox = tiny2
    x, lg, b = synth.activations(w, T, 1400), synth.logits(w, T, 1400), synth.router_bias(w)
    g = GpuLayer(table, w, T).run(x, lg, b, trace=True)
    r = oracle_layer(ox, w, x, lg, b)
    check_front(g, r)
    check_trace(g, ox, w, r, tokens=range(min(T, 9)))
    assert_bitexact("y", g["y"], r["y"])
    assert_within_tol("y", g["y"], r["y"], r["absterm"])


def test_int2_int4_int8_tables_agree():
    """One code set in [-2, 1] in all three containers: identical layer outputs
    on the GPU, equal to the oracle."""
    w = synth.WORKLOADS[0]
    rng = np.random.default_rng(52)
    ex = {2: [], 4: [], 8: []}
    for e in range(w.E + w.S):
        mats = [rng.integers(-2, 2, size=shape).astype(np.int8)
                for shape in ((w.F, w.D), (w.F, w.D), (w.D, w.F))]
        sc = [rng.uniform(1e-3, 1e-2, m.shape[0]).astype(np.float32) for m in mats]
        ex[2].append(oracle.Expert(*[a for m, s_ in zip(mats, sc) for a in (oracle.pack_q2(m), s_)],
                                   bits=2))
        ex[4].append(oracle.Expert(*[a for m, s_ in zip(mats, sc) for a in (oracle.pack_q4(m), s_)],
                                   bits=4))
        ex[8].append(oracle.Expert(*[a for m, s_ in zip(mats, sc) for a in (m, s_)], bits=8))
    tables = {b: table_from_experts(w, ex[b], b) for b in (2, 4, 8)}
    for T in (1, 4, 11):
        x, lg, b = synth.activations(w, T, 1500), synth.logits(w, T, 1500), synth.router_bias(w)
        ys = {bits: GpuLayer(t, w, T).run(x, lg, b)["y"] for bits, t in tables.items()}
        assert_bitexact(f"int2 vs int8, T={T}", ys[2], ys[8])
        assert_bitexact(f"int4 vs int8, T={T}", ys[4], ys[8])
        xq, xd = oracle.q8_quant(x)
        idx, wt = oracle.route(lg, b, w.k)
        yr, _ = oracle.moe_layer({e: ex[2][e] for e in range(w.E + w.S)}, w.E, w.S, xq, xd, idx, wt)
        assert_bitexact(f"int2 vs oracle, T={T}", ys[2], yr)


@pytest.fixture(scope="module")
def big2():
    w = synth.WORKLOADS[2]
    return build_table(w, layer=2, bits=2), OracleExperts(w, layer=2, bits=2)


@pytest.mark.parametrize("wid", [1, 2])
def test_int2_page_shape(big2, wid):
    """Decode (1 token) and verify (4 tokens) of a page-shape int2 layer."""
    table, ox = big2
    w = synth.WORKLOADS[wid]
    x, lg, b = synth.activations(w, w.T, 1600), synth.logits(w, w.T, 1600), synth.router_bias(w)
    g = GpuLayer(table, w, w.T).run(x, lg, b)
    r = oracle_layer(ox, w, x, lg, b)
    check_front(g, r)
    assert_bitexact("y", g["y"], r["y"])
    assert_within_tol("y", g["y"], r["y"], r["absterm"])
