"""int8-container expert tables (the int8 speculative head) against the
oracle (GPU).

The head's experts are quantised per row to int8 (s = max|w| / 127) and run
through the same Q8_0 block dot; the GEMV kernels read two 1 KB chunks per
32-column block.  Checked here: the int8 quantiser and the table layout bit
for bit, every partial and intermediate of traced passes at the tiny shape,
the pages' invariant that the int8 container holding int4 codes gives the
int4 table's results exactly, and the decode (1 token) and verify (4 tokens)
shapes of a 6144 x 2048, 256 + 1 expert head.
"""
import numpy as np
import pytest

import oracle
import synth
from tests.gpu_util import (OracleExperts, assert_bitexact, assert_within_tol, build_table,
                            decode_table_expert8, table_from_experts)
from tests.test_gpu_moe import GpuLayer, check_front, check_trace, oracle_layer, to_dev

pytestmark = pytest.mark.gpu
torch = pytest.importorskip("torch")
if not torch.cuda.is_available():
    pytest.skip("no GPU", allow_module_level=True)
import int4_routed_expert_sigmoid_amd as coli  # noqa: E402

dev = "cuda"
HEAD_LAYER = 78   # the speculative head sits after the 78 main layers


def test_quant_weight_q8_bitexact():
    """Random rows, an all-zero row, a constant row and exact half-integer
    quotients (ties) against the oracle's per-row int8 rule."""
    rng = np.random.default_rng(31)
    w = (rng.standard_normal((67, 512)) * 0.02).astype(np.float32)
    w[3] = 0.0
    w[4] = -0.75
    ties = np.array([0.5, 1.5, 2.5, 3.5, -0.5, -1.5, -2.5, 125.5, 126.5, -126.5, 127.0, -3.0],
                    np.float32) * np.float32(2.0 ** -3)
    w[5] = 0.0
    w[5, :ties.size] = ties
    q = torch.empty(w.shape, dtype=torch.int8, device=dev)
    s = torch.empty(w.shape[0], dtype=torch.float32, device=dev)
    coli.coli_quant_weight_q8(to_dev(w), q, s)
    rq, rs = oracle.q8w_quant(w)
    assert_bitexact("int8 codes", q.cpu().numpy(), rq)
    assert_bitexact("int8 scales", s.cpu().numpy(), rs)
    assert rs[3] == 0.0 and not rq[3].any()


@pytest.fixture(scope="module")
def tiny8():
    w = synth.WORKLOADS[0]
    return w, build_table(w, bits=8), OracleExperts(w, bits=8)


def test_int8_table_layout(tiny8):
    w, table, ox = tiny8
    host = [t.cpu().numpy() for t in (table.gu_q, table.gu_s, table.dn_q, table.dn_s)]
    for e in (0, 7, w.E):
        gate, up, gs, us, down, ds = decode_table_expert8(w, *host, e)
        ref = ox[e]
        assert_bitexact(f"gate {e}", gate, ref.gate_q.astype(np.int64))
        assert_bitexact(f"up {e}", up, ref.up_q.astype(np.int64))
        assert_bitexact(f"down {e}", down, ref.down_q.astype(np.int64))
        assert_bitexact(f"scales {e}", np.concatenate([gs, us, ds]),
                        np.concatenate([ref.gate_s, ref.up_s, ref.down_s]))


@pytest.mark.parametrize("T", [1, 2, 3, 4, 5, 9, 17, 130])
def test_int8_tiny_traced(tiny8, T):
    """Every pass size of the GEMV kernels, ragged passes, and (130) a batch
    that takes the GEMV path for int8 where int4 would go grouped."""
    w, table, ox = tiny8
    x, lg, b = synth.activations(w, T, 900), synth.logits(w, T, 900), synth.router_bias(w)
    g = GpuLayer(table, w, T).run(x, lg, b, trace=True)
    r = oracle_layer(ox, w, x, lg, b)
    check_front(g, r)
    check_trace(g, ox, w, r, tokens=range(min(T, 9)))
    assert_bitexact("y", g["y"], r["y"])
    assert_within_tol("y", g["y"], r["y"], r["absterm"])


def test_int8_accumulate(tiny8):
    w, table, ox = tiny8
    T = 4
    x, lg, b = synth.activations(w, T, 950), synth.logits(w, T, 950), synth.router_bias(w)
    y0 = synth.hidden0(w, T)
    g = GpuLayer(table, w, T).run(x, lg, b, y0=y0, accumulate=True)
    r = oracle_layer(ox, w, x, lg, b, y0=y0, accumulate=True)
    assert_bitexact("y += moe", g["y"], r["y"])


def test_int8_container_of_int4_codes_matches_int4_table():
    """The pages' bit-identity invariant on the GPU: an int8 table holding the
    int4 codes gives the int4 table's layer output bit for bit (and both match
    the oracle)."""
    w = synth.WORKLOADS[0]
    ox4 = OracleExperts(w, layer=3)
    ex4 = [ox4[e] for e in range(w.E + w.S)]
    ex8 = [oracle.Expert(oracle.unpack_q4(e.gate_q), e.gate_s, oracle.unpack_q4(e.up_q), e.up_s,
                         oracle.unpack_q4(e.down_q), e.down_s, bits=8) for e in ex4]
    t4 = table_from_experts(w, ex4, 4)
    t8 = table_from_experts(w, ex8, 8)
    for T in (1, 4, 11):
        x, lg, b = synth.activations(w, T, 990), synth.logits(w, T, 990), synth.router_bias(w)
        g4 = GpuLayer(t4, w, T).run(x, lg, b)
        g8 = GpuLayer(t8, w, T).run(x, lg, b)
        assert_bitexact(f"int8 container vs int4, T={T}", g8["y"], g4["y"])
        r = oracle_layer(ox4, w, x, lg, b)
        assert_bitexact(f"int4 table vs oracle, T={T}", g4["y"], r["y"])


@pytest.fixture(scope="module")
def head8():
    """The 6144 x 2048, 256 + 1 expert head in int8 (9.7 GB)."""
    w = synth.WORKLOADS[2]
    return build_table(w, layer=HEAD_LAYER, bits=8), OracleExperts(w, layer=HEAD_LAYER, bits=8)


@pytest.mark.parametrize("wid", [1, 2])
def test_int8_head_page_shape(head8, wid):
    """Decode (1 token) and the batched verify pass (4 tokens) of the int8
    head at the page shape: every token against the oracle, bit for bit."""
    table, ox = head8
    w = synth.WORKLOADS[wid]
    T = w.T
    x, lg, b = synth.activations(w, T, 1000), synth.logits(w, T, 1000), synth.router_bias(w)
    g = GpuLayer(table, w, T).run(x, lg, b)
    r = oracle_layer(ox, w, x, lg, b)
    check_front(g, r)
    assert_bitexact("y", g["y"], r["y"])
    assert_within_tol("y", g["y"], r["y"], r["absterm"])


def test_int8_head_traced_sample(head8):
    """Partials of one verify pass at the page shape, for tokens 0 and 3."""
    table, ox = head8
    w = synth.WORKLOADS[2]
    T = w.T
    x, lg, b = synth.activations(w, T, 1100), synth.logits(w, T, 1100), synth.router_bias(w)
    g = GpuLayer(table, w, T).run(x, lg, b, trace=True)
    r = oracle_layer(ox, w, x, lg, b)
    check_trace(g, ox, w, r, tokens=(0, 3))
    assert_bitexact("y", g["y"], r["y"])
