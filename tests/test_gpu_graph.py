"""Parity in the launch configuration the benchmark times: whole layers
(coli_moe_layer: fused front, gate/up, down, combine) captured in a HIP graph
and replayed.

Each graph holds a pool of independent steps sharing one workspace, as the
benchmark's graphs do.  It is replayed several times with eager library work
and synchronisations in between, the outputs cleared by a fill kernel before
each replay, and every replay is compared bit for bit with the oracle on the
same seeded inputs (all tokens for decode and verify; sampled tokens for the
2048-token prefill pass).
"""
import numpy as np
import pytest

import oracle
import synth
from tests.gpu_util import OracleExperts, assert_bitexact, build_table

pytestmark = pytest.mark.gpu
torch = pytest.importorskip("torch")
if not torch.cuda.is_available():
    pytest.skip("no GPU", allow_module_level=True)
import int4_routed_expert_sigmoid_amd as coli  # noqa: E402

dev = "cuda"
REPLAYS = 3


def to_dev(a):
    return torch.from_numpy(np.ascontiguousarray(a)).to(dev)


def oracle_y(ox, w, x, lg, b, rows=None):
    xq, xd = oracle.q8_quant(x)
    idx, wt = oracle.route(lg, b, w.k)
    if rows is not None:
        xq, xd, idx, wt = xq[rows], xd[rows], idx[rows], wt[rows]
    y, _ = oracle.moe_layer(ox.table_for(idx), w.E, w.S, xq, xd, idx, wt)
    return y


def graph_replays(table, w, T, pool, token0, check):
    """Captures `pool` layer calls of T tokens in one graph and replays it;
    check(j, y_j) runs on every step's output after every replay."""
    xs = [to_dev(synth.activations(w, T, token0 + j * T)) for j in range(pool)]
    lgs = [to_dev(synth.logits(w, T, token0 + j * T)) for j in range(pool)]
    bias = to_dev(synth.router_bias(w))
    ys = torch.zeros((pool, T, w.D), dtype=torch.float32, device=dev)
    ws = torch.empty(coli.coli_moe_layer_workspace_bytes(table, T, w.k), dtype=torch.uint8,
                     device=dev)
    # eager side work between replays: another token through its own workspace
    xe, lge = to_dev(synth.activations(w, 1, 9000)), to_dev(synth.logits(w, 1, 9000))
    ye = torch.empty((1, w.D), dtype=torch.float32, device=dev)
    wse = torch.empty(coli.coli_moe_layer_workspace_bytes(table, 1, w.k), dtype=torch.uint8,
                      device=dev)

    def steps():
        for j in range(pool):
            coli.coli_moe_layer(table, xs[j], lgs[j], bias, w.k, ys[j], ws)

    steps()                                  # eager pass first, as the benchmark does
    torch.cuda.synchronize()
    assert coli.coli_moe_status(ws) == coli.COLI_OK
    eager = ys.cpu().numpy()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        steps()
    for r in range(REPLAYS):
        ys.zero_()
        coli.coli_moe_layer(table, xe, lge, bias, w.k, ye, wse)
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        assert coli.coli_moe_status(ws) == coli.COLI_OK
        got = ys.cpu().numpy()
        assert_bitexact(f"replay {r} vs eager", got, eager)
        for j in range(pool):
            check(j, got[j], f"replay {r} step {j}")


@pytest.fixture(scope="module")
def big():
    w = synth.WORKLOADS[1]
    return build_table(w), OracleExperts(w)


def test_graph_decode_page_shape(big):
    """The benchmark's decode step (1 token, 4.86 GB table) under graph replay."""
    table, ox = big
    w = synth.WORKLOADS[1]
    pool, token0 = 4, 500
    ref = [oracle_y(ox, w, synth.activations(w, 1, token0 + j), synth.logits(w, 1, token0 + j),
                    synth.router_bias(w)) for j in range(pool)]
    graph_replays(table, w, 1, pool, token0,
                  lambda j, y, tag: assert_bitexact(f"y {tag}", y, ref[j]))


def test_graph_verify_page_shape(big):
    """4-token verify passes (batch union of their experts) under graph replay."""
    table, ox = big
    w = synth.WORKLOADS[2]
    pool, token0 = 2, 600
    ref = [oracle_y(ox, w, synth.activations(w, 4, token0 + 4 * j),
                    synth.logits(w, 4, token0 + 4 * j), synth.router_bias(w))
           for j in range(pool)]
    graph_replays(table, w, 4, pool, token0,
                  lambda j, y, tag: assert_bitexact(f"y {tag}", y, ref[j]))


def test_graph_prefill_page_shape_sampled(big):
    """A 2048-token pass (grouped matrix-core path) under graph replay; sampled
    tokens against the oracle, every token against the eager result."""
    table, ox = big
    w = synth.WORKLOADS[3]
    T, token0 = w.T, 700
    rows = [0, 1, T // 2, T - 2, T - 1]
    ref = oracle_y(ox, w, synth.activations(w, T, token0), synth.logits(w, T, token0),
                   synth.router_bias(w), rows=rows)
    graph_replays(table, w, T, 1, token0,
                  lambda j, y, tag: assert_bitexact(f"y {tag}", y[rows], ref))


@pytest.mark.parametrize("T,pool", [(1, 16), (4, 4), (64, 2)])
def test_graph_tiny(T, pool):
    """Tiny layer: decode, verify and grouped passes under graph replay."""
    w = synth.WORKLOADS[0]
    table, ox = build_table(w), OracleExperts(w)
    token0 = 40
    ref = [oracle_y(ox, w, synth.activations(w, T, token0 + j * T),
                    synth.logits(w, T, token0 + j * T), synth.router_bias(w))
           for j in range(pool)]
    graph_replays(table, w, T, pool, token0,
                  lambda j, y, tag: assert_bitexact(f"y {tag}", y, ref[j]))
