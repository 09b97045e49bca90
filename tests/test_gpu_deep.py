"""Deep decode stack: 40 MoE layers in the pre-norm residual form
h <- h + MoE(RMSNorm(h)) (RMSNorm eps 1e-6, unit gain), with Zipf(1.1)-skewed
router logits per layer, against the oracle (GPU).

In an MoE-only stack the tokens do not interact, so each token's 40-layer
trajectory is checked on its own.  The complete stack is compared bit for bit
at the tiny shape, both one token per pass (the GEMV path) and all tokens in
one pass per layer (the grouped path).  At the page shape (40 tables, 194 GB)
the stack runs on the GPU and sampled layers are recomputed by the oracle from
the GPU's own input to that layer.
"""
from dataclasses import replace

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
EPS = 1e-6
DEEP = synth.WORKLOADS[4]
DEEP_TINY = replace(DEEP, name="tiny deep stack d256 f128 e16+1 top2 zipf1.1", D=256, F=128,
                    E=16, k=2, family=0, tag=5)


def to_dev(a):
    return torch.from_numpy(np.ascontiguousarray(a)).to(dev)


class GpuStack:
    """rmsnorm_q8 -> route_topk -> moe_forward (accumulating into h) per layer."""

    def __init__(self, w, tables, T):
        self.w, self.tables, self.T = w, tables, T
        self.ws = torch.empty(coli.coli_moe_workspace_bytes(tables[0], T, w.k), dtype=torch.uint8,
                              device=dev)
        self.xq = torch.empty((T, w.D), dtype=torch.int8, device=dev)
        self.xd = torch.empty((T, w.D // 32), dtype=torch.float32, device=dev)
        self.idx = torch.empty((T, w.k), dtype=torch.int32, device=dev)
        self.wt = torch.empty((T, w.k), dtype=torch.float32, device=dev)
        self.bias = [to_dev(synth.router_bias(w, layer)) for layer in range(len(tables))]

    def layer(self, h, layer, token0):
        w = self.w
        coli.coli_rmsnorm_q8(h, EPS, self.xq, self.xd)
        lg = to_dev(synth.logits(w, self.T, token0, layer))
        coli.coli_route_topk(lg, self.bias[layer], w.k, self.idx, self.wt)
        coli.coli_moe_forward(self.tables[layer], self.xq, self.xd, self.idx, self.wt, h, self.ws,
                              accumulate=True)

    def run(self, h0, token0, layers=None, keep=()):
        """h after every layer in `keep` (and the final h)."""
        h = to_dev(h0)
        kept = {}
        for layer in range(layers or len(self.tables)):
            self.layer(h, layer, token0)
            if layer in keep:
                kept[layer] = h.cpu().numpy()
        assert coli.coli_moe_status(self.ws) == coli.COLI_OK
        return h.cpu().numpy(), kept


class BlockStack(GpuStack):
    """The same stack through coli_moe_block (RMSNorm + Q8, routing and
    dispatch in one front kernel for small batches; h updated in place)."""

    def __init__(self, w, tables, T):
        super().__init__(w, tables, T)
        self.ws = torch.empty(coli.coli_moe_layer_workspace_bytes(tables[0], T, w.k),
                              dtype=torch.uint8, device=dev)

    def layer(self, h, layer, token0):
        lg = to_dev(synth.logits(self.w, self.T, token0, layer))
        coli.coli_moe_block(self.tables[layer], h, lg, self.bias[layer], self.w.k, self.ws,
                            eps=EPS)


def oracle_layer(w, ox, h, layer, token0):
    T = h.shape[0]
    xh, _ = oracle.rmsnorm(h, EPS)
    xq, xd = oracle.q8_quant(xh)
    idx, wt = oracle.route(synth.logits(w, T, token0, layer), synth.router_bias(w, layer), w.k)
    y, _ = oracle.moe_layer(ox.table_for(idx), w.E, w.S, xq, xd, idx, wt, out=h, accumulate=True)
    return y, idx


@pytest.fixture(scope="module")
def tiny_stack():
    w = DEEP_TINY
    tables = [build_table(w, layer) for layer in range(w.layers)]
    oxs = [OracleExperts(w, layer) for layer in range(w.layers)]
    return w, tables, oxs


def oracle_stack(w, oxs, h0, token0):
    h = h0.copy()
    hot = np.zeros((w.layers, w.E), dtype=np.int64)   # selections per layer and expert
    for layer in range(w.layers):
        h, idx = oracle_layer(w, oxs[layer], h, layer, token0)
        np.add.at(hot[layer], idx.reshape(-1), 1)
    return h, hot


def test_tiny_stack_token_by_token(tiny_stack):
    """16 tokens, one pass per token per layer (GEMV path), 40 layers, bit-exact."""
    w, tables, oxs = tiny_stack
    n = 16
    h0 = synth.hidden0(w, n)
    ref, hot = oracle_stack(w, oxs, h0, 0)
    stack = GpuStack(w, tables, 1)
    for t in range(n):
        got, _ = stack.run(h0[t:t + 1], t)
        assert_bitexact(f"h after 40 layers, token {t}", got, ref[t:t + 1])
    # the Zipf routing concentrates each layer's picks on its few top-ranked
    # experts (every layer has its own ranking): sanity of the workload
    assert (hot.max(axis=1) / hot.mean(axis=1)).mean() > 2.5


def test_tiny_stack_batched(tiny_stack):
    """256 tokens in one pass per layer (grouped matrix-core path), 40 layers, bit-exact."""
    w, tables, oxs = tiny_stack
    T = w.steps
    h0 = synth.hidden0(w, T)
    ref, _ = oracle_stack(w, oxs, h0, 0)
    got, _ = GpuStack(w, tables, T).run(h0, 0)
    assert_bitexact("h after 40 layers, 256 tokens", got, ref)


def test_tiny_block_stack_token_by_token(tiny_stack):
    """coli_moe_block, one token per pass (fused front, GEMV path), 40 layers, bit-exact."""
    w, tables, oxs = tiny_stack
    n = 8
    h0 = synth.hidden0(w, n, 300)
    ref, _ = oracle_stack(w, oxs, h0, 300)
    stack = BlockStack(w, tables, 1)
    for t in range(n):
        got, _ = stack.run(h0[t:t + 1], 300 + t)
        assert_bitexact(f"block h after 40 layers, token {t}", got, ref[t:t + 1])


@pytest.mark.parametrize("T", [4, 64, 256])
def test_tiny_block_stack_batched(tiny_stack, T):
    """coli_moe_block with T tokens per pass: the fused front (one RMSNorm
    workgroup per token) with the GEMV path (4) and the grouped path (64),
    and the separate RMSNorm / routing kernels with the grouped path (256);
    40 layers, bit-exact."""
    w, tables, oxs = tiny_stack
    h0 = synth.hidden0(w, T, 400)
    ref, _ = oracle_stack(w, oxs, h0, 400)
    got, _ = BlockStack(w, tables, T).run(h0, 400)
    assert_bitexact(f"block h after 40 layers, {T} tokens", got, ref)


def test_page_shape_stack_full():
    """8 tokens through all 40 page-shape layers (194 GB of tables), one token
    per pass through coli_moe_block, as the benchmark runs the deep stack
    (also captured in a HIP graph and replayed), against the oracle's own
    40-layer stack from the same h0, every layer's output bit for bit."""
    from concurrent.futures import ThreadPoolExecutor
    w = DEEP
    n = 8
    tables = [build_table(w, layer) for layer in range(w.layers)]
    h0 = synth.hidden0(w, n)
    every = set(range(w.layers))
    got = []
    for t in range(n):
        final, kept = BlockStack(w, tables, 1).run(h0[t:t + 1], t, keep=every)
        got.append(kept)
    # the same stack captured in one graph (all tokens, all layers) and replayed
    lg = [to_dev(synth.logits(w, n, 0, layer)) for layer in range(w.layers)]
    bias = [to_dev(synth.router_bias(w, layer)) for layer in range(w.layers)]
    hg = to_dev(h0)
    ws = torch.empty(coli.coli_moe_layer_workspace_bytes(tables[0], 1, w.k), dtype=torch.uint8,
                     device=dev)
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        for t in range(n):
            for layer in range(w.layers):
                coli.coli_moe_block(tables[layer], hg[t:t + 1], lg[layer][t:t + 1], bias[layer],
                                    w.k, ws, eps=EPS)
    graph.replay()
    torch.cuda.synchronize()
    assert coli.coli_moe_status(ws) == coli.COLI_OK
    hgraph = hg.cpu().numpy()
    del graph, tables
    torch.cuda.empty_cache()
    # the oracle: routing does not depend on h (synthetic logits), so each
    # layer's experts are known up front and generated in a pool, one layer
    # ahead of the layer being computed
    idxs = [oracle.route(synth.logits(w, n, 0, layer), synth.router_bias(w, layer), w.k)[0]
            for layer in range(w.layers)]

    def experts_of(layer):
        ox = OracleExperts(w, layer)
        need = sorted(set(int(e) for e in idxs[layer].reshape(-1)) | {w.E})
        with ThreadPoolExecutor(4) as pool:
            list(pool.map(lambda e: ox[e], need))
        return ox

    h = h0.copy()
    with ThreadPoolExecutor(1) as ahead:
        nxt = ahead.submit(experts_of, 0)
        for layer in range(w.layers):
            ox = nxt.result()
            if layer + 1 < w.layers:
                nxt = ahead.submit(experts_of, layer + 1)
            h, idx = oracle_layer(w, ox, h, layer, 0)
            assert np.array_equal(idx, idxs[layer])
            for t in range(n):
                assert_bitexact(f"token {t} after layer {layer}", got[t][layer], h[t:t + 1])
            if layer % 10 == 9:
                print(f"deep stack: {layer + 1} of {w.layers} layers bit-exact", flush=True)
    assert_bitexact("graph replay, h after 40 layers", hgraph, h)
