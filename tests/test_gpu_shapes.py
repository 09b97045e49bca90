"""Layer parity on degenerate and ragged shapes (GPU), bit-exact against the oracle.

Shapes beyond the workloads: every expert selected (k = E) with no shared
expert, top-1, contraction lengths that leave partial weight-ring passes and
token-record tails (d_model 320 = 10 blocks, d_ff 96 = 3 blocks, d_ff 160),
and no shared expert at the tiny shape; and the library's limits
(COLI_MAX_DIM, COLI_MAX_EXPERTS, COLI_MAX_TOPK in coli.h): d_model 32768,
d_ff 32768 (the GEMV's token records then leave room for one token per pass,
so every batch runs one-token passes), and 256 routed experts with top-64 (16
tokens then fill the fused front's 1024 routing entries exactly).  Each runs
1, 2, 5, 16 and 33 tokens through both expert paths (GEMV, grouped matrix
cores), through the fused layer entry point, and through the pre-norm block
entry point.
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
EPS = 1e-6

SHAPES = {
    "k=E, no shared, ragged": synth.Workload("shape d320 f96 e8+0 top8", 320, 96, 8, 0, 8, 1,
                                              family=2, tag=10),
    "top-1": synth.Workload("shape d128 f64 e4+1 top1", 128, 64, 4, 1, 1, 1, family=3, tag=11),
    "d_ff 160, 32 experts": synth.Workload("shape d192 f160 e32+1 top4", 192, 160, 32, 1, 4, 1,
                                           family=4, tag=12),
    "no shared": synth.Workload("shape d256 f128 e16+0 top2", 256, 128, 16, 0, 2, 1, family=5,
                                tag=13),
    "d_model at the limit": synth.Workload("limit d32768 f64 e4+1 top2", 32768, 64, 4, 1, 2, 1,
                                           family=6, tag=14),
    "d_ff at the limit": synth.Workload("limit d64 f32768 e4+1 top2", 64, 32768, 4, 1, 2, 1,
                                        family=7, tag=15),
    "experts and top-k at the limit": synth.Workload("limit d128 f64 e256+1 top64", 128, 64, 256,
                                                     1, 64, 1, family=8, tag=16),
}
TOKENS = [1, 2, 5, 16, 33]


def to_dev(a):
    return torch.from_numpy(np.ascontiguousarray(a)).to(dev)


@pytest.fixture(scope="module", params=list(SHAPES))
def shape(request):
    w = SHAPES[request.param]
    return w, build_table(w), OracleExperts(w)


def inputs(w, T, token0=0):
    return synth.activations(w, T, token0), synth.logits(w, T, token0), synth.router_bias(w)


def oracle_y(ox, w, x, lg, b, y0=None):
    xq, xd = oracle.q8_quant(x)
    idx, wt = oracle.route(lg, b, w.k)
    y, _ = oracle.moe_layer(ox.table_for(idx), w.E, w.S, xq, xd, idx, wt, out=y0,
                            accumulate=y0 is not None)
    return y, idx, wt


@pytest.mark.parametrize("T", TOKENS)
def test_forward_both_paths(shape, T):
    w, table, ox = shape
    x, lg, b = inputs(w, T, 10)
    ref, idx, wt = oracle_y(ox, w, x, lg, b)
    xq = torch.empty((T, w.D), dtype=torch.int8, device=dev)
    xd = torch.empty((T, w.D // 32), dtype=torch.float32, device=dev)
    coli.coli_quant_act_q8(to_dev(x), xq, xd)
    gi = torch.empty((T, w.k), dtype=torch.int32, device=dev)
    gw = torch.empty((T, w.k), dtype=torch.float32, device=dev)
    coli.coli_route_topk(to_dev(lg), to_dev(b), w.k, gi, gw)
    assert_bitexact("idx", gi.cpu().numpy(), idx)
    assert_bitexact("w", gw.cpu().numpy(), wt)
    ws = torch.empty(coli.coli_moe_workspace_bytes(table, T, w.k), dtype=torch.uint8, device=dev)
    for path in (coli.COLI_PATH_GEMV, coli.COLI_PATH_GROUPED):
        y = torch.full((T, w.D), float("nan"), dtype=torch.float32, device=dev)
        coli.coli_moe_forward_path(table, xq, xd, gi, gw, y, ws, path)
        assert coli.coli_moe_status(ws) == coli.COLI_OK
        assert_bitexact(f"y path {path}", y.cpu().numpy(), ref)


@pytest.mark.parametrize("T", TOKENS)
def test_layer_entry(shape, T):
    """The fused front (T <= 64) with Q8_0, routing and dispatch in one kernel."""
    w, table, ox = shape
    x, lg, b = inputs(w, T, 50)
    y0 = synth.normal(777, T * w.D, 1.0).reshape(T, w.D)
    ref, _, _ = oracle_y(ox, w, x, lg, b, y0=y0)
    ws = torch.empty(coli.coli_moe_layer_workspace_bytes(table, T, w.k), dtype=torch.uint8,
                     device=dev)
    y = to_dev(y0)
    coli.coli_moe_layer(table, to_dev(x), to_dev(lg), to_dev(b), w.k, y, ws, accumulate=True)
    assert coli.coli_moe_status(ws) == coli.COLI_OK
    assert_bitexact("y", y.cpu().numpy(), ref)


@pytest.mark.parametrize("T", [1, 5, 33])
def test_block_entry(shape, T):
    """h <- h + MoE(RMSNorm(h)) in place, against the oracle's RMSNorm, Q8_0 and layer."""
    w, table, ox = shape
    h0 = synth.normal(4242, T * w.D, 1.0).reshape(T, w.D)
    lg, b = synth.logits(w, T, 90), synth.router_bias(w)
    xh, _ = oracle.rmsnorm(h0, EPS)
    xq, xd = oracle.q8_quant(xh)
    idx, wt = oracle.route(lg, b, w.k)
    ref, _ = oracle.moe_layer(ox.table_for(idx), w.E, w.S, xq, xd, idx, wt, out=h0,
                              accumulate=True)
    ws = torch.empty(coli.coli_moe_layer_workspace_bytes(table, T, w.k), dtype=torch.uint8,
                     device=dev)
    h = to_dev(h0)
    coli.coli_moe_block(table, h, to_dev(lg), to_dev(b), w.k, ws, eps=EPS)
    assert coli.coli_moe_status(ws) == coli.COLI_OK
    assert_bitexact("h", h.cpu().numpy(), ref)
