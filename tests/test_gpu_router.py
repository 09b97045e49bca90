"""Router projection on the GPU against the oracle (GPU).

logits[t][e] = sum_d wr[e][d] x[t][d] with F32 router weights, each product
exact in fp64, summed in fp64 and rounded once.  The GPU's fp64 summation
order differs from the oracle's ascending one, which can move an fp32 result
only when the fp64 sum lies within ~2^-29 relative of a rounding boundary:
the test requires every logit within the fp32 tolerance and all but a
vanishing fraction bit-identical, and the routing decided from the GPU's
logits identical to the oracle's routing of the same logits.
"""
import numpy as np
import pytest

import oracle
import synth
from tests.gpu_util import assert_bitexact, assert_within_tol

pytestmark = pytest.mark.gpu
torch = pytest.importorskip("torch")
if not torch.cuda.is_available():
    pytest.skip("no GPU", allow_module_level=True)
import int4_routed_expert_sigmoid_amd as coli  # noqa: E402

dev = "cuda"


def to_dev(a):
    return torch.from_numpy(np.ascontiguousarray(a)).to(dev)


def gpu_logits(x, wr):
    T, E = x.shape[0], wr.shape[0]
    out = torch.empty((T, E), dtype=torch.float32, device=dev)
    coli.coli_router_logits(to_dev(x), to_dev(wr), out)
    return out


@pytest.mark.parametrize("wl,T", [(0, 1), (0, 15), (0, 16), (0, 77), (1, 1), (1, 4), (1, 100),
                                  (1, 2048)])
def test_router_logits(wl, T):
    w = synth.WORKLOADS[wl]
    x = synth.activations(w, T, 900)
    wr = synth.router_weights(w)
    got_d = gpu_logits(x, wr)
    got = got_d.cpu().numpy()
    ref = oracle.router_logits(x, wr)
    absterm = np.abs(x.astype(np.float64)) @ np.abs(wr.astype(np.float64)).T
    assert_within_tol("router logits", got, ref, absterm)
    exact = np.mean(got == ref)
    assert exact >= 0.9999, f"only {exact:.6f} of the logits are bit-identical"
    # routing from the GPU's logits: the GPU router and the oracle agree exactly
    bias = synth.router_bias(w)
    idx = torch.empty((T, w.k), dtype=torch.int32, device=dev)
    wt = torch.empty((T, w.k), dtype=torch.float32, device=dev)
    coli.coli_route_topk(got_d, to_dev(bias), w.k, idx, wt)
    ridx, rw = oracle.route(got, bias, w.k)
    assert_bitexact("idx", idx.cpu().numpy(), ridx)
    assert_bitexact("w", wt.cpu().numpy(), rw)


@pytest.mark.parametrize("D,E,T", [(64, 5, 3), (64, 5, 40), (8256, 70, 2), (8256, 70, 33),
                                   (192, 129, 17)])
def test_router_logits_odd_shapes(D, E, T):
    """Shapes at the kernels' edges: a quarter row of one float4 per lane
    group (D = 64), rows too long for the few-token kernel (D = 8256 > 8192:
    the matrix-core kernel at 2 tokens too), expert and token counts that
    leave partial 64-expert / 32-token tiles."""
    from dataclasses import replace
    w = replace(synth.WORKLOADS[0], D=D, E=E, k=min(synth.WORKLOADS[0].k, E), tag=11)
    x = synth.activations(w, T, 950)
    wr = synth.router_weights(w)
    got = gpu_logits(x, wr).cpu().numpy()
    ref = oracle.router_logits(x, wr)
    absterm = np.abs(x.astype(np.float64)) @ np.abs(wr.astype(np.float64)).T
    assert_within_tol("router logits", got, ref, absterm)
    assert np.mean(got == ref) >= 0.999


def test_router_logits_closed_form():
    x = np.full((3, 6144), 0.25, np.float32)
    wr = np.full((256, 6144), 0.5, np.float32)
    assert np.all(gpu_logits(x, wr).cpu().numpy() == 768.0)
