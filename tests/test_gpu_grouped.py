"""Parity of the grouped (matrix-core) expert path against the oracle (GPU).

From COLI_GROUPED_MIN_TOKENS (5) tokens per pass the forward runs the grouped kernels: per active
expert, chunks of up to 128 tokens against 64-row weight groups.  These tests
check every int32 block partial, g, u, h, Q8(h) and per-pair output
bit-for-bit, over routings that exercise full, partial and single-token
chunks, plus the layer output.
"""
import numpy as np
import pytest

import oracle
import synth
from tests.gpu_util import OracleExperts, assert_bitexact, assert_within_tol, build_table
from tests.test_gpu_moe import GpuLayer, check_front, check_trace, oracle_layer, to_dev

pytestmark = pytest.mark.gpu
torch = pytest.importorskip("torch")
if not torch.cuda.is_available():
    pytest.skip("no GPU", allow_module_level=True)
import int4_routed_expert_sigmoid_amd as coli  # noqa: E402

dev = "cuda"


@pytest.fixture(scope="module")
def tiny():
    w = synth.WORKLOADS[0]
    return w, build_table(w), OracleExperts(w)


def trace_buffers(w, T):
    P, A = T * (w.k + w.S), w.E + w.S
    shapes = {"counts": ((A,), torch.int32), "lists": ((A, T), torch.int32),
              "n_active": ((1,), torch.int32), "active": ((A,), torch.int32),
              "p_gate": ((P, w.F, w.D // 32), torch.int32),
              "p_up": ((P, w.F, w.D // 32), torch.int32),
              "p_down": ((P, w.D, w.F // 32), torch.int32),
              "g": ((P, w.F), torch.float32), "u": ((P, w.F), torch.float32),
              "h": ((P, w.F), torch.float32), "hq": ((P, w.F), torch.int8),
              "hd": ((P, w.F // 32), torch.float32), "o": ((P, w.D), torch.float32)}
    return {k: torch.full(s, -7, dtype=d, device=dev) for k, (s, d) in shapes.items()}


@pytest.mark.parametrize("T", [128, 200, 333])
def test_grouped_tiny_traced(tiny, T):
    w, table, ox = tiny
    x, lg, b = synth.activations(w, T, 500), synth.logits(w, T, 500), synth.router_bias(w)
    g = GpuLayer(table, w, T).run(x, lg, b, trace=True)
    r = oracle_layer(ox, w, x, lg, b)
    check_front(g, r)
    check_trace(g, ox, w, r)
    assert_bitexact("y", g["y"], r["y"])
    assert_within_tol("y", g["y"], r["y"], r["absterm"])


def skewed_routing(T):
    """Hand-made top-2 routing over 16 experts: expert 0 takes tokens 0-129
    (chunks of 64, 64 and 2), expert 1 only token 7, expert 2 tokens 135-199
    (64 + 1), the rest spread thinly; the shared expert takes all T."""
    idx = np.empty((T, 2), np.int32)
    for t in range(T):
        s0 = 0 if t < 130 else 3 + t % 13
        s1 = 1 if t == 7 else (2 if t >= 135 else 4 + t % 12)
        idx[t] = (s0, s1)
    rng = np.random.default_rng(11)
    wt = rng.uniform(0.05, 1.0, size=(T, 2)).astype(np.float32)
    wt /= wt.sum(axis=1, keepdims=True)
    return idx, wt.astype(np.float32)


def test_grouped_skewed_counts_traced(tiny):
    w, table, ox = tiny
    T = 200
    idx, wt = skewed_routing(T)
    x = synth.activations(w, T, 600)
    xq, xd = oracle.q8_quant(x)
    xq_d = torch.empty((T, w.D), dtype=torch.int8, device=dev)
    xd_d = torch.empty((T, w.D // 32), dtype=torch.float32, device=dev)
    coli.coli_quant_act_q8(to_dev(x), xq_d, xd_d)
    assert_bitexact("xq", xq_d.cpu().numpy(), xq)
    ws = torch.empty(coli.coli_moe_workspace_bytes(table, T, w.k), dtype=torch.uint8, device=dev)
    y = torch.empty((T, w.D), dtype=torch.float32, device=dev)
    tr = trace_buffers(w, T)
    coli.coli_moe_forward_traced(table, xq_d, xd_d, to_dev(idx), to_dev(wt), y, ws, tr)
    assert coli.coli_moe_status(ws) == coli.COLI_OK
    g = {k: v.cpu().numpy() for k, v in tr.items()}
    counts = g["counts"]
    assert counts[0] == 130 and counts[1] == 1 and counts[2] == 65 and counts[w.E] == T
    r = dict(xq=xq, xd=xd, idx=idx, w=wt)
    check_trace(g, ox, w, r)
    yr, A = oracle.moe_layer(ox.table_for(idx), w.E, w.S, xq, xd, idx, wt)
    assert_bitexact("y", y.cpu().numpy(), yr)
    assert_within_tol("y", y.cpu().numpy(), yr, A)


def test_grouped_repeat_is_deterministic(tiny):
    w, table, _ = tiny
    T = 256
    x, lg, b = synth.activations(w, T, 700), synth.logits(w, T, 700), synth.router_bias(w)
    lay = GpuLayer(table, w, T)
    y1 = lay.run(x, lg, b)["y"]
    y2 = lay.run(x, lg, b)["y"]
    assert_bitexact("y repeat", y1, y2)


@pytest.fixture(scope="module")
def big():
    w = synth.WORKLOADS[1]
    return build_table(w), OracleExperts(w)


@pytest.mark.parametrize("T", [128, 300])
def test_grouped_full_shape_sampled(big, T):
    """6144 x 2048 experts, 256 + 1 of them: sampled tokens against the oracle."""
    table, ox = big
    w = synth.WORKLOADS[3]
    x, lg, b = synth.activations(w, T, 800), synth.logits(w, T, 800), synth.router_bias(w)
    g = GpuLayer(table, w, T).run(x, lg, b)
    xq, xd = oracle.q8_quant(x)
    idx, wt = oracle.route(lg, b, w.k)
    assert_bitexact("idx", g["idx"], idx)
    sample = [0, T // 3, T - 1]
    ys, A = oracle.moe_layer(ox.table_for(idx[sample]), w.E, w.S, xq[sample], xd[sample],
                             idx[sample], wt[sample])
    assert_bitexact("y sample", g["y"][sample], ys)
    assert_within_tol("y sample", g["y"][sample], ys, A)


def forward_on(table, w, path, xq, xd, idx, wt):
    T = idx.shape[0]
    ws = torch.empty(coli.coli_moe_workspace_bytes(table, T, w.k), dtype=torch.uint8, device=dev)
    y = torch.empty((T, w.D), dtype=torch.float32, device=dev)
    coli.coli_moe_forward_path(table, xq, xd, idx, wt, y, ws, path)
    assert coli.coli_moe_status(ws) == coli.COLI_OK
    return y.cpu().numpy()


def routed_batch(w, T, token0):
    x, lg, b = synth.activations(w, T, token0), synth.logits(w, T, token0), synth.router_bias(w)
    xq = torch.empty((T, w.D), dtype=torch.int8, device=dev)
    xd = torch.empty((T, w.D // 32), dtype=torch.float32, device=dev)
    coli.coli_quant_act_q8(to_dev(x), xq, xd)
    idx = torch.empty((T, w.k), dtype=torch.int32, device=dev)
    wt = torch.empty((T, w.k), dtype=torch.float32, device=dev)
    coli.coli_route_topk(to_dev(lg), to_dev(b), w.k, idx, wt)
    return xq, xd, idx, wt


@pytest.mark.parametrize("T", [1, 4, 37, 64, 128, 300])
def test_forced_paths_bit_identical(tiny, T):
    """Both paths at every batch size, including the grouped path below its
    automatic threshold and the GEMV above it: identical outputs, equal to
    the oracle."""
    w, table, ox = tiny
    xq, xd, idx, wt = routed_batch(w, T, 1200)
    y1 = forward_on(table, w, coli.COLI_PATH_GEMV, xq, xd, idx, wt)
    y2 = forward_on(table, w, coli.COLI_PATH_GROUPED, xq, xd, idx, wt)
    assert_bitexact("GEMV vs grouped", y1, y2)
    xq_h, xd_h, idx_h, wt_h = (a.cpu().numpy() for a in (xq, xd, idx, wt))
    yr, _ = oracle.moe_layer(ox.table_for(idx_h), w.E, w.S, xq_h, xd_h, idx_h, wt_h)
    assert_bitexact("y vs oracle", y1, yr)


@pytest.mark.parametrize("T", [16, 96])
def test_forced_paths_full_shape(big, T):
    table, _ = big
    w = synth.WORKLOADS[3]
    xq, xd, idx, wt = routed_batch(w, T, 1300)
    y1 = forward_on(table, w, coli.COLI_PATH_GEMV, xq, xd, idx, wt)
    y2 = forward_on(table, w, coli.COLI_PATH_GROUPED, xq, xd, idx, wt)
    assert_bitexact("GEMV vs grouped, page shape", y1, y2)
