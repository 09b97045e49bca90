"""MoE layer parity of the HIP path against the oracle (GPU).

Each side draws the same seeded fp32 inputs and quantises them with its own
code; the comparison is bit-exact for every integer, quantised value and
fp32 intermediate of the decode path, and the layer output is also checked
against the |gpu - oracle| <= 1e-5 * sum|terms| + 1e-6 bound.
"""
import numpy as np
import pytest

import oracle
import synth
from tests.gpu_util import (OracleExperts, assert_bitexact, assert_within_tol, build_table)

pytestmark = pytest.mark.gpu
torch = pytest.importorskip("torch")
if not torch.cuda.is_available():
    pytest.skip("no GPU", allow_module_level=True)
import int4_routed_expert_sigmoid_amd as coli  # noqa: E402

dev = "cuda"


def to_dev(a):
    return torch.from_numpy(np.ascontiguousarray(a)).to(dev)


class GpuLayer:
    """quant -> route -> forward through the C ABI for one batch of tokens."""

    def __init__(self, table, w, T):
        self.table, self.w, self.T = table, w, T
        self.ws = torch.empty(coli.coli_moe_workspace_bytes(table, T, w.k), dtype=torch.uint8,
                              device=dev)

    def run(self, x, logits, bias, trace=False, y0=None, accumulate=False):
        w, T = self.w, self.T
        xq = torch.empty((T, w.D), dtype=torch.int8, device=dev)
        xd = torch.empty((T, w.D // 32), dtype=torch.float32, device=dev)
        coli.coli_quant_act_q8(to_dev(x), xq, xd)
        idx = torch.empty((T, w.k), dtype=torch.int32, device=dev)
        wt = torch.empty((T, w.k), dtype=torch.float32, device=dev)
        coli.coli_route_topk(to_dev(logits), to_dev(bias), w.k, idx, wt)
        y = to_dev(y0) if y0 is not None else torch.empty((T, w.D), dtype=torch.float32,
                                                          device=dev)
        out = {}
        if trace:
            P = T * (w.k + w.S)
            A = w.E + w.S
            tr = {
                "counts": torch.empty(A, dtype=torch.int32, device=dev),
                "lists": torch.empty((A, T), dtype=torch.int32, device=dev),
                "n_active": torch.empty(1, dtype=torch.int32, device=dev),
                "active": torch.empty(A, dtype=torch.int32, device=dev),
                "p_gate": torch.empty((P, w.F, w.D // 32), dtype=torch.int32, device=dev),
                "p_up": torch.empty((P, w.F, w.D // 32), dtype=torch.int32, device=dev),
                "p_down": torch.empty((P, w.D, w.F // 32), dtype=torch.int32, device=dev),
                "g": torch.empty((P, w.F), dtype=torch.float32, device=dev),
                "u": torch.empty((P, w.F), dtype=torch.float32, device=dev),
                "h": torch.empty((P, w.F), dtype=torch.float32, device=dev),
                "hq": torch.empty((P, w.F), dtype=torch.int8, device=dev),
                "hd": torch.empty((P, w.F // 32), dtype=torch.float32, device=dev),
                "o": torch.empty((P, w.D), dtype=torch.float32, device=dev),
            }
            coli.coli_moe_forward_traced(self.table, xq, xd, idx, wt, y, self.ws, tr,
                                         accumulate=accumulate)
            out = {k: v.cpu().numpy() for k, v in tr.items()}
        else:
            coli.coli_moe_forward(self.table, xq, xd, idx, wt, y, self.ws, accumulate=accumulate)
        assert coli.coli_moe_status(self.ws) == coli.COLI_OK
        out.update(xq=xq.cpu().numpy(), xd=xd.cpu().numpy(), idx=idx.cpu().numpy(),
                   w=wt.cpu().numpy(), y=y.cpu().numpy())
        return out


def oracle_layer(ox: OracleExperts, w, x, logits, bias, y0=None, accumulate=False):
    xq, xd = oracle.q8_quant(x)
    idx, wt = oracle.route(logits, bias, w.k)
    y, A = oracle.moe_layer(ox.table_for(idx), w.E, w.S, xq, xd, idx, wt, out=y0,
                            accumulate=accumulate)
    return dict(xq=xq, xd=xd, idx=idx, w=wt, y=y, absterm=A)


def check_front(g, r):
    assert_bitexact("xq", g["xq"], r["xq"])
    assert_bitexact("xd", g["xd"], r["xd"])
    assert_bitexact("idx", g["idx"], r["idx"])
    assert_bitexact("w", g["w"], r["w"])


def check_trace(g, ox, w, r, tokens=None):
    """Every pair's partials and intermediates against the oracle's expert."""
    T = r["idx"].shape[0]
    counts, lists, na, act = oracle.dispatch(r["idx"], w.E, w.S)
    assert_bitexact("counts", g["counts"], counts)
    assert int(g["n_active"][0]) == na
    assert_bitexact("active", g["active"][:na], act)
    for e in act:
        assert_bitexact(f"list {e}", g["lists"][e, :counts[e]], lists[e, :counts[e]])
    for t in (range(T) if tokens is None else tokens):
        for slot in range(w.k + w.S):
            e = w.E if slot == w.k else int(r["idx"][t, slot])
            p = t * (w.k + w.S) + slot
            ref = oracle.expert_forward(ox[e], r["xq"][t], r["xd"][t], want_partials=True)
            tag = f"t{t} slot{slot} e{e}"
            assert_bitexact(f"P_gate {tag}", g["p_gate"][p], ref["P_gate"])
            assert_bitexact(f"P_up {tag}", g["p_up"][p], ref["P_up"])
            assert_bitexact(f"g {tag}", g["g"][p], ref["g"])
            assert_bitexact(f"u {tag}", g["u"][p], ref["u"])
            assert_bitexact(f"h {tag}", g["h"][p], ref["h"])
            assert_bitexact(f"hq {tag}", g["hq"][p], ref["hq"])
            assert_bitexact(f"hd {tag}", g["hd"][p], ref["hd"])
            assert_bitexact(f"P_down {tag}", g["p_down"][p], ref["P_down"])
            assert_bitexact(f"o {tag}", g["o"][p], ref["o"])


# ---------------------------------------------------------------- tiny layer
@pytest.fixture(scope="module")
def tiny():
    w = synth.WORKLOADS[0]
    return w, build_table(w), OracleExperts(w)


def test_tiny_layer_traced(tiny):
    w, table, ox = tiny
    x, lg, b = synth.activations(w, w.T), synth.logits(w, w.T), synth.router_bias(w)
    g = GpuLayer(table, w, w.T).run(x, lg, b, trace=True)
    r = oracle_layer(ox, w, x, lg, b)
    check_front(g, r)
    check_trace(g, ox, w, r)
    assert_bitexact("y", g["y"], r["y"])
    assert_within_tol("y", g["y"], r["y"], r["absterm"])


@pytest.mark.parametrize("T", [1, 2, 3, 5, 8, 9, 17, 64])
def test_tiny_layer_token_counts(tiny, T):
    """Ragged batches: GEMV pass sizes (1-4 tokens), the grouped path from 5, partial chunks."""
    w, table, ox = tiny
    x, lg, b = synth.activations(w, T, 100), synth.logits(w, T, 100), synth.router_bias(w)
    g = GpuLayer(table, w, T).run(x, lg, b)
    r = oracle_layer(ox, w, x, lg, b)
    check_front(g, r)
    assert_bitexact("y", g["y"], r["y"])


def test_tiny_layer_accumulate_and_determinism(tiny):
    w, table, ox = tiny
    x, lg, b = synth.activations(w, w.T, 7), synth.logits(w, w.T, 7), synth.router_bias(w)
    y0 = synth.normal(12345, w.T * w.D, 1.0).reshape(w.T, w.D)
    L = GpuLayer(table, w, w.T)
    g1 = L.run(x, lg, b, y0=y0, accumulate=True)
    g2 = L.run(x, lg, b, y0=y0, accumulate=True)
    r = oracle_layer(ox, w, x, lg, b, y0=y0, accumulate=True)
    assert_bitexact("y (run 1)", g1["y"], r["y"])
    assert_bitexact("y (run 2)", g2["y"], g1["y"])


def _dropped_case(w, table, ox, idx, path, seed):
    """Forward of a routing with dropped entries (out of range, or a repeat of
    an earlier slot of the token) against the oracle serving the kept entries."""
    T = idx.shape[0]
    x = synth.activations(w, T, seed)
    xq_h, xd_h = oracle.q8_quant(x)
    wt_h = np.random.default_rng(seed).uniform(0.05, 0.5, size=idx.shape).astype(np.float32)
    xq, xd = to_dev(xq_h), to_dev(xd_h)
    y = torch.full((T, w.D), float("nan"), dtype=torch.float32, device=dev)
    ws = torch.empty(coli.coli_moe_workspace_bytes(table, T, w.k), dtype=torch.uint8, device=dev)
    ws.fill_(0x7F)                      # stale contents must not reach y
    coli.coli_moe_forward_path(table, xq, xd, to_dev(idx), to_dev(wt_h), y, ws, path)
    keep, dropped = oracle.keep_entries(idx, w.E)
    assert coli.coli_moe_status(ws) == (coli.COLI_E_INDEX if dropped else coli.COLI_OK)
    ry, _ = oracle.moe_layer(ox.table_for(idx), w.E, w.S, xq_h, xd_h, idx, wt_h, keep=keep)
    assert_bitexact(f"y (T={T}, path {path})", y.cpu().numpy(), ry)
    return ws


@pytest.mark.parametrize("bad", [[[5, 5]], [[0, 16]], [[-1, 3]], [[16, 16]]])
def test_dropped_entries_one_token(tiny, bad):
    """One token: a repeated or out-of-range slot contributes nothing (the y of
    the kept slots, bit-exact), the flag is raised, and the next valid call on
    the same workspace clears it."""
    w, table, ox = tiny
    ws = _dropped_case(w, table, ox, np.int32(bad), coli.COLI_PATH_AUTO, 31)
    xq = torch.zeros((1, w.D), dtype=torch.int8, device=dev)
    xd = torch.ones((1, w.D // 32), dtype=torch.float32, device=dev)
    wt = torch.full((1, w.k), 0.5, dtype=torch.float32, device=dev)
    y = torch.empty((1, w.D), dtype=torch.float32, device=dev)
    coli.coli_moe_forward(table, xq, xd, to_dev(np.int32([[0, 1]])), wt, y, ws)
    assert coli.coli_moe_status(ws) == coli.COLI_OK


@pytest.mark.parametrize("path", ["gemv", "grouped"])
@pytest.mark.parametrize("T", [2, 9, 100, 333])
def test_dropped_entries_many_tokens(tiny, path, T):
    """Batches with repeats and out-of-range slots through both expert paths:
    T = 2 with a repeat that precedes a valid slot of the next token, and
    ragged batches past the shared-list workgroup's 256-token sweep."""
    w, table, ox = tiny
    rng = np.random.default_rng(T)
    idx = np.stack([rng.choice(w.E, w.k, replace=False) for _ in range(T)]).astype(np.int32)
    if T == 2:
        idx = np.int32([[5, 5], [5, 4]])
    else:
        idx[::3, 1] = idx[::3, 0]                        # repeats
        idx[1::7, 0] = w.E + 3                           # out of range
        idx[2::11, 1] = -1
    p = coli.COLI_PATH_GEMV if path == "gemv" else coli.COLI_PATH_GROUPED
    _dropped_case(w, table, ox, idx, p, 40 + T)


# ---------------------------------------------------------------- page-scale layer
@pytest.fixture(scope="module")
def big():
    w = synth.WORKLOADS[1]
    return build_table(w), OracleExperts(w)


def test_decode_layer_traced(big):
    """1 token, d_model 6144, d_ff 2048, 256+1 experts, top-8 (4.86 GB table in HBM)."""
    table, ox = big
    w = synth.WORKLOADS[1]
    L = GpuLayer(table, w, 1)
    for tok in (0, 1):
        x, lg, b = synth.activations(w, 1, tok), synth.logits(w, 1, tok), synth.router_bias(w)
        g = L.run(x, lg, b, trace=True)
        r = oracle_layer(ox, w, x, lg, b)
        check_front(g, r)
        check_trace(g, ox, w, r)
        assert_bitexact("y", g["y"], r["y"])
        assert_within_tol("y", g["y"], r["y"], r["absterm"])


def test_verify_layer_traced(big):
    """4 tokens through one pass: the batch union of their experts."""
    table, ox = big
    w = synth.WORKLOADS[2]
    x, lg, b = synth.activations(w, 4), synth.logits(w, 4), synth.router_bias(w)
    g = GpuLayer(table, w, 4).run(x, lg, b, trace=True)
    r = oracle_layer(ox, w, x, lg, b)
    check_front(g, r)
    check_trace(g, ox, w, r)
    assert_bitexact("y", g["y"], r["y"])
    assert_within_tol("y", g["y"], r["y"], r["absterm"])


def _prefill_full(table, ox, bias_free):
    """Every token of the 2048-token pass, as the benchmark runs it (one
    coli_moe_layer call: fused Q8 + routing front, dispatch, grouped matrix-core
    kernels, combine), against the oracle on all 2048 tokens."""
    w = synth.WORKLOADS[3]
    T = w.T
    x, lg, b = synth.activations(w, T), synth.logits(w, T), synth.router_bias(w)
    if bias_free:
        b = np.zeros_like(b)
    assert coli.coli_moe_path(table, T, w.k) == coli.COLI_PATH_GROUPED
    g = run_layer(table, w, x, lg, b)
    xq, xd = oracle.q8_quant(x)
    idx, wt = oracle.route(lg, b, w.k)
    print(f"prefill full ({'bias 0' if bias_free else 'bias N(0,0.1)'}): GPU done, oracle on "
          f"{T} tokens", flush=True)
    ry, A = oracle.moe_layer(ox.table_for(idx), w.E, w.S, xq, xd, idx, wt)
    counts = np.bincount(idx.reshape(-1), minlength=w.E)
    # the busiest experts span many 128-token work items and end in a partial one
    assert counts.max() > 3 * 128 and counts.max() % 128 != 0
    assert_bitexact("y, all 2048 tokens", g["y"], ry)
    assert_within_tol("y, all 2048 tokens", g["y"], ry, A)


def test_prefill_layer_full(big):
    """2048 tokens, router bias N(0, 0.1): 185 experts, up to 610 tokens each."""
    table, ox = big
    _prefill_full(table, ox, bias_free=False)
    ox.cache.clear()


# ---------------------------------------------------------------- coli_moe_layer (fused front)
def run_layer(table, w, x, logits, bias, trace=False, y0=None, accumulate=False):
    T = x.shape[0]
    ws = torch.empty(coli.coli_moe_layer_workspace_bytes(table, T, w.k), dtype=torch.uint8,
                     device=dev)
    y = to_dev(y0) if y0 is not None else torch.empty((T, w.D), dtype=torch.float32, device=dev)
    tr = None
    if trace:
        P, A = T * (w.k + w.S), w.E + w.S
        shapes = {"counts": ((A,), torch.int32), "lists": ((A, T), torch.int32),
                  "n_active": ((1,), torch.int32), "active": ((A,), torch.int32),
                  "p_gate": ((P, w.F, w.D // 32), torch.int32),
                  "p_up": ((P, w.F, w.D // 32), torch.int32),
                  "p_down": ((P, w.D, w.F // 32), torch.int32),
                  "g": ((P, w.F), torch.float32), "u": ((P, w.F), torch.float32),
                  "h": ((P, w.F), torch.float32), "hq": ((P, w.F), torch.int8),
                  "hd": ((P, w.F // 32), torch.float32), "o": ((P, w.D), torch.float32),
                  "xq": ((T, w.D), torch.int8), "xd": ((T, w.D // 32), torch.float32),
                  "idx": ((T, w.k), torch.int32), "w": ((T, w.k), torch.float32)}
        tr = {k: torch.empty(s, dtype=d, device=dev) for k, (s, d) in shapes.items()}
    coli.coli_moe_layer(table, to_dev(x), to_dev(logits), to_dev(bias), w.k, y, ws,
                        accumulate=accumulate, trace=tr)
    assert coli.coli_moe_status(ws) == coli.COLI_OK
    out = {"y": y.cpu().numpy()}
    if tr:
        out.update({k: v.cpu().numpy() for k, v in tr.items()})
    return out


def test_layer_entry_tiny_traced(tiny):
    """Fused front (Q8 + route + dispatch in one workgroup): every intermediate."""
    w, table, ox = tiny
    x, lg, b = synth.activations(w, w.T, 300), synth.logits(w, w.T, 300), synth.router_bias(w)
    g = run_layer(table, w, x, lg, b, trace=True)
    r = oracle_layer(ox, w, x, lg, b)
    check_front(g, r)
    check_trace(g, ox, w, r)
    assert_bitexact("y", g["y"], r["y"])


@pytest.mark.parametrize("T", [1, 64, 65, 200, 512])
def test_layer_entry_batch_sizes(tiny, T):
    """Both sides of the fused-front threshold (T <= 64 and T*k <= 1024)."""
    w, table, ox = tiny
    x, lg, b = synth.activations(w, T, 400), synth.logits(w, T, 400), synth.router_bias(w)
    y0 = synth.normal(999, T * w.D, 1.0).reshape(T, w.D)
    g = run_layer(table, w, x, lg, b, y0=y0, accumulate=True)
    r = oracle_layer(ox, w, x, lg, b, y0=y0, accumulate=True)
    assert_bitexact("y", g["y"], r["y"])


def test_layer_entry_decode_traced(big):
    table, ox = big
    w = synth.WORKLOADS[1]
    x, lg, b = synth.activations(w, 1, 5), synth.logits(w, 1, 5), synth.router_bias(w)
    g = run_layer(table, w, x, lg, b, trace=True)
    r = oracle_layer(ox, w, x, lg, b)
    check_front(g, r)
    check_trace(g, ox, w, r)
    assert_bitexact("y", g["y"], r["y"])
    assert_within_tol("y", g["y"], r["y"], r["absterm"])


def test_layer_entry_verify(big):
    table, ox = big
    w = synth.WORKLOADS[2]
    x, lg, b = synth.activations(w, 4, 8), synth.logits(w, 4, 8), synth.router_bias(w)
    g = run_layer(table, w, x, lg, b)
    r = oracle_layer(ox, w, x, lg, b)
    assert_bitexact("y", g["y"], r["y"])
